// Exact attention backward for gfx950: dQ, dK, dV by recomputing the
// probabilities from Q, K and the forward's log-sum-exp.
//
// The pages obtain the backward pass by recomputation instead of storing the
// N x N probabilities ("Flash Attention | Hermes Skill", Quick start: IO-aware
// tiling and recomputation; FP8 section: the 16-bit kernels run forward and
// backward).  With P_ij = exp(s_ij - LSE_i), the chain rule through the
// standard-attention definition gives
//     dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i,  dS = P o (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q.
// Two kernels, no atomics (results do not depend on the order workgroups run
// in):
//   * attn_bwd_dq_kernel: one workgroup per (batch, head, 128 query rows),
//     the mirror of the forward: Q^T and dO^T stay in registers (lane = query
//     row), K and V tiles of 64 keys stream through LDS.  Per 32-key half:
//     S^T = K Q^T and dP^T = V dO^T on the MFMA, dS^T = P^T o (dP^T - D) in
//     the accumulator layout, which is the B-operand layout of
//     dQ^T += K^T dS^T (K^T from the transposing LDS read).  It also computes
//     D = rowsum(dO o O) and writes it for the second kernel.
//   * attn_bwd_dkdv_kernel: one workgroup per (batch, K/V head, 128 keys), K^T
//     and V^T in registers (lane = key), Q and dO tiles of 64 rows streaming
//     through LDS, for every query head that reads this K/V head.  Per 32-row
//     half: S = Q K^T, dP = dO V^T; P and dS in the accumulator layout (lane
//     = key) are the B operands of dV^T += dO^T P and dK^T += Q^T dS, with
//     dO^T and Q^T from the transposing LDS read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bwd_kernel.h"
#include "kernel_common.h"

namespace ea {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <In IN, int D>
struct BwdCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRow = D * 2;                 // bytes per 16-bit row in LDS
  static constexpr int kTile = 64 * kRow;            // a 64-row tile of K, V, Q or dO
  static constexpr int kSteps = D / 16;              // MFMA k-steps over d
  static constexpr int kDBlocks = D / 32;
  static constexpr int kDma = kTile / 1024 / kWaves; // 1 KB DMA instructions per wave per tile
};

// Tile row and byte column of the 16-byte unit lane `ln` fetches in DMA block
// `blk` of a 64-row tile (the swizzle of kernel_common.h applied in reverse).
template <int ROW_BYTES>
__device__ __forceinline__ uint32_t dma_offset(int blk, int ln, int row_stride) {
  const int pos = blk * 64 + ln;
  const int row = pos / (ROW_BYTES / 16);
  const int phys = pos % (ROW_BYTES / 16);
  return (uint32_t)(row * row_stride + swizzled_unit<ROW_BYTES>(row, phys) * 16);
}

// Byte range [base, base + bytes) of rows [r0, r0 + 64) of a head, cut at row
// n (the buffer range makes rows past it read as zeros).
struct Rows64 {
  const unsigned char* base;
  int bytes;
};
__device__ __forceinline__ Rows64 rows64(const unsigned char* head, int row_stride, int row_bytes, int r0, int n) {
  const int rows = min(n - r0, 64);
  return Rows64{head + (int64_t)r0 * row_stride, rows > 0 ? (rows - 1) * row_stride + row_bytes : 0};
}

// 32 lanes x 8 values of a 16-bit row fragment: lane holds d = 16 st + 8 half
// + [0, 8) of row `row_ptr` for every k-step (zeros if !ok).
template <int D>
__device__ __forceinline__ void load_row_frags(uint4 (&f)[D / 16], const unsigned char* row_ptr, bool ok, int half) {
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    f[st] = ok ? *(const uint4*)(row_ptr + (16 * st + 8 * half) * 2) : make_uint4(0, 0, 0, 0);
}

template <In IN>
__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
  const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = __builtin_fmaf(unpack_lo<IN>(wa[i]), unpack_lo<IN>(wb[i]), s);
    s = __builtin_fmaf(unpack_hi<IN>(wa[i]), unpack_hi<IN>(wb[i]), s);
  }
  return s;
}

// This lane's transposing-read offsets within a tile (see pv_half).
template <int D>
__device__ __forceinline__ void tr_offsets(uint32_t (&va)[2][D / 32], int lane) {
  const int g = lane >> 4, sl = lane & 15;
#pragma unroll
  for (int r8 = 0; r8 < 2; ++r8)
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const int vrow = 4 * (g >> 1) + (sl >> 2) + 8 * r8;
      const int dcol = 32 * c + 16 * (g & 1) + 4 * (sl & 3);
      va[r8][c] = (uint32_t)(lds_offset<D * 2>(vrow, dcol >> 3) + (dcol & 7) * 2);
      asm volatile("" : "+v"(va[r8][c]));
    }
}

// Row-read offsets of a tile: row `col` of a 32-row block, k-step st.
template <int D>
__device__ __forceinline__ void row_offsets(uint32_t (&ka)[D / 16], int col, int half) {
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    ka[st] = (uint32_t)lds_offset<D * 2>(col, 2 * st + half);
    asm volatile("" : "+v"(ka[st]));
  }
}

// Write a 32-row x D accumulator held with lane = row (registers = columns
// 32 c + 8 j + 4 half + [0, 4)) as 16-bit values times `mul`.
template <In IN, int D>
__device__ __forceinline__ void store_rows(unsigned char* row_ptr, const f32x16 (&acc)[D / 32], float mul, int half) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * c + 8 * j + 4 * half;
      uint2 w;
      w.x = pack2<IN>(acc[c][4 * j] * mul, acc[c][4 * j + 1] * mul);
      w.y = pack2<IN>(acc[c][4 * j + 2] * mul, acc[c][4 * j + 3] * mul);
      *(uint2*)(row_ptr + d * 2) = w;
    }
}

}  // namespace

// The backward's work order: groups of up to four heads per XCD (the
// largest of 4, 2, 1 that splits the heads evenly), else unit-major over
// all heads.
__device__ __forceinline__ int2 bwd_order(int w, int units, int heads) {
  if (heads % 8 != 0) return make_int2(w / heads, w % heads);
  return xcd_grouped(w, units, heads % 32 == 0 ? 4 : heads % 16 == 0 ? 2 : 1);
}

// ---------------------------------------------------------------------------
// dQ (and D)
// ---------------------------------------------------------------------------
template <In IN, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_kernel(const BwdParams p) {
  using C = BwdCfg<IN, D>;
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf0[C::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf1[C::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf0[C::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf1[C::kTile];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int n = p.n;

  // heaviest query tiles first, a few heads at a time per XCD (workgroup w
  // runs on XCD w % 8): with shared K/V heads, the query heads of two K/V
  // heads (one if the K/V heads only split into eights), the unit being
  // (query tile, query head of the group); else groups of heads
  const int bh_count = p.batch * p.heads;
  const int bhk_count = bh_count / p.group;
  int tile = p.q_tiles - 1 - (int)(blockIdx.x / bh_count);
  int bh = (int)(blockIdx.x % bh_count);
  if (p.group > 1 && bhk_count % 8 == 0) {
    const int2 wo = xcd_grouped((int)blockIdx.x, p.q_tiles * p.group, bhk_count % 16 == 0 ? 2 : 1);
    tile = p.q_tiles - 1 - wo.x / p.group;
    bh = wo.y * p.group + wo.x % p.group;
  } else if (p.group == 1) {
    const int2 wo = bwd_order((int)blockIdx.x, p.q_tiles, bh_count);
    tile = p.q_tiles - 1 - wo.x;
    bh = wo.y;
  }
  const int b = bh / p.heads;
  const int h = bh - b * p.heads;
  const int hkv = h / p.group;
  const int q0 = tile * 128;
  const int qrow = q0 + wave * 32 + col;
  const bool ok = qrow < n;

  // Q^T, dO^T in registers; D = dO . O (each lane holds half of the row's d)
  uint4 qf[C::kSteps], df[C::kSteps];
  float delta;
  {
    const int qr = ok ? qrow : 0;
    load_row_frags<D>(qf, (const unsigned char*)p.q + ((int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)qr * p.q_ss) * 2, ok, half);
    load_row_frags<D>(df, (const unsigned char*)p.dout + ((int64_t)b * p.do_sb + (int64_t)h * p.do_sh + (int64_t)qr * p.do_ss) * 2, ok, half);
    uint4 of[C::kSteps];
    load_row_frags<D>(of, (const unsigned char*)p.o + ((int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)qr * p.o_ss) * 2, ok, half);
    float part = 0.f;
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) part += dot8<IN>(df[st], of[st]);
    delta = pair_sum(part);
  }
  // P = exp2(s c - lse log2 e); rows past n (and rows that saw no key) give 0
  float lse2 = INFINITY;
  if (ok) {
    const float l = p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + qrow];
    if (__builtin_isfinite(l)) lse2 = l * kLog2e;
  }
  const float cexp = p.c_log2;

  const KeyRange kr = tile_key_range(q0, 128, n, p.causal, p.wl, p.wr);
  const int kt_begin = kr.lo / kBN;
  const int kt_end = (kr.hi + kBN - 1) / kBN;
  const int wr0 = q0 + wave * 32;
  const int wr1 = min(wr0 + 32, n);
  int vis_lo;
  uint32_t vis_span;
  {
    vis_lo = p.wl >= 0 ? qrow - p.wl : 0;
    int hi = n - 1;
    if (p.causal) hi = min(hi, qrow);
    if (p.wr >= 0) hi = min(hi, qrow + p.wr);
    vis_span = (uint32_t)(hi - vis_lo);
  }

  const unsigned char* kg = (const unsigned char*)p.k + ((int64_t)b * p.k_sb + (int64_t)hkv * p.k_sh) * 2;
  const unsigned char* vg = (const unsigned char*)p.v + ((int64_t)b * p.v_sb + (int64_t)hkv * p.v_sh) * 2;
  const int k_stride = (int)(p.k_ss * 2), v_stride = (int)(p.v_ss * 2);
  uint32_t k_off[C::kDma], v_off[C::kDma];
#pragma unroll
  for (int i = 0; i < C::kDma; ++i) {
    k_off[i] = dma_offset<C::kRow>(wave * C::kDma + i, lane, k_stride);
    v_off[i] = dma_offset<C::kRow>(wave * C::kDma + i, lane, v_stride);
  }
  auto issue = [&](int kt, unsigned char* kdst, unsigned char* vdst) {
    const Rows64 rk = rows64(kg, k_stride, C::kRow, kt * kBN, n);
    const Rows64 rv = rows64(vg, v_stride, C::kRow, kt * kBN, n);
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) {
      load_16b_to_lds(rk.base, rk.bytes, k_off[i], kdst + (wave * C::kDma + i) * 1024);
      load_16b_to_lds(rv.base, rv.bytes, v_off[i], vdst + (wave * C::kDma + i) * 1024);
    }
  };
  uint32_t ka[C::kSteps];
  row_offsets<D>(ka, col, half);
  uint32_t va[2][C::kDBlocks];
  tr_offsets<D>(va, lane);

  f32x16 acc[1][C::kDBlocks];
#pragma unroll
  for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][c][r] = 0.f;

  // Tiles crossing a mask edge or the sequence end, for this wave's rows:
  // every visibility condition is monotone in the key tile index, so the
  // tiles seen in full form one interval [t_lo, t_lo + t_span).
  int t_hi_key = n - kBN;
  if (p.causal) t_hi_key = min(t_hi_key, wr0 - (kBN - 1));
  if (p.wr >= 0) t_hi_key = min(t_hi_key, wr0 + p.wr - (kBN - 1));
  const int t_hi = t_hi_key < 0 ? 0 : t_hi_key / kBN + 1;
  const int t_lo_key = p.wl >= 0 ? (wr1 - 1) - p.wl : 0;
  const int t_lo = t_lo_key <= 0 ? 0 : (t_lo_key + kBN - 1) / kBN;
  const uint32_t t_span = (uint32_t)max(t_hi - t_lo, 0);

  constexpr int kS = C::kSteps;             // first-product k-steps per half
  constexpr int kPV = 2 * C::kDBlocks;      // dQ MFMAs per half
  static_assert(kPV == kS, "one dQ MFMA per first-product step");
  constexpr int kEPS = 16 / kS;             // dS elements per first-product step
  constexpr int kLag = 2;                   // steps between an accumulator's last MFMA and its vector work
  static_assert(kLag <= C::kDBlocks && (kS - kLag) * kEPS >= 8, "lagged vector work");
  // registers r of a half hold keys 8 (r / 4) + 4 half + r % 4 (of the half)
  auto mask_half = [&](f32x16& x, int k0) {
    const int base = k0 + 4 * half - vis_lo;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t rel = (uint32_t)(base + 8 * (r >> 2) + (r & 3));
      if (rel > vis_span) x[r] = -INFINITY;
    }
  };
  // dS^T elements [e0, e0 + cnt) of a half, packed to 16 bits: P = exp2(s c -
  // lse log2 e) times dP - D
  auto ds_elems = [&](const f32x16& x, const f32x16& dp, int e0, int cnt, uint32_t (&y)[8]) {
#pragma unroll
    for (int e = e0; e < e0 + cnt; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], cexp, -lse2));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + 1], cexp, -lse2));
      y[e / 2] = pack2<IN>(p0 * (dp[e] - delta), p1 * (dp[e + 1] - delta));
    }
  };
  auto row_frag = [&](const unsigned char* tile, int hb, int st) {
    return *(const uint4*)(tile + 32 * hb * C::kRow + ka[st]);
  };
  // K^T fragment of dQ MFMA m of half hb (16 keys j = m / kDBlocks, column block m % kDBlocks)
  auto tr_frag = [&](const unsigned char* tile, int hb, int m) {
    const int jj = m / C::kDBlocks, c = m % C::kDBlocks;
    const unsigned char* base = tile + (32 * hb + 16 * jj) * (2 * D);
    const uint2 w0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + va[0][c])));
    const uint2 w1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + va[1][c])));
    return make_uint4(w0.x, w0.y, w1.x, w1.y);
  };
  auto dq_mfma = [&](uint4 a, const uint32_t (&y)[8], int m) {
    const int jj = m / C::kDBlocks, c = m % C::kDBlocks;
    acc[0][c] = mfma_16bit<IN>(a, make_uint4(y[4 * jj], y[4 * jj + 1], y[4 * jj + 2], y[4 * jj + 3]), acc[0][c]);
  };

  // One 64-key tile from the slots (kc, vc), in four phases so that each
  // half's vector work runs beside matrix work of the other:
  //   1. S_a = K_a Q^T, dP_a = V_a dO^T
  //   2. S_b, dP_b, step by step; half a's dS from step kLag on
  //   3. dQ^T += K_a^T dS_a^T; the rest of half a's dS first, then half b's
  //      from step kLag on (the MFMAs that need the last elements of dS_a
  //      come after step kLag)
  //   4. dQ^T += K_b^T dS_b^T, after the rest of half b's dS
  // Row fragments are read two steps ahead of their MFMAs, K^T fragments one
  // MFMA ahead; `hook(st)` (the next tile's loads) runs after phase-1 step
  // st.  Each step is fenced so the compiler keeps this order.
  auto step = [&](int kt, const unsigned char* kc, const unsigned char* vc, auto&& hook) {
    const bool masked = (uint32_t)(kt - t_lo) >= t_span;
    f32x16 sa, dpa, sb, dpb;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sa[r] = 0.f; dpa[r] = 0.f; sb[r] = 0.f; dpb[r] = 0.f;
    }
    uint32_t ya[8], yb[8];
    // the row fragments of both halves in order: step i < kS of half a, then of half b
    auto read_rows = [&](int i, uint4& rk, uint4& rv) {
      const int hb = i < kS ? 0 : 1, st = i < kS ? i : i - kS;
      rk = row_frag(kc, hb, st);
      rv = row_frag(vc, hb, st);
    };
    uint4 rk[2], rv[2];
    read_rows(0, rk[0], rv[0]);
    read_rows(1, rk[1], rv[1]);
    __builtin_amdgcn_sched_barrier(0);
    // 1
#pragma unroll
    for (int st = 0; st < kS; ++st) {
      const uint4 ck = rk[st & 1], cv = rv[st & 1];
      read_rows(st + 2, rk[st & 1], rv[st & 1]);
      sa = mfma_16bit<IN>(ck, qf[st], sa);
      dpa = mfma_16bit<IN>(cv, df[st], dpa);
      hook(st);
      __builtin_amdgcn_sched_barrier(0);
    }
    // 2
    uint4 ta = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int st = 0; st < kS; ++st) {
      const uint4 ck = rk[st & 1], cv = rv[st & 1];
      if (st + 2 < kS) read_rows(kS + st + 2, rk[st & 1], rv[st & 1]);
      if (st == kS - 1) ta = tr_frag(kc, 0, 0);
      sb = mfma_16bit<IN>(ck, qf[st], sb);
      dpb = mfma_16bit<IN>(cv, df[st], dpb);
      if (st == kLag && masked) mask_half(sa, kt * kBN);
      if (st >= kLag) ds_elems(sa, dpa, (st - kLag) * kEPS, kEPS, ya);
      __builtin_amdgcn_sched_barrier(0);
    }
    // 3
    uint4 tb = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int m = 0; m < kPV; ++m) {
      const uint4 cur = ta;
      if (m + 1 < kPV) ta = tr_frag(kc, 0, m + 1);
      else tb = tr_frag(kc, 1, 0);
      if (m < kLag) ds_elems(sa, dpa, (kS - kLag + m) * kEPS, kEPS, ya);
      dq_mfma(cur, ya, m);
      if (m == kLag && masked) mask_half(sb, kt * kBN + 32);
      if (m >= kLag) ds_elems(sb, dpb, (m - kLag) * kEPS, kEPS, yb);
      __builtin_amdgcn_sched_barrier(0);
    }
    // 4
#pragma unroll
    for (int m = 0; m < kPV; ++m) {
      const uint4 cur = tb;
      if (m + 1 < kPV) tb = tr_frag(kc, 1, m + 1);
      if (m < kLag) ds_elems(sb, dpb, (kPV - kLag + m) * kEPS, kEPS, yb);
      dq_mfma(cur, yb, m);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (kt_begin < kt_end) {
    issue(kt_begin, kbuf0, vbuf0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int kt = kt_begin;
    // The next tile's loads go out one per phase-1 step (its kDma K
    // blocks, then its kDma V blocks) rather than all before the step:
    // issued together right after the barrier, the four waves' loads queue
    // on the address unit (measured: the dQ kernel 2.4% faster spread).
    constexpr int kPer = (2 * C::kDma + kS - 1) / kS;
    auto dma_block = [&](const Rows64& rk, const Rows64& rv, unsigned char* kdst, unsigned char* vdst, int i) {
      if (i < C::kDma) load_16b_to_lds(rk.base, rk.bytes, k_off[i], kdst + (wave * C::kDma + i) * 1024);
      else if (i < 2 * C::kDma)
        load_16b_to_lds(rv.base, rv.bytes, v_off[i - C::kDma], vdst + (wave * C::kDma + i - C::kDma) * 1024);
    };
    auto none = [](int) {};
    for (; kt + 1 < kt_end; kt += 2) {
      {
        const Rows64 rk = rows64(kg, k_stride, C::kRow, (kt + 1) * kBN, n);
        const Rows64 rv = rows64(vg, v_stride, C::kRow, (kt + 1) * kBN, n);
        step(kt, kbuf0, vbuf0, [&](int st) {
#pragma unroll
          for (int u = 0; u < kPer; ++u) dma_block(rk, rv, kbuf1, vbuf1, st * kPer + u);
        });
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      {
        const bool more = kt + 2 < kt_end;
        const int kn = more ? kt + 2 : kt + 1;   // (a tile inside the range either way)
        const Rows64 rk = rows64(kg, k_stride, C::kRow, kn * kBN, n);
        const Rows64 rv = rows64(vg, v_stride, C::kRow, kn * kBN, n);
        step(kt + 1, kbuf1, vbuf1, [&](int st) {
          if (more) {
#pragma unroll
            for (int u = 0; u < kPer; ++u) dma_block(rk, rv, kbuf0, vbuf0, st * kPer + u);
          }
        });
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (kt < kt_end) step(kt, kbuf0, vbuf0, none);
  }

  if (ok) {
    unsigned char* dqg = (unsigned char*)p.dq + ((int64_t)b * p.dq_sb + (int64_t)h * p.dq_sh + (int64_t)qrow * p.dq_ss) * 2;
    store_rows<IN, D>(dqg, acc[0], p.scale, half);
    if (half == 0) p.delta[(int64_t)b * p.delta_sb + (int64_t)h * p.delta_sh + qrow] = delta;
  }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
// One workgroup of 8 waves per (batch, K/V head, 128 keys), two roles per 32
// keys (waves w and w + 4, which the hardware places on the same SIMD):
//   * role A (waves 0-3): S = Q K^T, P = exp2(S c - lse log2 e), dV^T += dO^T P;
//     P also goes to LDS;
//   * role B (waves 4-7), one tile behind: dP = dO V^T, dS = P o (dP - D)
//     with P from LDS, dK^T += Q^T dS.
// Each role issues 32 MFMAs per 64-row tile, and the two waves of a SIMD
// interleave one's vector work with the other's MFMAs.  Q and dO tiles of 64
// rows stream through three LDS slots: role A reads tile i, role B tile i - 1,
// and the DMA fills tile i + 1.  K^T (role A) or V^T (role B) and the dV^T or
// dK^T accumulators stay in registers (lane = key).
template <In IN, int D>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv_kernel(const BwdParams p) {
  using C = BwdCfg<IN, D>;
  constexpr int kDma = C::kTile / 1024 / 8;   // 1 KB DMA instructions per tile and tensor, per wave of eight
  // three slots as separate objects, so the compiler can tell the DMA into one
  // from the reads of another (a single array would make it wait for the DMA)
  __shared__ __attribute__((aligned(1024))) unsigned char qbuf0[C::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char qbuf1[C::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char qbuf2[C::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char obuf0[C::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char obuf1[C::kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char obuf2[C::kTile];
  // P of a tile from role A to role B: [parity][wave pair][16-byte group j][lane]
  __shared__ __attribute__((aligned(1024))) uint4 pbuf[2][4][4][64];
  __shared__ __attribute__((aligned(16))) float lbuf[3][64];   // lse * log2(e) per query row
  __shared__ __attribute__((aligned(16))) float dbuf[3][64];   // -D per query row

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool role_b = wave >= 4;
  const int kw = wave & 3;           // which 32 keys of the block
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int n = p.n;

  // key blocks near the start first: under a causal mask they see the most queries
  const int bhk_count = p.batch * p.heads_kv;
  const int2 wo = bwd_order((int)blockIdx.x, p.k_blocks, bhk_count);
  const int kb = wo.x;
  const int bhk = wo.y;
  const int b = bhk / p.heads_kv;
  const int hkv = bhk - b * p.heads_kv;
  const int k0 = kb * 128;
  const int key = k0 + kw * 32 + col;
  const bool kok = key < n;

  // K^T (role A) or V^T (role B) in registers (lane = key)
  uint4 kvf[C::kSteps];
  {
    const int kr = kok ? key : 0;
    const unsigned char* src = role_b
        ? (const unsigned char*)p.v + ((int64_t)b * p.v_sb + (int64_t)hkv * p.v_sh + (int64_t)kr * p.v_ss) * 2
        : (const unsigned char*)p.k + ((int64_t)b * p.k_sb + (int64_t)hkv * p.k_sh + (int64_t)kr * p.k_ss) * 2;
    load_row_frags<D>(kvf, src, kok, half);
  }
  const float cexp = p.c_log2;

  // queries that can see a key of this block: [qlo, qhi)
  int qlo = 0, qhi = n;
  if (p.causal) qlo = max(qlo, k0);
  if (p.wr >= 0) qlo = max(qlo, k0 - p.wr);
  if (p.wl >= 0) qhi = min(qhi, k0 + 128 + p.wl);
  const int qt_begin = qlo / 64;
  const int qt_end = qhi > qlo ? (qhi + 63) / 64 : qt_begin;
  // queries that see this lane's key: [qv_lo, qv_lo + qv_span]
  int qv_lo = 0, qv_hi = n - 1;
  if (p.causal) qv_lo = max(qv_lo, key);
  if (p.wr >= 0) qv_lo = max(qv_lo, key - p.wr);
  if (p.wl >= 0) qv_hi = min(qv_hi, key + p.wl);
  const uint32_t qv_span = (uint32_t)(qv_hi - qv_lo);   // (keys past n: never stored)
  const int kw0 = k0 + kw * 32;
  const int kw1 = min(kw0 + 32, n);
  // 32-row blocks starting at r0 whose rows see every key of this wave's
  // keys: each visibility condition is monotone in r0, so they form one
  // interval [vis_r0, vis_r1]
  int vis_r0 = 0, vis_r1 = 1 << 30;
  {
    const int kw1s = kw1 > kw0 ? kw1 : kw0 + 1;
    if (p.causal) vis_r0 = max(vis_r0, kw1s - 1);
    if (p.wr >= 0) vis_r0 = max(vis_r0, kw1s - 1 - p.wr);
    if (p.wl >= 0 && n > kw0 + p.wl + 1) vis_r1 = kw0 + p.wl - 31;
    if (kw1s > n) vis_r1 = -1;
  }

  const int q_stride = (int)(p.q_ss * 2), o_stride = (int)(p.do_ss * 2);
  uint32_t ka[C::kSteps];
  row_offsets<D>(ka, col, half);
  uint32_t va[2][C::kDBlocks];
  tr_offsets<D>(va, lane);

  // dV^T (role A) or dK^T (role B)
  f32x16 acc[1][C::kDBlocks];
#pragma unroll
  for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][c][r] = 0.f;

  // work: (query head of the group, query tile) pairs
  const int qtiles = qt_end - qt_begin;
  const int items = qtiles * p.group;
  float row_val = 0.f;   // lse or D of one query row, staged through a register
  // The items in order: query head hkv * group + gi, query tile qt (fastest).
  // A cursor carries its head's Q and dO bases and lse and D rows, so a tile
  // costs a 32-bit offset (the host bounds a head's rows below 2^32 bytes)
  // and a select between the whole-tile and last-tile byte counts.
  struct Cursor {
    int gi, qt;
    const unsigned char* qh;
    const unsigned char* oh;
    const float* lh;
    const float* dh;
  };
  auto set_head = [&](Cursor& c) {
    const int h = hkv * p.group + min(c.gi, p.group - 1);
    c.qh = (const unsigned char*)p.q + ((int64_t)b * p.q_sb + (int64_t)h * p.q_sh) * 2;
    c.oh = (const unsigned char*)p.dout + ((int64_t)b * p.do_sb + (int64_t)h * p.do_sh) * 2;
    c.lh = p.lse + (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh;
    c.dh = p.delta + (int64_t)b * p.delta_sb + (int64_t)h * p.delta_sh;
  };
  auto advance = [&](Cursor& c) {
    if (++c.qt == qt_end) {
      c.qt = qt_begin;
      ++c.gi;
      set_head(c);
    }
  };
  const int qt_last = (n - 1) / 64;
  const int q_full = 63 * q_stride + C::kRow, q_tail = (n - 1 - 64 * qt_last) * q_stride + C::kRow;
  const int o_full = 63 * o_stride + C::kRow, o_tail = (n - 1 - 64 * qt_last) * o_stride + C::kRow;
  const uint32_t q_tstride = 64u * (uint32_t)q_stride, o_tstride = 64u * (uint32_t)o_stride;
  // DMA of item c's Q and dO tiles (c.qt < qt_end <= qt_last + 1) and load of
  // its rows' lse and D values
  auto issue = [&](const Cursor& c, unsigned char* qdst, unsigned char* odst) {
    const bool last = c.qt == qt_last;
    const unsigned char* qbase = c.qh + (uint32_t)c.qt * q_tstride;
    const unsigned char* obase = c.oh + (uint32_t)c.qt * o_tstride;
    const int qbytes = last ? q_tail : q_full, obytes = last ? o_tail : o_full;
    // the row value first: its load is then not queued behind the DMA
    const int r = c.qt * 64 + (tid & 63);
    if (tid < 64) {
      row_val = r < n ? c.lh[r] : INFINITY;
    } else if (tid < 128) {
      row_val = r < n ? c.dh[r] : 0.f;
    }
    // Only role A's waves issue the tile's blocks: role B's waves reach the
    // end-of-tile barrier last, role A's wait there (measured 0.7-0.9% off
    // the backward against all eight waves issuing).
    if (!role_b) {
#pragma unroll
      for (int i = 0; i < 2 * kDma; ++i) {
        // (recomputed per tile: a few VALU instead of registers held across the loop)
        const int blk = wave * 2 * kDma + i;
        load_16b_to_lds(qbase, qbytes, dma_offset<C::kRow>(blk, lane, q_stride), qdst + blk * 1024);
        load_16b_to_lds(obase, obytes, dma_offset<C::kRow>(blk, lane, o_stride), odst + blk * 1024);
      }
    }
  };
  auto commit = [&](int slot) {
    if (tid < 64) lbuf[slot][tid] = __builtin_isfinite(row_val) ? row_val * kLog2e : INFINITY;
    else if (tid < 128) dbuf[slot][tid - 64] = -row_val;
  };

  constexpr int kPV = 2 * C::kDBlocks;                 // second-product MFMAs per half
  constexpr int kElemPerStep = 16 / C::kSteps;         // vector elements of a half per first-product step
  constexpr int kElemPerPV = 16 / kPV;                 // ... per second-product MFMA
  static_assert(kPV == C::kSteps, "one second-product MFMA per first-product step");
  // registers r of a half hold query rows 8 (r / 4) + 4 half + r % 4
  auto mask_half = [&](f32x16& s, int r0) {
    const int base = r0 + 4 * half - qv_lo;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t rel = (uint32_t)(base + 8 * (r >> 2) + (r & 3));
      if (rel > qv_span) s[r] = -INFINITY;
    }
  };
  auto row_frag = [&](const unsigned char* tile, int qh, int st) {
    return *(const uint4*)(tile + 32 * qh * C::kRow + ka[st]);
  };
  auto tr_frag = [&](const unsigned char* tile, int qh, int m) {
    const int jj = m / C::kDBlocks, c = m % C::kDBlocks;
    const unsigned char* base = tile + (32 * qh + 16 * jj) * (2 * D);
    const uint2 w0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + va[0][c])));
    const uint2 w1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + va[1][c])));
    return make_uint4(w0.x, w0.y, w1.x, w1.y);
  };
  auto pv_mfma = [&](uint4 a, const uint32_t (&pk)[8], int m) {
    const int jj = m / C::kDBlocks, c = m % C::kDBlocks;
    acc[0][c] = mfma_16bit<IN>(a, make_uint4(pk[4 * jj], pk[4 * jj + 1], pk[4 * jj + 2], pk[4 * jj + 3]), acc[0][c]);
  };
  // elements [e0, e0 + cnt) of a half.  Role A: P = exp2(s c - lse), packed,
  // with `vals` the lse of the tile's rows (registers r of a half hold query
  // rows 8 (r / 4) + 4 half + r % 4; read four at a time, when needed).
  // Role B: dS = P x with x = dP - D (its accumulator started at -D), from
  // P's packed pairs.
  // Role B reads P's pairs from `pin` (the half's two 16-byte groups in LDS),
  // four pairs at a time.  `rv` and `pv` carry the values read for element e
  // with e % 4 == 0 (e % 8 == 0) over the following calls.
  auto elems = [&](auto role_tag, const f32x16& x, const float* vals, int qh, const uint4* pin, int e0, int cnt,
                   uint32_t (&out)[8], float4& rv, uint4& pv) {
#pragma unroll
    for (int e = e0; e < e0 + cnt; e += 2) {
      if constexpr (decltype(role_tag)::value) {
        if (e % 8 == 0) pv = pin[(e / 8) * 64 + lane];
        const uint32_t w = (e % 8) / 2 == 0 ? pv.x : (e % 8) / 2 == 1 ? pv.y : (e % 8) / 2 == 2 ? pv.z : pv.w;
        const float p0 = unpack_lo<IN>(w), p1 = unpack_hi<IN>(w);
        out[e / 2] = pack2<IN>(p0 * x[e], p1 * x[e + 1]);
      } else {
        if (e % 4 == 0) rv = *(const float4*)&vals[32 * qh + 8 * (e / 4) + 4 * half];
        const float r0 = (e % 4 == 0) ? rv.x : rv.z;
        const float r1 = (e % 4 == 0) ? rv.y : rv.w;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], cexp, -r0));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + 1], cexp, -r1));
        out[e / 2] = pack2<IN>(p0, p1);
      }
    }
  };

  // One 64-row tile (halves a, b of 32 query rows) of one role, in four
  // phases so each half's vector work runs beside matrix work of the other:
  //   1. X_a = R_a F^T                  (R = Q, F = K for role A; dO, V for B)
  //   2. X_b, step by step between the vector work of half a
  //   3. acc += T_a^T Y_a                (T = dO, Y = P for role A; Q, dS for B)
  //      between the vector work of half b
  //   4. acc += T_b^T Y_b
  // Operand reads run one phase ahead of their MFMAs, and a half's vector
  // work starts kLag MFMA steps after its accumulator's last MFMA (whose
  // result it waits for otherwise).  Each step is fenced so the compiler
  // keeps this order.  `par`: the tile's parity (its P buffer), `q0`: its
  // first query row.
  constexpr int kLag = 2;
  auto tile_step = [&](auto role_tag, int par, int q0, const unsigned char* rows, const unsigned char* trs, int lslot) {
    constexpr bool kB = decltype(role_tag)::value;
    const float* vals = kB ? dbuf[lslot] : lbuf[lslot];
    const uint4* pb = &pbuf[par][kw][0][0];
    bool masked_a = false, masked_b = false;
    if constexpr (!kB) {
      masked_a = !(q0 >= vis_r0 && q0 <= vis_r1);
      masked_b = !(q0 + 32 >= vis_r0 && q0 + 32 <= vis_r1);
    }
    // role B's dP accumulators start at -D of their rows (four consecutive
    // registers hold four consecutive rows), so the MFMAs leave dP - D
    f32x16 xa, xb;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float4 da = kB ? *(const float4*)&vals[8 * jj + 4 * half] : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 db = kB ? *(const float4*)&vals[32 + 8 * jj + 4 * half] : make_float4(0.f, 0.f, 0.f, 0.f);
      xa[4 * jj] = da.x; xa[4 * jj + 1] = da.y; xa[4 * jj + 2] = da.z; xa[4 * jj + 3] = da.w;
      xb[4 * jj] = db.x; xb[4 * jj + 1] = db.y; xb[4 * jj + 2] = db.z; xb[4 * jj + 3] = db.w;
    }
    // 1
    uint4 ra[C::kSteps], rb[C::kSteps];
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) ra[st] = row_frag(rows, 0, st);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) {
      xa = mfma_16bit<IN>(ra[st], kvf[st], xa);
      rb[st] = row_frag(rows, 1, st);
      __builtin_amdgcn_sched_barrier(0);
    }
    // 2: X_b; half a's vector work from step kLag on
    uint32_t ya[8], yb[8];
    uint4 ta[kPV], tb[kPV];
    float4 rva = make_float4(0.f, 0.f, 0.f, 0.f), rvb = rva;
    uint4 pva = make_uint4(0, 0, 0, 0), pvb = pva;
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) {
      xb = mfma_16bit<IN>(rb[st], kvf[st], xb);
      ta[st] = tr_frag(trs, 0, st);
      if (st == kLag && masked_a) mask_half(xa, q0);
      if (st >= kLag) elems(role_tag, xa, vals, 0, pb, (st - kLag) * kElemPerStep, kElemPerStep, ya, rva, pva);
      __builtin_amdgcn_sched_barrier(0);
    }
    // 3: acc += T_a^T Y_a; the rest of half a's vector work, then half b's
    // from step kLag on (the MFMAs that need Y_a's last elements come after
    // step kLag)
    // (the MFMAs of steps < kLag read elements 0-7 only, all done in phase 2)
    static_assert(kLag <= C::kDBlocks && (C::kSteps - kLag) * kElemPerStep >= 8 && (kPV - kLag) * kElemPerPV >= 8,
                  "lagged vector work");
#pragma unroll
    for (int m = 0; m < kPV; ++m) {
      if (m < kLag)
        elems(role_tag, xa, vals, 0, pb, (C::kSteps - kLag + m) * kElemPerStep, kElemPerStep, ya, rva, pva);
      pv_mfma(ta[m], ya, m);
      tb[m] = tr_frag(trs, 1, m);
      if (m == kLag && masked_b) mask_half(xb, q0 + 32);
      if (m >= kLag) elems(role_tag, xb, vals, 1, pb + 2 * 64, (m - kLag) * kElemPerPV, kElemPerPV, yb, rvb, pvb);
      if (!kB && m == kLag - 1) {
        uint4* pw = &pbuf[par][kw][0][0];
        pw[0 * 64 + lane] = make_uint4(ya[0], ya[1], ya[2], ya[3]);
        pw[1 * 64 + lane] = make_uint4(ya[4], ya[5], ya[6], ya[7]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // 4: acc += T_b^T Y_b, after the rest of half b's vector work
#pragma unroll
    for (int m = 0; m < kPV; ++m) {
      if (m < kLag)
        elems(role_tag, xb, vals, 1, pb + 2 * 64, (kPV - kLag + m) * kElemPerPV, kElemPerPV, yb, rvb, pvb);
      pv_mfma(tb[m], yb, m);
      if (!kB && m == kLag - 1) {
        uint4* pw = &pbuf[par][kw][0][0];
        pw[2 * 64 + lane] = make_uint4(yb[0], yb[1], yb[2], yb[3]);
        pw[3 * 64 + lane] = make_uint4(yb[4], yb[5], yb[6], yb[7]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Iteration i: role A takes tile i (slot i % 3), role B tile i - 1 (slot
  // (i - 1) % 3, P from iteration i - 1), the DMA fetches tile i + 1 into slot
  // (i + 1) % 3; the barrier at its end publishes tile i + 1 and P(i), and
  // frees slot (i - 1) % 3 for the next fetch.  Slots are named statically
  // (loop unrolled by three).
  // `nxt`: item i + 1; `cur`: item i.
  // Each role runs its own copy of the loop (roles are fixed per wave), so
  // the accumulators keep one register assignment throughout; both copies
  // meet the same barriers.
  Cursor nxt{0, qt_begin, nullptr, nullptr, nullptr, nullptr};
  set_head(nxt);
  Cursor cur = nxt;
  auto iteration = [&](auto role_tag, int i, unsigned char* qa, unsigned char* oa, unsigned char* qb,
                       unsigned char* ob, unsigned char* qn, unsigned char* on, int sa, int sb, int sn)
                       __attribute__((always_inline)) {
    if (i + 1 < items) issue(nxt, qn, on);
    advance(nxt);
    if constexpr (!decltype(role_tag)::value) {
      if (i < items) tile_step(role_tag, i & 1, cur.qt * 64, qa, oa, sa);
    } else {
      if (i >= 1) tile_step(role_tag, (i - 1) & 1, 0, ob, qb, sb);
    }
    advance(cur);
    __builtin_amdgcn_s_waitcnt(0);
    if (i + 1 < items) commit(sn);
    __syncthreads();
  };
  auto loop = [&](auto role_tag) __attribute__((always_inline)) {
    const int total = items + 1;
    for (int i = 0; i < total; i += 3) {
      iteration(role_tag, i, qbuf0, obuf0, qbuf2, obuf2, qbuf1, obuf1, 0, 2, 1);
      if (i + 1 >= total) break;
      iteration(role_tag, i + 1, qbuf1, obuf1, qbuf0, obuf0, qbuf2, obuf2, 1, 0, 2);
      if (i + 2 >= total) break;
      iteration(role_tag, i + 2, qbuf2, obuf2, qbuf1, obuf1, qbuf0, obuf0, 2, 1, 0);
    }
  };
  if (items > 0) {
    issue(nxt, qbuf0, obuf0);
    advance(nxt);
    __builtin_amdgcn_s_waitcnt(0);
    commit(0);
    __syncthreads();
    if (role_b) loop(BoolTag<true>{});
    else loop(BoolTag<false>{});
  }

  if (kok) {
    if (role_b) {
      unsigned char* dkg = (unsigned char*)p.dk + ((int64_t)b * p.dk_sb + (int64_t)hkv * p.dk_sh + (int64_t)key * p.dk_ss) * 2;
      store_rows<IN, D>(dkg, acc[0], p.scale, half);
    } else {
      unsigned char* dvg = (unsigned char*)p.dv + ((int64_t)b * p.dv_sb + (int64_t)hkv * p.dv_sh + (int64_t)key * p.dv_ss) * 2;
      store_rows<IN, D>(dvg, acc[0], 1.f, half);
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launch
// ---------------------------------------------------------------------------
template <In IN, int D>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  const dim3 block(256);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<IN, D>), dim3((unsigned)((int64_t)p.q_tiles * p.batch * p.heads)), block, 0,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<IN, D>), dim3((unsigned)((int64_t)p.k_blocks * p.batch * p.heads_kv)),
                     dim3(512), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int in_dtype, int d, hipStream_t stream) {
  if (in_dtype == 1 && d == 64) return launch_bwd_t<In::F16, 64>(p, stream);
  if (in_dtype == 1 && d == 128) return launch_bwd_t<In::F16, 128>(p, stream);
  if (in_dtype == 2 && d == 64) return launch_bwd_t<In::BF16, 64>(p, stream);
  if (in_dtype == 2 && d == 128) return launch_bwd_t<In::BF16, 128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace ea
