// Exact attention forward for gfx950 (CDNA4): fused Q.K^T -> online softmax
// -> P.V, one workgroup per (batch, head, query tile).
//
// The method ("FlashAttention", aiunderstanding.org, "Teknisk insikt"): load
// small blocks of queries, keys and values on chip, compute partial outputs,
// and rescale running sums as new blocks arrive, so the N x N score matrix is
// never written to HBM and the whole attention is one kernel.
//
// How it maps onto a CDNA4 compute unit:
//   * 4 wavefronts x 32 query rows = 128 rows per workgroup (BM); K/V tiles of
//     64 keys (BN) are staged in LDS, double buffered, shared by the 4 waves.
//   * Each wave computes S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16}
//     (v_mfma_scale_f32_32x32x64_f8f6f4 for fp8): K (the A operand) comes
//     from LDS, Q^T (the B operand) stays in registers for the whole kernel.
//     In the 32x32 accumulator layout lane l holds column l%32, i.e. one
//     query row, and 16 of the 32 keys; lane l^32 holds the other 16.  A row
//     max therefore needs one exchange between the two wave halves, and the
//     row sum needs none until the epilogue.
//   * P^T leaves the accumulator already in the B-operand layout of
//     O^T += V^T P^T (after a bf16/f16 conversion), so P never touches LDS.
//     V^T fragments come from LDS with ds_read_b64_tr_b16 (transposing read).
//   * LDS rows are XOR-swizzled in 16-byte units so that both the K reads
//     (32 rows, same column) and the transposing V reads (4 rows x 64 bytes)
//     hit 64 distinct banks per half-wave.
//   * The running max is only moved (and O, l rescaled) when it grows by
//     more than 2^8 in the exp2 domain; O and l always share the same
//     reference, so O/l is unchanged in exact arithmetic.
//   * Only tiles that cross the causal diagonal, the window edge or the end
//     of the sequence evaluate the mask; tiles outside the visible range are
//     never loaded.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_kernel.h"

namespace ea {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 32 * kWaves;   // query rows per workgroup
constexpr int kBN = 64;            // keys per K/V tile
constexpr float kLn2 = 0.6931471805599453f;
// Largest growth of the running max (in log2 units) tolerated before O and l
// are rescaled: p <= 2^8 stays far from fp16/bf16/fp32 overflow.
constexpr float kRescaleThreshold = 8.0f;

enum class In { F16, BF16, FP8 };

// ---------------------------------------------------------------------------
// LDS layout: a K or V tile is kBN rows of `row_bytes` bytes, split into
// 16-byte units.  Unit u of row r is stored at unit u ^ swz(r).
//   256-byte rows (16 units, d=128 at 16 bits): swz = ((r&3)<<2) | ((r>>2)&3)
//   128-byte rows (8 units, d=64 at 16 bits or d=128 at 8 bits):
//       swz = (((r>>1)&1)<<2) | ((r>>2)&3)
// Both are bijections on 16 consecutive rows (K reads: 16 lanes, 16 rows,
// one unit) and spread 4 consecutive rows x 4 consecutive units over 16
// distinct bank groups (the transposing V reads).
// ---------------------------------------------------------------------------
template <int ROW_BYTES>
__device__ __forceinline__ int swz_of(int row) {
  static_assert(ROW_BYTES == 256 || ROW_BYTES == 128, "row size");
  if constexpr (ROW_BYTES == 256) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Byte offset of logical 16-byte unit `unit` of tile row `row`.
template <int ROW_BYTES>
__device__ __forceinline__ int lds_offset(int row, int unit) {
  return row * ROW_BYTES + ((unit ^ swz_of<ROW_BYTES>(row)) << 4);
}

// Logical unit held at physical unit `phys` of `row` (XOR is an involution).
template <int ROW_BYTES>
__device__ __forceinline__ int swizzled_unit(int row, int phys) {
  return phys ^ swz_of<ROW_BYTES>(row);
}

template <In IN>
__device__ __forceinline__ f32x16 mfma_16bit(uint4 a, uint4 b, f32x16 c) {
  if constexpr (IN == In::BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Pack two fp32 values into the P operand type (round to nearest even).
template <In IN>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (IN == In::F16) {
    _Float16 x = (_Float16)a, y = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
  } else {
    __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
  }
}

// Store 4 consecutive output elements (fp32 -> output type, RNE).
template <In IN>
__device__ __forceinline__ void store4(void* dst, float a, float b, float c, float d) {
  uint2 w;
  if constexpr (IN == In::F16) { w.x = pack2<In::F16>(a, b); w.y = pack2<In::F16>(c, d); }
  else { w.x = pack2<In::BF16>(a, b); w.y = pack2<In::BF16>(c, d); }
  *(uint2*)dst = w;
}

// fp8 e4m3 x16 (one uint4) -> bf16 x16 (two uint4), exact.
__device__ __forceinline__ void fp8x16_to_bf16(uint4 in, uint4& lo, uint4& hi) {
  uint32_t w[4] = {in.x, in.y, in.z, in.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 0);
    float b = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 1);
    float c = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 2);
    float d = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 3);
    o[2 * i] = pack2<In::BF16>(a, b);
    o[2 * i + 1] = pack2<In::BF16>(c, d);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// Visible-key range of a query tile [q0, q0+BM) and the mask classification of
// a key tile.  Mirrors the mask definition: key j visible from query i iff
// j < n, (!causal || j <= i), (wl < 0 || j >= i - wl), (wr < 0 || j <= i + wr).
struct KeyRange {
  int lo, hi;   // [lo, hi) keys that any row of the tile can see
};

__device__ __forceinline__ KeyRange tile_key_range(int q0, int qrows, int n, int causal, int wl, int wr) {
  int qlast = min(q0 + qrows, n) - 1;
  int lo = wl >= 0 ? max(0, q0 - wl) : 0;
  int hi = n;
  if (causal) hi = min(hi, qlast + 1);
  if (wr >= 0) hi = min(hi, qlast + wr + 1);
  return {lo, max(lo, hi)};
}

// True when every (row, key) pair of rows [r0, r1) x keys [k0, k1) is visible.
__device__ __forceinline__ bool block_all_visible(int r0, int r1, int k0, int k1, int n, int causal, int wl, int wr) {
  if (k1 > n) return false;
  if (causal && k1 - 1 > r0) return false;
  if (wl >= 0 && k0 < (r1 - 1) - wl) return false;
  if (wr >= 0 && k1 - 1 > r0 + wr) return false;
  return true;
}

// True when no (row, key) pair of rows [r0, r1) x keys [k0, k1) is visible.
__device__ __forceinline__ bool block_none_visible(int r0, int r1, int k0, int k1, int n, int causal, int wl, int wr) {
  if (k0 >= n || r0 >= r1) return true;
  if (causal && k0 > r1 - 1) return true;
  if (wl >= 0 && k1 - 1 < r0 - wl) return true;
  if (wr >= 0 && k0 > (r1 - 1) + wr) return true;
  return false;
}

// Value of the low / high 16-bit half of a packed pair, as fp32.
template <In IN>
__device__ __forceinline__ float unpack_lo(uint32_t w) {
  if constexpr (IN == In::F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  else return __builtin_bit_cast(float, w << 16);
}
template <In IN>
__device__ __forceinline__ float unpack_hi(uint32_t w) {
  if constexpr (IN == In::F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  else return __builtin_bit_cast(float, w & 0xffff0000u);
}

// O^T += V^T P^T over one 64-key tile.  P^T (16-bit, B operand) is in the
// layout the S^T accumulator left it: lane l holds query l%32 and, for
// k-step (kb, j0), keys 32 kb + 8 j0 + {4 half + t, 8 + 4 half + t}, t < 4.
// The matching V^T fragment (A operand: row d = l%32 of the 32-column block,
// the same 8 keys) is gathered with two transposing LDS reads: within each
// 16-lane group, source lane sl points at key (base + sl/4), columns
// 4 (sl%4) .. +3, and lane i receives column i of 4 consecutive keys.
template <In PIN, int D>
__device__ __forceinline__ void pv_accumulate(f32x16 (&acc)[D / 32], const uint32_t (&pk)[2][8],
                                              const unsigned char* vl, int lane) {
  const int g = lane >> 4;          // 16-lane group
  const int sl = lane & 15;         // source lane within the group
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += 2) {
      const uint4 bop = make_uint4(pk[kb][2 * j0], pk[kb][2 * j0 + 1], pk[kb][2 * j0 + 2], pk[kb][2 * j0 + 3]);
      const int kbase = 32 * kb + 8 * j0;
      const int vrow = kbase + 4 * (g >> 1) + (sl >> 2);
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const int dcol = 32 * c + 16 * (g & 1) + 4 * (sl & 3);
        const int unit = dcol >> 3;
        const int hoff = (dcol & 7) * 2;
        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vl + lds_offset<2 * D>(vrow, unit) + hoff));
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vl + lds_offset<2 * D>(vrow + 8, unit) + hoff));
        const uint2 w0 = __builtin_bit_cast(uint2, t0);
        const uint2 w1 = __builtin_bit_cast(uint2, t1);
        const uint4 aop = make_uint4(w0.x, w0.y, w1.x, w1.y);
        acc[c] = mfma_16bit<PIN>(aop, bop, acc[c]);
      }
    }
  }
}

template <In IN, int D>
struct Cfg {
  static constexpr bool kFp8 = (IN == In::FP8);
  static constexpr int kInBytes = kFp8 ? 1 : 2;
  static constexpr int kKRow = D * kInBytes;         // bytes per K row in LDS
  static constexpr int kVRow = D * 2;                // V is 16-bit in LDS
  static constexpr int kKTile = kBN * kKRow;
  static constexpr int kVTile = kBN * kVRow;
  static constexpr int kStage = kKTile + kVTile;
  static constexpr int kLds = 2 * kStage;            // double buffered
  // fp8 V: 16-byte global chunks per thread per tile (register staged)
  static constexpr int kVPer = kBN * D * kInBytes / 16 / kThreads;
  static_assert(kFp8 ? (kBN * D * kInBytes / 16) % kThreads == 0 : true, "tile split");
  static_assert(kKTile % (1024 * kWaves) == 0 && kVTile % (1024 * kWaves) == 0, "DMA split");
  static constexpr int kQSteps = kFp8 ? D / 64 : D / 16;   // MFMA k-steps for S
  static constexpr int kDBlocks = D / 32;                  // 32-wide output column blocks
};

template <In IN, int D>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(const FwdParams p) {
  using C = Cfg<IN, D>;
  constexpr In PIN = (IN == In::F16) ? In::F16 : In::BF16;   // type of P, V in LDS and O
  // Two statically distinct stage buffers (K tile then V tile): the loop below
  // is unrolled by two so that each half names its buffers at compile time,
  // which lets the compiler keep the LDS DMA into one buffer in flight while
  // the other one is read.
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[C::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[C::kStage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
  const int lane = tid & 63;
  const int half = lane >> 5;      // which 16 of each 32 keys this lane holds
  const int col = lane & 31;       // the query row (within the wave) this lane owns

  // ---- work assignment: heaviest query tiles first; consecutive workgroups
  // take consecutive (batch, head) pairs so one head stays on one XCD when
  // B*H is a multiple of 8.
  const int bh_count = p.batch * p.heads;
  const int tile = p.q_tiles - 1 - (int)(blockIdx.x / bh_count);
  const int bh = (int)(blockIdx.x % bh_count);
  const int b = bh / p.heads;
  const int h = bh - b * p.heads;
  const int q0 = tile * kBM;
  const int n = p.n;

  const unsigned char* qg = (const unsigned char*)p.q + ((int64_t)b * p.q_sb + (int64_t)h * p.q_sh) * C::kInBytes;
  const unsigned char* kg = (const unsigned char*)p.k + ((int64_t)b * p.k_sb + (int64_t)h * p.k_sh) * C::kInBytes;
  const unsigned char* vg = (const unsigned char*)p.v + ((int64_t)b * p.v_sb + (int64_t)h * p.v_sh) * C::kInBytes;
  const int k_row_stride = (int)(p.k_ss * C::kInBytes);   // bytes; < 2^31 (checked by the host)
  const int v_row_stride = (int)(p.v_ss * C::kInBytes);

  const KeyRange kr = tile_key_range(q0, kBM, n, p.causal, p.wl, p.wr);
  const int kt_begin = kr.lo / kBN;
  const int kt_end = (kr.hi + kBN - 1) / kBN;

  // ---- Q^T fragments (B operand), kept in registers for the whole kernel.
  const int qrow = q0 + wave * 32 + col;
  uint4 qf[C::kFp8 ? 2 * C::kQSteps : C::kQSteps];
  {
    const bool ok = qrow < n;
    const unsigned char* src = qg + (int64_t)(ok ? qrow : 0) * p.q_ss * C::kInBytes;
    if constexpr (C::kFp8) {
#pragma unroll
      for (int st = 0; st < C::kQSteps; ++st) {
        // lane holds d = 64 st + 32 half + [0, 32): two 16-byte pieces
        const uint4* g = (const uint4*)(src + 64 * st + 32 * half);
        qf[2 * st] = ok ? g[0] : make_uint4(0, 0, 0, 0);
        qf[2 * st + 1] = ok ? g[1] : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int st = 0; st < C::kQSteps; ++st) {
        // lane holds d = 16 st + 8 half + [0, 8)
        qf[st] = ok ? *(const uint4*)(src + (16 * st + 8 * half) * 2) : make_uint4(0, 0, 0, 0);
      }
    }
  }

  // ---- staging of one K/V tile into LDS (swizzled layout).
  // 16-bit K and V, and fp8 K, go straight from global memory to LDS
  // (global_load_lds_dwordx4): one wave instruction fills 1 KB of LDS, lane L
  // writing 16-byte unit L of it, so each lane fetches the global unit that
  // the swizzle maps to that LDS position.  Keys past the end are clamped to
  // the last key; those keys are masked (p = 0) in the boundary tile.
  // fp8 V goes through registers and is widened to bf16 on the way into LDS.
  constexpr int kKBlocks = C::kKTile / 1024 / kWaves;      // DMA instructions per wave, K
  constexpr int kVBlocks = C::kFp8 ? 0 : C::kVTile / 1024 / kWaves;
  int k_row[kKBlocks], k_col[kKBlocks];                    // tile row and byte column per DMA
  int v_row[kVBlocks > 0 ? kVBlocks : 1], v_col[kVBlocks > 0 ? kVBlocks : 1];
#pragma unroll
  for (int i = 0; i < kKBlocks; ++i) {
    const int pos = (wave * kKBlocks + i) * 64 + lane;       // physical unit in the tile
    k_row[i] = pos / (C::kKRow / 16);
    k_col[i] = (swizzled_unit<C::kKRow>(k_row[i], pos % (C::kKRow / 16))) * 16;
  }
#pragma unroll
  for (int i = 0; i < kVBlocks; ++i) {
    const int pos = (wave * kVBlocks + i) * 64 + lane;
    v_row[i] = pos / (C::kVRow / 16);
    v_col[i] = (swizzled_unit<C::kVRow>(v_row[i], pos % (C::kVRow / 16))) * 16;
  }
  uint4 vreg[C::kFp8 ? C::kVPer : 1];
  auto issue_tile = [&](int kt, unsigned char* dst) {
    const int k0 = kt * kBN;
    const int last = n - 1 - k0;                             // clamp rows past the end
    const unsigned char* kb_ = kg + (int64_t)k0 * k_row_stride;
#pragma unroll
    for (int i = 0; i < kKBlocks; ++i) {
      const int r = min(k_row[i], last);
      __builtin_amdgcn_global_load_lds((const void*)(kb_ + r * k_row_stride + k_col[i]),
                                       (__attribute__((address_space(3))) void*)(dst + (wave * kKBlocks + i) * 1024),
                                       16, 0, 0);
    }
    if constexpr (!C::kFp8) {
      const unsigned char* vb_ = vg + (int64_t)k0 * v_row_stride;
#pragma unroll
      for (int i = 0; i < kVBlocks; ++i) {
        const int r = min(v_row[i], last);
        __builtin_amdgcn_global_load_lds(
            (const void*)(vb_ + r * v_row_stride + v_col[i]),
            (__attribute__((address_space(3))) void*)(dst + C::kKTile + (wave * kVBlocks + i) * 1024), 16, 0, 0);
      }
    } else {
      const unsigned char* vb_ = vg + (int64_t)k0 * v_row_stride;
#pragma unroll
      for (int i = 0; i < C::kVPer; ++i) {
        const int id = tid + i * kThreads;
        const int r = min(id / (D / 16), last);
        vreg[i] = *(const uint4*)(vb_ + r * v_row_stride + (id % (D / 16)) * 16);
      }
    }
  };
  // fp8 only: widen the V tile held in registers and store it (bf16) to LDS.
  auto store_v_fp8 = [&](unsigned char* dst) {
    if constexpr (C::kFp8) {
      unsigned char* vl = dst + C::kKTile;
#pragma unroll
      for (int i = 0; i < C::kVPer; ++i) {
        const int id = tid + i * kThreads;
        const int row = id / (D / 16);           // 16 fp8 per global chunk
        const int unit = (id % (D / 16)) * 2;    // two 16-byte bf16 units
        uint4 lo, hi;
        fp8x16_to_bf16(vreg[i], lo, hi);
        *(uint4*)(vl + lds_offset<C::kVRow>(row, unit)) = lo;
        *(uint4*)(vl + lds_offset<C::kVRow>(row, unit + 1)) = hi;
      }
    }
  };

  // ---- running state
  f32x16 acc[C::kDBlocks];
#pragma unroll
  for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  float m_run = -INFINITY;     // reference max of the raw (unscaled) scores
  float neg_mc = 0.f;          // -m_run * c, or 0 while no key was seen
  float l_part = 0.f;          // this lane's share of the row sum
  const float cexp = p.c_log2;  // softmax scale * log2(e) (* fp8 descales)

  const int wr0 = q0 + wave * 32;          // this wave's first row
  const int wr1 = min(wr0 + 32, n);        // one past its last real row

  // One K/V tile of work for this wave, reading the tile staged in `cur`.
  auto compute_tile = [&](int kt, const unsigned char* cur) {
    const int k0 = kt * kBN;
    const unsigned char* kl = cur;
    const unsigned char* vl = cur + C::kKTile;
    if (block_none_visible(wr0, wr1, k0, k0 + kBN, n, p.causal, p.wl, p.wr)) return;
    const bool masked = !block_all_visible(wr0, wr1, k0, k0 + kBN, n, p.causal, p.wl, p.wr);
    // ---- S^T = K Q^T for the 64 keys: two 32x32 blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const int krow = 32 * kb + col;
      if constexpr (C::kFp8) {
#pragma unroll
        for (int st = 0; st < C::kQSteps; ++st) {
          const int u0 = (64 * st + 32 * half) / 16;
          const uint4 a0 = *(const uint4*)(kl + lds_offset<C::kKRow>(krow, u0));
          const uint4 a1 = *(const uint4*)(kl + lds_offset<C::kKRow>(krow, u0 + 1));
          i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          const uint4 b0 = qf[2 * st], b1 = qf[2 * st + 1];
          i32x8 bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, s[kb], 0, 0, 0, 127, 0, 127);
        }
      } else {
#pragma unroll
        for (int st = 0; st < C::kQSteps; ++st) {
          const uint4 a = *(const uint4*)(kl + lds_offset<C::kKRow>(krow, 2 * st + half));
          s[kb] = mfma_16bit<IN>(a, qf[st], s[kb]);
        }
      }
    }
    // ---- mask (boundary tiles only)
    if (masked) {
      const int qi = wr0 + col;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          bool vis = kj < n;
          if (p.causal) vis = vis && (kj <= qi);
          if (p.wl >= 0) vis = vis && (kj >= qi - p.wl);
          if (p.wr >= 0) vis = vis && (kj <= qi + p.wr);
          if (!vis) s[kb][r] = -INFINITY;
        }
    }
    // ---- online softmax
    float mt = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[1][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const bool grow = (m_new != -INFINITY) && (m_run == -INFINITY || (m_new - m_run) * cexp > kRescaleThreshold);
    if (__ballot(grow) != 0ull) {
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * cexp);
      m_run = m_new;
      neg_mc = (m_run == -INFINITY) ? 0.f : -m_run * cexp;
      l_part *= alpha;
#pragma unroll
      for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] *= alpha;
    }
    // p = exp2(s c - m c); the row sum uses the unrounded fp32 p.
    float e[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], cexp, neg_mc));
        l_part += e[kb][r];
      }
    uint32_t pk[2][8], pr[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        pk[kb][r] = pack2<PIN>(e[kb][2 * r], e[kb][2 * r + 1]);
        // Boundary tiles carry the rows with few visible keys, where the
        // 16-bit rounding of p does not average out: there the rounding
        // residual p - round16(p) goes through a second P.V pass.
        if (masked)
          pr[kb][r] = pack2<PIN>(e[kb][2 * r] - unpack_lo<PIN>(pk[kb][r]), e[kb][2 * r + 1] - unpack_hi<PIN>(pk[kb][r]));
      }
    pv_accumulate<PIN, D>(acc, pk, vl, lane);
    if (masked) pv_accumulate<PIN, D>(acc, pr, vl, lane);
  };

  // ---- main loop: tile kt is read from one stage while tile kt+1 lands in
  // the other.  Each barrier publishes the next tile (its DMA must have
  // landed, hence the full wait) and frees the stage just read.
  if (kt_begin < kt_end) {
    issue_tile(kt_begin, stage0);
    store_v_fp8(stage0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int kt = kt_begin;
    while (true) {
      issue_tile(min(kt + 1, kt_end - 1), stage1);
      compute_tile(kt, stage0);
      store_v_fp8(stage1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (++kt == kt_end) break;
      issue_tile(min(kt + 1, kt_end - 1), stage0);
      compute_tile(kt, stage1);
      store_v_fp8(stage0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (++kt == kt_end) break;
    }
  }

  // ---- epilogue: O = O_acc / l (* v descale), LSE = ln(2) * (m c + log2 l)
  const float l_row = l_part + __shfl_xor(l_part, 32);
  if (qrow < n) {
    const float inv = l_row > 0.f ? p.v_descale / l_row : 0.f;
    constexpr int kOutBytes = 2;
    unsigned char* og = (unsigned char*)p.o + ((int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)qrow * p.o_ss) * kOutBytes;
#pragma unroll
    for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * c + 8 * j + 4 * half;
        store4<PIN>(og + d * kOutBytes, acc[c][4 * j] * inv, acc[c][4 * j + 1] * inv, acc[c][4 * j + 2] * inv,
                    acc[c][4 * j + 3] * inv);
      }
    if (p.lse != nullptr && half == 0) {
      const float lse = (m_run == -INFINITY || !(l_row > 0.f))
                            ? -INFINITY
                            : (m_run * cexp + __builtin_amdgcn_logf(l_row)) * kLn2;
      p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + qrow] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launch
// ---------------------------------------------------------------------------
template <In IN, int D>
static hipError_t launch_t(const FwdParams& p, hipStream_t stream) {
  using C = Cfg<IN, D>;
  const dim3 grid((unsigned)((int64_t)p.q_tiles * p.batch * p.heads));
  const dim3 block(kThreads);
  hipLaunchKernelGGL((attn_fwd_kernel<IN, D>), grid, block, 0, stream, p);
  return hipGetLastError();
}

int tile_bm() { return kBM; }
int tile_bn() { return kBN; }
int tile_waves() { return kWaves; }

int lds_bytes(int in_dtype, int d) {
  const bool fp8 = in_dtype == 3;
  const int kin = fp8 ? 1 : 2;
  return 2 * (kBN * d * kin + kBN * d * 2);
}

hipError_t launch_fwd(const FwdParams& p, int in_dtype, int d, hipStream_t stream) {
  // in_dtype: 1 = f16, 2 = bf16, 3 = fp8 e4m3 (validated by the caller)
  if (in_dtype == 1 && d == 64) return launch_t<In::F16, 64>(p, stream);
  if (in_dtype == 1 && d == 128) return launch_t<In::F16, 128>(p, stream);
  if (in_dtype == 2 && d == 64) return launch_t<In::BF16, 64>(p, stream);
  if (in_dtype == 2 && d == 128) return launch_t<In::BF16, 128>(p, stream);
  if (in_dtype == 3 && d == 128) return launch_t<In::FP8, 128>(p, stream);
  return hipErrorInvalidValue;
}

const char* kernel_name(int in_dtype, int d) {
  switch (in_dtype * 1000 + d) {
    case 1064: return "attn_fwd<f16,d64,bm128,bn64>";
    case 1128: return "attn_fwd<f16,d128,bm128,bn64>";
    case 2064: return "attn_fwd<bf16,d64,bm128,bn64>";
    case 2128: return "attn_fwd<bf16,d128,bm128,bn64>";
    case 3128: return "attn_fwd<fp8,d128,bm128,bn64>";
    default: return "none";
  }
}

}  // namespace ea
