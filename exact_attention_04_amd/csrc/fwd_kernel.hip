// Exact attention forward for gfx950 (CDNA4): fused Q.K^T -> online softmax
// -> P.V, one workgroup per (batch, head, query tile).
//
// Method: "FlashAttention" (aiunderstanding.org), section "Teknisk insikt".
// Each workgroup keeps its query rows' partial output, row maximum and row
// sum on chip while it walks over the key/value blocks, so scores and
// probabilities exist only in registers, one block at a time; HBM sees Q, K
// and V read and O and the log-sum-exp written, nothing of size N x N.
//
// How it maps onto a CDNA4 compute unit:
//   * A workgroup is 4 waves; each wave owns RB blocks of 32 query rows
//     (RB = 1: 128 rows per workgroup, two waves per SIMD; RB = 2: 256 rows,
//     one wave per SIMD).  K/V tiles of 64 keys are staged in LDS, double
//     buffered, by direct global-to-LDS loads.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16} (fp8:
//     v_mfma_scale_f32_32x32x64_f8f6f4).  K (A operand) comes from LDS and
//     each K fragment feeds every row block; Q^T (B operand) stays in
//     registers.  In the 32x32 accumulator lane l holds column l%32 -- one
//     query row -- and 16 of 32 keys; lane l^32 holds the other 16, so a row
//     max needs one exchange between wave halves and the row sum none until
//     the epilogue.
//   * P^T leaves the accumulator in the B-operand layout of O^T += V^T P^T
//     (after a 16-bit conversion), so P never touches LDS; V^T fragments come
//     from LDS with ds_read_b64_tr_b16 and feed every row block.  With fp8
//     inputs, P is bf16 and V is widened to bf16 on its way into LDS; or
//     (P8) both stay e4m3 and one v_mfma_scale_f32_32x32x64_f8f6f4 covers a
//     whole 64-key tile, V^T coming from ds_read_b64_tr_b8.
//   * Issue is in order per wave, so matrix and vector work overlap only if
//     they are interleaved in program order: a 64-key tile is processed as
//     two 32-key halves a, b with
//        S_a | max_a | S_b MFMAs interleaved with exp(S_a) |
//        max_b | P_a.V MFMAs interleaved with exp(S_b) | P_b.V
//   * LDS rows are XOR-swizzled in 16-byte units so the K reads (32 rows, one
//     column) and the transposing V reads (4 rows x 64 bytes) are free of
//     bank conflicts.
//   * Softmax reference: each row's reference max is fixed at the first block
//     where it sees a key, so O and l are never rescaled inside the loop.
//     p = exp2((s - m_ref) c) may exceed 1 by a bounded factor; a row whose
//     scores climb past that bound makes the workgroup repeat its key loop
//     with the exact row maximum (rare: scores would have to grow by more
//     than 2^15 / 2^64 in the exp2 domain after the first block).
//   * Only tiles that cross the causal diagonal, a window edge or the end of
//     the sequence evaluate the mask; tiles outside the visible range are
//     never loaded.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fwd_kernel.h"
#include "kernel_common.h"

namespace ea {

// V16: fp8 inputs whose V arrives already widened to bf16 (FwdParams::v_wide).
template <In IN, int D, int WAVES, int RB, bool P8, int KS, bool V16>
struct Cfg {
  static constexpr bool kFp8 = (IN == In::FP8);
  static_assert(!P8 || (kFp8 && D == 128), "e4m3 P.V: fp8 inputs, d = 128");
  static_assert(KS == 1 || !kFp8, "key streams: 16-bit inputs");
  static_assert(!V16 || (kFp8 && !P8), "a widened V copy: fp8 inputs, bf16 P.V");
  static constexpr int kThreads = 64 * WAVES;                 // one key stream's threads
  static constexpr int kBM = 32 * RB * WAVES;        // query rows per workgroup
  static constexpr int kInBytes = kFp8 ? 1 : 2;
  static constexpr int kKRow = D * kInBytes;         // bytes per K row in LDS
  static constexpr int kVRow = P8 ? D : D * 2;       // V in LDS: e4m3 for P8, else 16-bit
  static constexpr bool kVWiden = kFp8 && !P8 && !V16;   // fp8 V widened to bf16 through registers
  static constexpr int kVInBytes = V16 ? 2 : kInBytes;   // bytes per V element in global memory
  static constexpr int kKTile = kBN * kKRow;
  static constexpr int kVTile = kBN * kVRow;
  static constexpr int kStage = kKTile + kVTile;
  // widened fp8 V: 16-byte global chunks per thread per tile (register staged)
  static constexpr int kVPer = kBN * D * kInBytes / 16 / kThreads;
  static_assert(kVWiden ? (kBN * D * kInBytes / 16) % kThreads == 0 : true, "tile split");
  static_assert(kKTile % (1024 * WAVES) == 0 && kVTile % (1024 * WAVES) == 0, "DMA split");
  static constexpr int kQSteps = kFp8 ? D / 64 : D / 16;   // MFMA k-steps for S (per row block)
  static constexpr int kDBlocks = D / 32;                  // 32-wide output column blocks
};

// LDS layout of an e4m3 V tile (64 rows of 128 bytes, 8 units of 16 bytes):
// unit u of row r at unit u ^ v8_swz(r).  A transposing 8-bit read
// (ds_read_b64_tr_b8) gathers, per 16-lane group, one unit of 8 rows
// {b, b+1, b+2, b+3, b+8, ..., b+11} with b % 16 in {0, 4}; this swizzle puts
// those 8 units at 8 distinct positions, so the read is free of bank
// conflicts.
__device__ __forceinline__ int v8_swz(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }

// Waves per SIMD: two for 32 rows per wave (256 registers each), one for 64
// rows per wave or for four key streams (whose LDS holds one workgroup per CU).
template <int RB, int KS>
constexpr int kWavesPerEu = (RB == 2 || KS >= 4) ? 1 : 2;

template <In IN, int D, int WAVES, int RB, bool P8, int KS, bool V16>
__global__ void __launch_bounds__(64 * WAVES * KS)
    __attribute__((amdgpu_waves_per_eu(kWavesPerEu<RB, KS>, kWavesPerEu<RB, KS>)))
attn_fwd_kernel(const FwdParams p) {
  using C = Cfg<IN, D, WAVES, RB, P8, KS, V16>;
  constexpr In PIN = (IN == In::F16) ? In::F16 : In::BF16;   // type of P, V in LDS and O
  constexpr int kBM = C::kBM;
  // LDS: two K slots and two V slots.  K of tile i+1 and V of tile i are
  // read in the same iteration (the S MFMAs run one tile ahead of P.V), so
  // the two rings are offset by one tile.  The loop is unrolled by two so that
  // every slot is named at compile time (immediate offsets in the LDS
  // instructions).  The slots are separate objects so that the compiler can
  // tell the DMA into one slot from the reads of another: in a single array
  // it cannot, and it then waits for the DMA just issued before the first
  // read, which serialises the prefetch with the compute.
  //
  // Key streams (KS > 1): the workgroup's waves form KS groups of WAVES waves,
  // each covering all of the workgroup's query rows over every KS-th key tile
  // with slots of its own; at the end the streams' partial results (row
  // maximum, row sum, O) are merged through LDS.  This fills the GPU when the
  // query tiles alone are too few (short sequences, few heads).
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf0_s[KS][C::kKTile];
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf1_s[KS][C::kKTile];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf0_s[KS][C::kVTile];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf1_s[KS][C::kVTile];

  const int tid_all = threadIdx.x;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid_all >> 6);   // wave-uniform, kept in an SGPR
  const int stream = KS == 1 ? 0 : wave_all / WAVES;                   // this wave's key stream
  const int wave = wave_all - stream * WAVES;                           // its row block within the stream
  const int tid = tid_all - stream * C::kThreads;                       // thread index within the stream
  unsigned char* const kbuf0 = kbuf0_s[stream];
  unsigned char* const kbuf1 = kbuf1_s[stream];
  unsigned char* const vbuf0 = vbuf0_s[stream];
  unsigned char* const vbuf1 = vbuf1_s[stream];
  static_assert(KS == 1 || RB == 1, "key streams: one row block per wave (O fits a slot)");
  // per stream, row block and row: the row's maximum and sum, for the merge
  __shared__ float merge_ml[KS][WAVES][RB][2][32];
  const int lane = tid & 63;
  const int half = lane >> 5;      // which 16 of each 32 keys this lane holds
  const int col = lane & 31;       // the query row (within each row block) this lane owns

  // ---- work assignment: heaviest query tiles first (causal tiles near the
  // end of the sequence see the most keys).  Workgroups go to the 8 XCDs
  // round robin (workgroup w on XCD w % 8), each with its own L2.  Each XCD
  // runs a few K/V heads' work at a time (all their query tiles, heaviest
  // first, then the next few), so its resident workgroups share those heads'
  // K/V in its L2: four heads without shared K/V heads, the query heads of
  // two K/V heads (one if the K/V head count only splits into eights) with
  // them.  Where the heads do not split evenly over the XCDs, all heads of
  // one tile index run together (with shared K/V heads, the (batch, head)
  // order permuted to put each whole group on one XCD).
  // With the keys split (p.splits > 1: too few query tiles to fill the GPU),
  // workgroup item = (query tile, batch and head, key chunk), the chunk index
  // varying fastest.
  const int bh_count = p.batch * p.heads;
  const int chunk = (int)(blockIdx.x % p.splits);
  const int item = (int)(blockIdx.x / p.splits);
  int tile = p.q_tiles - 1 - item / bh_count;
  int bh = item % bh_count;
  const int bhk_count = bh_count / p.group;
  if (p.group > 1 && p.splits == 1 && bhk_count % 8 == 0) {
    // units of a K/V head: (tile, query head of its group), the tile slowest
    const int2 wo = xcd_grouped(item, p.q_tiles * p.group, bhk_count % 16 == 0 ? 2 : 1);
    tile = p.q_tiles - 1 - wo.x / p.group;
    bh = wo.y * p.group + wo.x % p.group;
  } else if (p.group > 1 && bh_count % (8 * p.group) == 0) {
    const int x = bh & 7, y = bh >> 3;
    bh = ((y / p.group) * 8 + x) * p.group + y % p.group;
  } else if (p.group == 1 && p.splits == 1 && bh_count % 32 == 0) {
    const int2 wo = xcd_grouped(item, p.q_tiles, 4);
    tile = p.q_tiles - 1 - wo.x;
    bh = wo.y;
  }
  const int b = bh / p.heads;
  const int h = bh - b * p.heads;
  const int hkv = h / p.group;      // the K/V head this query head reads
  const int q0 = tile * kBM;
  const int n = p.n;

  const unsigned char* qg = (const unsigned char*)p.q + ((int64_t)b * p.q_sb + (int64_t)h * p.q_sh) * C::kInBytes;
  const unsigned char* kg = (const unsigned char*)p.k + ((int64_t)b * p.k_sb + (int64_t)hkv * p.k_sh) * C::kInBytes;
  const unsigned char* vg = (const unsigned char*)p.v + ((int64_t)b * p.v_sb + (int64_t)hkv * p.v_sh) * C::kVInBytes;
  const int k_row_stride = (int)(p.k_ss * C::kInBytes);   // bytes; < 2^31 (checked by the host)
  const int v_row_stride = (int)(p.v_ss * C::kVInBytes);

  const KeyRange kr = tile_key_range(q0, kBM, n, p.causal, p.wl, p.wr);
  // this workgroup's key tiles: chunk `chunk` of p.splits contiguous chunks
  // of the tile's visible key tiles (an empty chunk leaves l = 0)
  const int kt_first = kr.lo / kBN;
  const int kt_count = (kr.hi + kBN - 1) / kBN - kt_first;
  const int kt_begin = kt_first + (int)((int64_t)kt_count * chunk / p.splits);
  const int kt_end = kt_first + (int)((int64_t)kt_count * (chunk + 1) / p.splits);
  // This stream's key tiles: kt_begin + stream + KS i for i < iters.  Every
  // stream runs `iters` iterations, so that each wave meets each barrier; only
  // a stream's last tile can lie past kt_end, and that one is loaded as zeros
  // and not computed.
  const int iters = (kt_end - kt_begin + KS - 1) / KS;
  const int kt_first_s = kt_begin + stream;

  // ---- this wave's rows: RB blocks of 32, lane `col` owns one row in each
  const int wr0 = q0 + wave * 32 * RB;     // first row of the wave
  const int wr1 = min(wr0 + 32 * RB, n);   // one past its last real row
  int qrow[RB];
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) qrow[qb] = wr0 + 32 * qb + col;

  // ---- Q^T fragments (B operand), kept in registers for the whole kernel.
  uint4 qf[RB][C::kFp8 ? 2 * C::kQSteps : C::kQSteps];
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) {
    const bool ok = qrow[qb] < n;
    const unsigned char* src = qg + (int64_t)(ok ? qrow[qb] : 0) * p.q_ss * C::kInBytes;
    if constexpr (C::kFp8) {
#pragma unroll
      for (int st = 0; st < C::kQSteps; ++st) {
        // lane holds d = 64 st + 32 half + [0, 32): two 16-byte pieces
        const uint4* g = (const uint4*)(src + 64 * st + 32 * half);
        qf[qb][2 * st] = ok ? g[0] : make_uint4(0, 0, 0, 0);
        qf[qb][2 * st + 1] = ok ? g[1] : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int st = 0; st < C::kQSteps; ++st) {
        // lane holds d = 16 st + 8 half + [0, 8)
        qf[qb][st] = ok ? *(const uint4*)(src + (16 * st + 8 * half) * 2) : make_uint4(0, 0, 0, 0);
      }
    }
  }

  // ---- staging of K and V tiles into LDS (swizzled layout).
  // 16-bit K and V, and fp8 K, go straight from global memory to LDS
  // (buffer_load_dwordx4 ... lds): one wave instruction fills 1 KB of LDS,
  // lane L writing 16-byte unit L of it, so each lane fetches the global unit
  // that the swizzle maps to that LDS position.  Each tile is addressed
  // through a buffer resource whose range ends with the sequence's last key:
  // rows past the end are written as zeros (K: masked; V: met by p = 0), so
  // the last tile needs no special path and the slots need no clearing.  A
  // resource of range 0 (a tile past the visible range) makes the load write
  // zeros, into a slot that is then never read.
  // fp8 V for the bf16 P.V goes through registers and is widened to bf16 on
  // the way into LDS; for the e4m3 P.V it goes straight in, in its own
  // swizzle (v8_swz).
  constexpr int kKBlocks = C::kKTile / 1024 / WAVES;     // DMA instructions per wave, K
  constexpr int kVBlocks = C::kVWiden ? 0 : C::kVTile / 1024 / WAVES;
  constexpr int kVB = kVBlocks > 0 ? kVBlocks : 1;
  // Tile row and byte column of the unit lane `ln` fetches in DMA block `blk`.
  auto dma_row = [](int blk, int row_bytes, int ln) { return (blk * 64 + ln) / (row_bytes / 16); };
  auto dma_col = [](int blk, int row_bytes, int ln) {
    const int pos = blk * 64 + ln;
    const int row = pos / (row_bytes / 16);
    const int phys = pos % (row_bytes / 16);
    return (row_bytes == 256 ? swizzled_unit<256>(row, phys) : swizzled_unit<128>(row, phys)) * 16;
  };
  // Byte offset, from the tile's first key, of the unit this lane fetches in
  // each of its DMA blocks (< 2^31: the host bounds 64 rows of stride).
  uint32_t k_off[kKBlocks], v_off[kVB];
#pragma unroll
  for (int i = 0; i < kKBlocks; ++i) {
    const int blk = wave * kKBlocks + i;
    k_off[i] = (uint32_t)(dma_row(blk, C::kKRow, lane) * k_row_stride + dma_col(blk, C::kKRow, lane));
  }
#pragma unroll
  for (int i = 0; i < kVB; ++i) {
    const int blk = wave * kVBlocks + i;
    if constexpr (P8) {
      const int row = dma_row(blk, C::kVRow, lane);
      const int phys = (blk * 64 + lane) % (C::kVRow / 16);
      v_off[i] = (uint32_t)(row * v_row_stride + (phys ^ v8_swz(row)) * 16);
    } else {
      v_off[i] = kVBlocks > 0 ? (uint32_t)(dma_row(blk, C::kVRow, lane) * v_row_stride + dma_col(blk, C::kVRow, lane))
                              : 0u;
    }
  }
  // Buffer range of tile kt of a K or V head: the tile's first key and the
  // bytes up to the end of its last key (the sequence's last key in the last
  // tile; 0 if kt >= kt_end).  The resource is built at each load from these
  // plain values; the compiler shares the scalar work between the loads of a
  // tile.  A whole tile's and the last tile's byte counts are fixed per
  // launch, so a tile costs a select and one 32 x 32 -> 64-bit product (the
  // host bounds 64 rows of stride below 2^31).
  struct TileRange {
    const unsigned char* base;
    int bytes;
  };
  const int kt_last = (n - 1) / kBN;
  const int last_rows = n - kt_last * kBN;
  const int k_full = (kBN - 1) * k_row_stride + C::kKRow, k_tail = (last_rows - 1) * k_row_stride + C::kKRow;
  const int v_full = (kBN - 1) * v_row_stride + D * C::kVInBytes;
  const int v_tail = (last_rows - 1) * v_row_stride + D * C::kVInBytes;
  const uint32_t k_tstride = (uint32_t)(kBN * k_row_stride), v_tstride = (uint32_t)(kBN * v_row_stride);
  auto tile_range = [&](const unsigned char* head, uint32_t tstride, int full, int tail, int kt) {
    const int bytes = kt >= kt_end ? 0 : (kt < kt_last ? full : tail);
    return TileRange{head + (uint64_t)(uint32_t)kt * tstride, bytes};
  };
  uint4 vreg[C::kVWiden ? C::kVPer : 1];
  // One load of a tile: K block i, or V item i.
  constexpr int kDmaK = kKBlocks;
  constexpr int kDmaV = C::kVWiden ? C::kVPer : kVBlocks;
  auto load_k = [&](TileRange t, unsigned char* dst, int i) {
    load_16b_to_lds(t.base, t.bytes, k_off[i], dst + (wave * kKBlocks + i) * 1024);
  };
  auto load_v = [&](TileRange t, unsigned char* dst, int i) {
    if constexpr (C::kVWiden) {
      const int id = tid + i * C::kThreads;
      vreg[i] = load_16b(t.base, t.bytes, (uint32_t)((id / (D / 16)) * v_row_stride + (id % (D / 16)) * 16));
    } else {
      load_16b_to_lds(t.base, t.bytes, v_off[i], dst + (wave * kVBlocks + i) * 1024);
    }
  };
  auto k_range = [&](int kt) { return tile_range(kg, k_tstride, k_full, k_tail, kt); };
  auto v_range = [&](int kt) { return tile_range(vg, v_tstride, v_full, v_tail, kt); };
  auto issue_k = [&](int kt, unsigned char* dst) {
    const TileRange t = k_range(kt);
#pragma unroll
    for (int i = 0; i < kDmaK; ++i) load_k(t, dst, i);
  };
  auto issue_v = [&](int kt, unsigned char* dst) {
    const TileRange t = v_range(kt);
#pragma unroll
    for (int i = 0; i < kDmaV; ++i) load_v(t, dst, i);
  };
  // widened fp8 V only: widen the V tile held in registers and store it
  // (bf16) to LDS.
  auto store_v_fp8 = [&](unsigned char* vl) {
    if constexpr (C::kVWiden) {
#pragma unroll
      for (int i = 0; i < C::kVPer; ++i) {
        const int id = tid + i * C::kThreads;
        const int row = id / (D / 16);           // 16 fp8 per global chunk
        const int unit = (id % (D / 16)) * 2;    // two 16-byte bf16 units
        uint4 lo, hi;
        fp8x16_to_bf16(vreg[i], lo, hi);
        *(uint4*)(vl + lds_offset<C::kVRow>(row, unit)) = lo;
        *(uint4*)(vl + lds_offset<C::kVRow>(row, unit + 1)) = hi;
      }
    }
  };
  // ---- running state, per row block
  f32x16 acc[RB][C::kDBlocks];
#pragma unroll
  for (int qb = 0; qb < RB; ++qb)
#pragma unroll
    for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][c][r] = 0.f;
  // e4m3 P (P8) carries p * 2^kPShift: values up to 2^kPShift at the row
  // reference stay clear of e4m3's top (448), values down to 2^-(6 + kPShift)
  // stay normal.  O and l carry the same factor, so only the LSE removes it.
  constexpr float kPShift = P8 ? 3.f : 0.f;
  float m_run[RB], neg_mc[RB], l_part[RB];
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) {
    m_run[qb] = -INFINITY;   // reference max of the raw (unscaled) scores
    neg_mc[qb] = 0.f;        // -m_run * c (+ kPShift), or 0 while no key was seen
    l_part[qb] = 0.f;        // this lane's share of the row sum
  }
  const float cexp = p.c_log2;                 // softmax scale * log2(e) (* fp8 descales)
  // Keys visible from each of this lane's rows form one interval [vis_lo, vis_hi].
  int vis_lo[RB];
  uint32_t vis_span[RB];
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) {
    const int qi = qrow[qb];
    vis_lo[qb] = p.wl >= 0 ? qi - p.wl : 0;
    int hi = n - 1;
    if (p.causal) hi = min(hi, qi);
    if (p.wr >= 0) hi = min(hi, qi + p.wr);
    vis_span[qb] = (uint32_t)(hi - vis_lo[qb]);
  }

  // This lane's transposing-read offsets within a V tile (see pv_half).
  uint32_t va[2][C::kDBlocks];
  if constexpr (!P8) {
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int r8 = 0; r8 < 2; ++r8)
#pragma unroll
      for (int c = 0; c < C::kDBlocks; ++c) {
        const int vrow = 4 * (g >> 1) + (sl >> 2) + 8 * r8;
        const int dcol = 32 * c + 16 * (g & 1) + 4 * (sl & 3);
        va[r8][c] = (uint32_t)(lds_offset<C::kVRow>(vrow, dcol >> 3) + (dcol & 7) * 2);
        asm volatile("" : "+v"(va[r8][c]));
      }
  }
  // e4m3 V (P8): this lane's offset, within a V tile, of its 8-bit
  // transposing read for keys 8 (j/4) + 4 (g/2) + j%4, j = sl/2 (source lane
  // sl of 16-lane group g reads 8 bytes of one such key row: columns
  // 32 c + 16 (g%2) + 8 (sl%2) ..+7); the reads for keys 16 rr + those add
  // 2048 rr bytes (16 rows; the swizzle depends on row bits 0, 1, 3 only).
  uint32_t va8[P8 ? C::kDBlocks : 1];
  if constexpr (P8) {
    const int g = lane >> 4, sl = lane & 15;
    const int j = sl >> 1;
    const int row = 8 * (j >> 2) + 4 * (g >> 1) + (j & 3);
#pragma unroll
    for (int c = 0; c < C::kDBlocks; ++c) {
      const int unit = 2 * c + (g & 1);
      va8[c] = (uint32_t)(row * C::kVRow + ((unit ^ v8_swz(row)) << 4) + 8 * (sl & 1));
      asm volatile("" : "+v"(va8[c]));
    }
  }

  // This lane's K-fragment read offsets within a K tile, for k-step st of the
  // first 32 keys (the second 32 keys add a constant).
  uint32_t ka[C::kQSteps];
#pragma unroll
  for (int st = 0; st < C::kQSteps; ++st) {
    ka[st] = C::kFp8 ? 0u : (uint32_t)lds_offset<C::kKRow>(col, 2 * st + half);
    asm volatile("" : "+v"(ka[st]));
  }

  // ---- building blocks over 32-key halves of a staged tile ----------------
  // S^T for keys [32 hb, 32 hb + 32) of the K tile at `kl`, for every row
  // block (each K fragment feeds RB MFMAs).
  auto s_half = [&](const unsigned char* kl, int hb, f32x16 (&s)[RB], auto&& hook) {
#pragma unroll
    for (int qb = 0; qb < RB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[qb][r] = 0.f;
    const int krow = 32 * hb + col;
    if constexpr (C::kFp8) {
      uint4 a[2 * C::kQSteps];
#pragma unroll
      for (int st = 0; st < C::kQSteps; ++st) {
        const int u0 = (64 * st + 32 * half) / 16;
        a[2 * st] = *(const uint4*)(kl + lds_offset<C::kKRow>(krow, u0));
        a[2 * st + 1] = *(const uint4*)(kl + lds_offset<C::kKRow>(krow, u0 + 1));
      }
#pragma unroll
      for (int st = 0; st < C::kQSteps; ++st) {
#pragma unroll
        for (int qb = 0; qb < RB; ++qb) s[qb] = mfma_fp8(a[2 * st], a[2 * st + 1], qf[qb][2 * st], qf[qb][2 * st + 1], s[qb]);
        hook(st);
      }
    } else {
      // K fragment reads are issued in groups ahead of their MFMAs, so their
      // latency is paid once per group rather than per MFMA
      constexpr int kGroup = 4;
#pragma unroll
      for (int st0 = 0; st0 < C::kQSteps; st0 += kGroup) {
        uint4 a[kGroup];
#pragma unroll
        for (int j = 0; j < kGroup; ++j) a[j] = *(const uint4*)(kl + lds_offset<C::kKRow>(krow, 2 * (st0 + j) + half));
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
#pragma unroll
          for (int qb = 0; qb < RB; ++qb) s[qb] = mfma_16bit<IN>(a[j], qf[qb][st0 + j], s[qb]);
          hook(st0 + j);
        }
      }
    }
  };
  auto block_max = [](const f32x16& x) {
    float m = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) m = fmaxf(m, x[r]);
    return m;
  };
  // Reference max.  A row's reference is fixed at the first block where it
  // sees a key (O and l are still zero then, so nothing needs rescaling) and
  // never moves afterwards: later p may exceed 1, which the 16-bit P format
  // and the fp32 sums hold with unchanged relative precision.  Only a p
  // beyond the P format's range (2^16 in fp16, 2^128 in bf16) or an fp32
  // overflow goes wrong, and it does so visibly: it leaves inf or NaN in l or
  // O, which the epilogue checks; the workgroup then repeats the key loop with
  // the exact row maximum as reference.  Block maxima are therefore computed
  // only while some row of the wave has no reference yet (the first visible
  // tile of each row).
  auto wave_needs_ref = [&]() {
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) any = any || (m_run[qb] == -INFINITY);
    return __builtin_amdgcn_ballot_w64(any) != 0;
  };
  auto fold_max = [&](const f32x16 (&sa)[RB], const f32x16 (&sb)[RB]) {
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) {
      if (m_run[qb] == -INFINITY) {
        const float m = pair_max(fmaxf(block_max(sa[qb]), block_max(sb[qb])));
        m_run[qb] = m;
        neg_mc[qb] = (m == -INFINITY) ? 0.f : -m * cexp + kPShift;
      }
    }
  };
  // p = exp2(x), x = s c - m c, for a 32-key half of every row block, packed
  // to 16 bits; the row sum takes the unrounded fp32 p (the LSE needs it to
  // fp32 accuracy, which a sum of 16-bit p would miss by up to 2^-9).
  auto exp_pack = [&](const f32x16 (&s)[RB], uint32_t (&pk)[RB][8]) {
#pragma unroll
    for (int qb = 0; qb < RB; ++qb)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float x0 = __builtin_fmaf(s[qb][2 * r], cexp, neg_mc[qb]);
        const float x1 = __builtin_fmaf(s[qb][2 * r + 1], cexp, neg_mc[qb]);
        const float e0 = __builtin_amdgcn_exp2f(x0);
        const float e1 = __builtin_amdgcn_exp2f(x1);
        l_part[qb] += e0;
        l_part[qb] += e1;
        pk[qb][r] = pack2<PIN>(e0, e1);
      }
  };
  // The 16-bit rounding residual p - round16(p) of k-step j (keys
  // 16 j .. 16 j + 15 of a half packed by exp_pack, with the same reference),
  // itself packed to 16 bits.
  auto residual = [&](const f32x16 (&s)[RB], const uint32_t (&pk)[RB][8], int j, uint32_t (&pr)[RB][4]) {
#pragma unroll
    for (int qb = 0; qb < RB; ++qb)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 4 * j + t;
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][2 * r], cexp, neg_mc[qb]));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][2 * r + 1], cexp, neg_mc[qb]));
        pr[qb][t] = pack2<PIN>(e0 - unpack_lo<PIN>(pk[qb][r]), e1 - unpack_hi<PIN>(pk[qb][r]));
      }
  };
  // e4m3 P (P8): p * 2^kPShift for a 32-key half, rounded to nearest e4m3
  // and packed four to a dword in accumulator order (byte t of dword w holds
  // register 4 w + t); the row sum takes the unrounded fp32 values.  A value
  // at or past 480 becomes NaN, which the epilogue's check turns into the
  // exact-maximum pass.
  auto exp_pack8 = [&](const f32x16 (&s)[RB], uint32_t (&pk)[RB][4]) {
#pragma unroll
    for (int qb = 0; qb < RB; ++qb)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float e[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          e[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][4 * w + t], cexp, neg_mc[qb]));
          l_part[qb] += e[t];
        }
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], x, true);
        pk[qb][w] = (uint32_t)x;
      }
  };
  // Its rounding residual times 16, p 2^(kPShift+4) - 16 e4m3(p 2^kPShift),
  // itself rounded to e4m3 (the P.V of the residual takes the 2^-4 back
  // through the matrix instruction's B scale): hi + lo / 16 carries p to
  // about 2^-8 relative.
  auto residual8 = [&](const f32x16 (&s)[RB], const uint32_t (&pk)[RB][4], uint32_t (&pr)[RB][4]) {
#pragma unroll
    for (int qb = 0; qb < RB; ++qb)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pk[qb][w], false);
        const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pk[qb][w], true);
        const float hi[4] = {h01[0], h01[1], h23[0], h23[1]};
        float lo[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float e16 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][4 * w + t], cexp, neg_mc[qb] + 4.f));
          lo[t] = __builtin_fmaf(hi[t], -16.f, e16);
        }
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(lo[0], lo[1], 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(lo[2], lo[3], x, true);
        pr[qb][w] = (uint32_t)x;
      }
  };
  // O^T += V^T P^T over a whole 64-key tile on the e4m3 matrix instruction
  // (32x32x64).  P^T (B operand): lane l holds query l%32 and 32 keys, its 16
  // of half a (bytes 0-15, `pa`) then its 16 of half b (`pb`), i.e. keys
  // 32 (t/16) + 8 ((t%16)/4) + 4 (l/32) + t%4 for byte t.  The V^T fragment
  // (A operand: row d = l%32 of a 32-column block, the same 32 keys) takes
  // four transposing 8-bit reads (see va8), 8 keys each; each fragment feeds
  // every row block.  `scale_b`: the B operand's power-of-two scale (E8M0,
  // 127 = 1).
  auto pv8 = [&](const uint32_t (&pa)[RB][4], const uint32_t (&pb)[RB][4], const unsigned char* vl, int scale_b) {
#pragma unroll
    for (int c = 0; c < C::kDBlocks; ++c) {
      uint2 r[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        r[rr] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vl + va8[c] + 2048 * rr)));
      const uint4 a0 = make_uint4(r[0].x, r[0].y, r[1].x, r[1].y);
      const uint4 a1 = make_uint4(r[2].x, r[2].y, r[3].x, r[3].y);
#pragma unroll
      for (int qb = 0; qb < RB; ++qb)
        acc[qb][c] = mfma_fp8_scaled(a0, a1, make_uint4(pa[qb][0], pa[qb][1], pa[qb][2], pa[qb][3]),
                                     make_uint4(pb[qb][0], pb[qb][1], pb[qb][2], pb[qb][3]), acc[qb][c], scale_b);
    }
  };
  // S MFMAs of one half (K tile at `kn`) interleaved, step by step in program
  // order, with the softmax of the current half `sc`: step st issues the
  // MFMA of k-step st, the read of a K fragment kPre steps ahead, the
  // loads `hook(st)` and the exp / sum / pack of 1 / kQSteps of the scores.
  // Each step is fenced (sched_barrier), so the compiler keeps this order
  // instead of grouping the MFMAs and the vector work apart (16-bit inputs).
  auto s_phase = [&](const unsigned char* kn, int hb, f32x16 (&sn)[RB], const f32x16 (&sc)[RB],
                     uint32_t (&pk)[RB][8], auto&& hook) {
    constexpr int kSteps = C::kQSteps;
    constexpr int kPre = kSteps < 4 ? kSteps : 4;      // K reads in flight
    constexpr int kPairsPerStep = 8 / kSteps;          // packed P pairs per step
#pragma unroll
    for (int qb = 0; qb < RB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[qb][r] = 0.f;
    const unsigned char* kb = kn + 32 * hb * C::kKRow;
    uint4 a[kSteps];
#pragma unroll
    for (int st = 0; st < kPre; ++st) a[st] = *(const uint4*)(kb + ka[st]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      if (st + kPre < kSteps) a[st + kPre] = *(const uint4*)(kb + ka[st + kPre]);
      auto softmax_slice = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < RB; ++qb)
#pragma unroll
          for (int u = 0; u < kPairsPerStep; ++u) {
            const int r = st * kPairsPerStep + u;
            const float x0 = __builtin_fmaf(sc[qb][2 * r], cexp, neg_mc[qb]);
            const float x1 = __builtin_fmaf(sc[qb][2 * r + 1], cexp, neg_mc[qb]);
            const float e0 = __builtin_amdgcn_exp2f(x0);
            const float e1 = __builtin_amdgcn_exp2f(x1);
            l_part[qb] += e0;
            l_part[qb] += e1;
            pk[qb][r] = pack2<PIN>(e0, e1);
          }
      };
      // d = 64 (four steps, two pairs each): the step's softmax slice goes
      // first, so the K fragment read has that long to land before its MFMA;
      // at d = 128 the MFMA goes first (measured faster there)
      if constexpr (D == 64) {
        softmax_slice();
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int qb = 0; qb < RB; ++qb) sn[qb] = mfma_16bit<IN>(a[st], qf[qb][st], sn[qb]);
      hook(st);
      if constexpr (D != 64) softmax_slice();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Mask a 32-key half: key k0 + 32 hb + 8 (r/4) + 4 half + (r%4).
  auto apply_mask = [&](f32x16 (&s)[RB], int k0, int hb) {
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) {
      const int base = k0 + 32 * hb + 4 * half - vis_lo[qb];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t rel = (uint32_t)(base + 8 * (r >> 2) + (r & 3));
        if (rel > vis_span[qb]) s[qb][r] = -INFINITY;
      }
    }
  };
  // Tiles crossing a mask edge or the sequence end, for this wave's rows.
  // Each visibility condition is monotone in the tile index, so the tiles
  // every (row, key) pair of which is visible form one interval [t_lo, t_lo
  // + t_span): a tile is masked iff it lies outside.
  int t_hi_key = n - kBN;                                 // last key tile start fully inside the sequence
  if (p.causal) t_hi_key = min(t_hi_key, wr0 - (kBN - 1));
  if (p.wr >= 0) t_hi_key = min(t_hi_key, wr0 + p.wr - (kBN - 1));
  const int t_hi = t_hi_key < 0 ? 0 : t_hi_key / kBN + 1;
  const int t_lo_key = p.wl >= 0 ? (wr1 - 1) - p.wl : 0;  // first key tile start past the left edge
  const int t_lo = t_lo_key <= 0 ? 0 : (t_lo_key + kBN - 1) / kBN;
  const uint32_t t_span = (uint32_t)max(t_hi - t_lo, 0);
  auto tile_masked = [&](int kt) { return (uint32_t)(kt - t_lo) >= t_span; };
  // keys [k0, k0 + 32) of half hb of tile kt seen by none of the wave's rows
  auto half_dead = [&](int kt, int hb) {
    const int k0 = kt * kBN + 32 * hb;
    return k0 >= n || (p.causal && k0 > wr1 - 1) || (p.wr >= 0 && k0 > wr1 - 1 + p.wr) ||
           (p.wl >= 0 && k0 + 31 < wr0 - p.wl);
  };

  // ---- one 32-key half ("unit") of the software pipeline.  The softmax of
  // the current scores `sc` (tile kt, half hb) runs interleaved with the S
  // MFMAs of the same half of the next tile (`sn`, from the K slot `kn`),
  // then O += P V over the current V slot `vl`.  Issue is in order per wave,
  // so this interleave is what lets the vector ALU and the matrix core work
  // at the same time.
  // Rounding of P.  A 16-bit p carries a relative error of up to 2^-8 (bf16)
  // or 2^-11 (fp16).  Spread over many keys these errors average out; they do
  // not where a few keys hold a large share of a row's weight: a row's first
  // keys, or a peaked row whose dominant keys may sit anywhere in its range.
  // So a half holding a key whose p exceeds 1/kPeak of its row's running sum
  // (kPeak 8 for bf16 P, 4 for fp16) also multiplies the rounding residual
  // p - round16(p), itself in 16 bits: P is effectively 16+16 bits there.
  // Every other key carries less than 1/kPeak of its row's final weight,
  // which caps its own rounding error at 2^-11 |v| (bf16) or 2^-13 |v|
  // (fp16).  The test runs in two steps, both wave-uniform (ballots over the
  // wave's rows), after the main P.V MFMAs are issued:
  //  * a filter: a half whose sum of p over this lane's keys is at most
  //    1/kPeak of the lane's running sum holds no such key (each p is at most
  //    that sum, the lane's sum at most the row's); it costs a subtract, a
  //    multiply and a compare, and passes only a row's first halves and
  //    halves that add much weight;
  //  * for halves that pass it, the largest packed p of each lane (16-bit
  //    values of one sign compare as unsigned integers) against the row's
  //    running sum, with 2^-7 of slack for the rounding of the packed p, so
  //    it flags every half the exact p would.
  constexpr int kSMfma = RB * C::kQSteps;            // S MFMAs per half (all row blocks)
  constexpr int kExpValu = RB * 56;                  // softmax VALU per half (all row blocks)
  // `hook(st)` runs after the S MFMA of k-step st; the units of an iteration
  // use it to issue the loads of later tiles a few at a time, so they are
  // spread between the MFMAs rather than issued in one burst, which would
  // stall the waves that leave a barrier together on the address unit.
  // (The scheduler cannot move those loads past LDS reads by itself: they
  // write LDS.)
  auto unit = [&](auto next_tag, f32x16 (&sc)[RB], int hb, const unsigned char* vl, const unsigned char* kn,
                  f32x16 (&sn)[RB], auto&& hook) {
    uint32_t pk[RB][8];
    float l_before[RB];   // this lane's row sums before the half
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) l_before[qb] = l_part[qb];
    // d = 64: the half's V^T fragments are read before its S phase, so they
    // have landed when its P.V starts (four MFMAs are too few to hide them)
    constexpr bool kVAhead = D == 64 && !C::kFp8;
    uint4 vfr[2][kVAhead ? C::kDBlocks : 1];
    if constexpr (kVAhead) {
      pv_frags<D>(vfr[0], vl, va, hb, 0);
      pv_frags<D>(vfr[1], vl, va, hb, 1);
    }
    if constexpr (decltype(next_tag)::value) {
      // raised priority while the S MFMAs and the softmax interleave: when
      // both waves of a SIMD have work, the one feeding the matrix core from
      // this phase issues first
      __builtin_amdgcn_s_setprio(1);
      if constexpr (C::kFp8) {
        // fp8: the compiler moves the two 8-bit S products (first read after
        // the mask branch) below this half's P.V, so the phase is the softmax
        // alone and the P.V and S products follow back to back.  Holding them
        // in the phase (an empty asm use) measured 1.2% slower, and also
        // moving half a's P.V into half b's phase 6% slower (e4m3 P.V: 12%):
        // here the two waves of a SIMD overlap better phase against phase.
        s_half(kn, hb, sn, hook);
        exp_pack(sc, pk);
#pragma unroll
        for (int i = 0; i < kSMfma; ++i) {
          if (i % (4 * RB) == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::kQSteps, 0);  // K reads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  // S MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, kExpValu / kSMfma, 0);                  // softmax VALU
        }
      } else {
        s_phase(kn, hb, sn, sc, pk, hook);
      }
    } else {
      exp_pack(sc, pk);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    constexpr float kPeak = (PIN == In::F16) ? 4.f : 8.f;
    // pre-filter: the half's share of this lane's sum bounds each of its p
    bool pre = false;
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) pre = pre || (l_part[qb] - l_before[qb]) * kPeak > l_part[qb];
    if constexpr (kVAhead) {
      pv_kstep_with<PIN, D, RB>(acc, pk, vfr[0], 0);
      pv_kstep_with<PIN, D, RB>(acc, pk, vfr[1], 1);
    } else {
      pv_half<PIN, D, RB>(acc, pk, vl, va, hb);
    }
    if (__builtin_amdgcn_ballot_w64(pre) != 0) {
      bool peak = false;
#pragma unroll
      for (int qb = 0; qb < RB; ++qb) {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        u16x2 m = __builtin_bit_cast(u16x2, pk[qb][0]);
#pragma unroll
        for (int r = 1; r < 8; ++r) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, pk[qb][r]));
        const uint32_t mw = __builtin_bit_cast(uint32_t, m);
        const float pmax = fmaxf(unpack_lo<PIN>(mw), unpack_hi<PIN>(mw));
        peak = peak || pmax * (kPeak * 1.0078125f) > pair_sum(l_part[qb]);
      }
      if (__builtin_amdgcn_ballot_w64(peak) != 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t pr[RB][4];
          residual(sc, pk, j, pr);
          pv_kstep<PIN, D, RB>(acc, pr, vl, va, hb, j);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // e4m3 P.V (P8): a unit issues the S MFMAs of the next tile's same half
  // and computes the softmax of the current half (the compiler places the
  // softmax after the mask branch, as it moves the S products in `unit` for
  // fp8) and packs P to e4m3; the P.V of the tile follows both halves
  // (tile_pv8).
  auto unit8 = [&](auto next_tag, f32x16 (&sc)[RB], int hb, const unsigned char* kn, f32x16 (&sn)[RB],
                   uint32_t (&pk)[RB][4], auto&& hook) {
    if constexpr (decltype(next_tag)::value) {
      __builtin_amdgcn_s_setprio(1);
      s_half(kn, hb, sn, hook);
      exp_pack8(sc, pk);
#pragma unroll
      for (int i = 0; i < kSMfma; ++i) {
        if (i % (4 * RB) == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::kQSteps, 0);  // K reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  // S MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kExpValu / kSMfma, 0);                  // softmax VALU
      }
    } else {
      exp_pack8(sc, pk);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // The tile's P.V from the e4m3 P of both halves.  e4m3 keeps 3 mantissa
  // bits, so a tile whose rounding errors would not average out against the
  // rest of a row -- one that adds more than 1/8 of some row's sum so far
  // (the first tiles of every row, or a tile holding a row's dominant keys)
  // -- also runs the P.V of the rounding residual (residual8), which brings
  // P to about 2^-8 relative there.  `l_tile`: l_part before the tile.
  auto tile_pv8 = [&](const f32x16 (&sa)[RB], const f32x16 (&sb)[RB], const uint32_t (&pa)[RB][4],
                      const uint32_t (&pb)[RB][4], const float (&l_tile)[RB], const unsigned char* vl) {
    __builtin_amdgcn_s_setprio(0);
    bool heavy = false;
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) heavy = heavy || ((l_part[qb] - l_tile[qb]) * 8.f > l_part[qb]);
    if (__builtin_amdgcn_ballot_w64(heavy) != 0) {
      uint32_t ra[RB][4], rb[RB][4];
      residual8(sa, pa, ra);
      residual8(sb, pb, rb);
      pv8(ra, rb, vl, 127 - 4);
    }
    pv8(pa, pb, vl, 127);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- the key loop.  Iteration i (tile kt = kt_begin + i) starts with the
  // scores S(i) in registers, K(i+1) and V(i) in LDS; it issues the DMA of
  // K(i+2) and V(i+1) into the slots freed by the previous iteration, runs
  // the two units, and ends with a barrier once its DMA has landed.
  f32x16 s_a[RB], s_b[RB];
  // whether some row of the wave still has no reference (wave-uniform); once
  // every row has one, the per-tile test is skipped
  bool need_ref = true;
  auto ref_step = [&]() __attribute__((always_inline)) {
    if (need_ref) {
      if (wave_needs_ref()) fold_max(s_a, s_b);
      need_ref = wave_needs_ref();
    }
  };
  auto iter = [&](int kt, const unsigned char* kread, const unsigned char* vread, unsigned char* kwrite,
                  unsigned char* vwrite) __attribute__((always_inline)) {
    ref_step();
    const int kt_next = kt + KS;     // this stream's next tile
    const bool m_next = tile_masked(kt_next);
    f32x16 n_a[RB], n_b[RB];
    // K of the tile after next (zeros past the last tile) and V of the next,
    // into the slots the previous iteration freed: K spread over the S MFMAs
    // of the first unit, V over those of the second (fp8 V that is widened
    // through registers goes with K, so that it has landed when the
    // iteration's end converts and stores it)
    const TileRange rk = k_range(kt_next + KS), rv = v_range(kt_next);
    constexpr int kPerK = (kDmaK + C::kQSteps - 1) / C::kQSteps;
    constexpr int kPerV = (kDmaV + C::kQSteps - 1) / C::kQSteps;
    auto dma_hook = [&](int st) {
#pragma unroll
      for (int u = 0; u < kPerK; ++u) {
        const int i = st * kPerK + u;
        if (i < kDmaK) load_k(rk, kwrite, i);
      }
      if constexpr (C::kVWiden) {
#pragma unroll
        for (int u = 0; u < kPerV; ++u) {
          const int i = st * kPerV + u;
          if (i < kDmaV) load_v(rv, vwrite, i);
        }
      }
    };
    auto dma_hook_v = [&](int st) {
      if constexpr (!C::kVWiden) {
#pragma unroll
        for (int u = 0; u < kPerV; ++u) {
          const int i = st * kPerV + u;
          if (i < kDmaV) load_v(rv, vwrite, i);
        }
      }
    };
    if constexpr (P8) {
      float l_tile[RB];
#pragma unroll
      for (int qb = 0; qb < RB; ++qb) l_tile[qb] = l_part[qb];
      uint32_t pa[RB][4], pb[RB][4];
      unit8(BoolTag<true>{}, s_a, 0, kread, n_a, pa, dma_hook);
      if (m_next) apply_mask(n_a, kt_next * kBN, 0);
      unit8(BoolTag<true>{}, s_b, 1, kread, n_b, pb, dma_hook_v);
      if (m_next) apply_mask(n_b, kt_next * kBN, 1);
      tile_pv8(s_a, s_b, pa, pb, l_tile, vread);
    } else {
      unit(BoolTag<true>{}, s_a, 0, vread, kread, n_a, dma_hook);
      if (m_next) apply_mask(n_a, kt_next * kBN, 0);
      unit(BoolTag<true>{}, s_b, 1, vread, kread, n_b, dma_hook_v);
      if (m_next) apply_mask(n_b, kt_next * kBN, 1);
    }
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) {
      s_a[qb] = n_a[qb];
      s_b[qb] = n_b[qb];
    }
    store_v_fp8(vwrite);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  auto key_loop = [&]() __attribute__((always_inline)) {
    if (iters <= 0) return;   // no visible key tile (the same in every stream)
    need_ref = wave_needs_ref();
    issue_k(kt_first_s, kbuf0);
    issue_v(kt_first_s, vbuf0);
    issue_k(kt_first_s + KS, kbuf1);   // zeros if there is no second tile
    store_v_fp8(vbuf0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    s_half(kbuf0, 0, s_a, [](int) {});
    s_half(kbuf0, 1, s_b, [](int) {});
    if (tile_masked(kt_first_s)) {
      apply_mask(s_a, kt_first_s * kBN, 0);
      apply_mask(s_b, kt_first_s * kBN, 1);
    }
    __syncthreads();   // every wave is done with the first K tile before its slot is refilled
    // tiles with a successor: pairs (static slot names), then an odd one
    const int with_next = iters - 1;
    int kt = kt_first_s;
    for (int j = 0; j < with_next / 2; ++j, kt += 2 * KS) {
      iter(kt, kbuf1, vbuf0, kbuf0, vbuf1);
      iter(kt + KS, kbuf0, vbuf1, kbuf1, vbuf0);
    }
    const bool odd = (with_next & 1) != 0;
    if (odd) {
      iter(kt, kbuf1, vbuf0, kbuf0, vbuf1);
      kt += KS;
    }
    // last tile: softmax and P.V only (none if this stream's last tile lies
    // past the range)
    const unsigned char* vlast = odd ? vbuf1 : vbuf0;
    if (kt < kt_end) {
      ref_step();
      if constexpr (P8) {
        float l_tile[RB];
#pragma unroll
        for (int qb = 0; qb < RB; ++qb) l_tile[qb] = l_part[qb];
        uint32_t pa[RB][4], pb[RB][4];
        unit8(BoolTag<false>{}, s_a, 0, kbuf0, s_a, pa, [](int) {});
        unit8(BoolTag<false>{}, s_b, 1, kbuf0, s_b, pb, [](int) {});
        tile_pv8(s_a, s_b, pa, pb, l_tile, vlast);
      } else {
        // a half none of whose keys any of this wave's rows sees (past the
        // causal diagonal or a window edge, or past the sequence) adds
        // exactly nothing (p = 0): its softmax and P.V are skipped
        if (!half_dead(kt, 0)) unit(BoolTag<false>{}, s_a, 0, vlast, kbuf0, s_a, [](int) {});
        if (!half_dead(kt, 1)) unit(BoolTag<false>{}, s_b, 1, vlast, kbuf0, s_b, [](int) {});
      }
    }
    __syncthreads();   // the slots are reused by a second pass
  };
  // Exact row maxima (second pass only): S and the mask, no softmax; one K
  // tile at a time, no prefetch.
  float m_exact[RB];
  auto max_loop = [&]() {
    for (int i = 0; i < iters; ++i) {
      const int kt = kt_first_s + KS * i;
      issue_k(kt, kbuf0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kt < kt_end) {
        const bool masked = tile_masked(kt);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          f32x16 s[RB];
          s_half(kbuf0, hb, s, [](int) {});
          if (masked) apply_mask(s, kt * kBN, hb);
#pragma unroll
          for (int qb = 0; qb < RB; ++qb) m_exact[qb] = fmaxf(m_exact[qb], block_max(s[qb]));
        }
      }
      __syncthreads();
    }
  };

  // Pass 0 takes each row's reference from its first visible block.  If any
  // row of the workgroup ended with inf or NaN in l or O (a p beyond the
  // range of the P format, or an fp32 overflow), pass 1 recomputes the
  // exact row maxima and repeats the key loop with them as references.
  for (int pass = 0; pass < 2; ++pass) {
    key_loop();
    if (pass == 1) break;
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) {
      float t = pair_sum(l_part[qb]);
#pragma unroll
      for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) t += acc[qb][c][r];
      bad = bad || !__builtin_isfinite(t);
    }
    if (!__syncthreads_or(bad ? 1 : 0)) break;
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) m_exact[qb] = -INFINITY;
    max_loop();
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) m_exact[qb] = pair_max(m_exact[qb]);
    if constexpr (KS > 1) {
      // the exact maximum over all key streams
#pragma unroll
      for (int qb = 0; qb < RB; ++qb)
        if (half == 0) merge_ml[stream][wave][qb][0][col] = m_exact[qb];
      __syncthreads();
#pragma unroll
      for (int qb = 0; qb < RB; ++qb)
#pragma unroll
        for (int ss = 0; ss < KS; ++ss) m_exact[qb] = fmaxf(m_exact[qb], merge_ml[ss][wave][qb][0][col]);
      __syncthreads();
    }
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) {
      const float m = m_exact[qb];
      m_run[qb] = m;
      neg_mc[qb] = (m == -INFINITY) ? 0.f : -m * cexp + kPShift;
      l_part[qb] = 0.f;
#pragma unroll
      for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qb][c][r] = 0.f;
    }
  }

  float l_fin[RB];
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) l_fin[qb] = pair_sum(l_part[qb]);
  if constexpr (KS > 1) {
    // Merge of the key streams: each stream's O, l are relative to its own
    // reference m_s; with M the largest, O = sum_s 2^((m_s - M) c) O_s and
    // l likewise.  Streams 1.. pass theirs to stream 0 through LDS (each wave
    // through its own stream's slot; the slots are free after the key loop's
    // final barrier), and stream 0 writes the result.
    unsigned char* const own = wave == 0 ? kbuf0 : wave == 1 ? kbuf1 : wave == 2 ? vbuf0 : vbuf1;
    if (stream > 0) {
      float* dst = (float*)own;
#pragma unroll
      for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(16 * c + r) * 64 + lane] = acc[0][c][r];
      if (half == 0) {
        merge_ml[stream][wave][0][0][col] = m_run[0];
        merge_ml[stream][wave][0][1][col] = l_fin[0];
      }
    }
    __syncthreads();
    if (stream > 0) return;   // no barrier follows
    float m_all = m_run[0];
#pragma unroll
    for (int ss = 1; ss < KS; ++ss) m_all = fmaxf(m_all, merge_ml[ss][wave][0][0][col]);
    auto weight = [&](float m_s) { return m_s == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_s - m_all) * cexp); };
    const float f0 = weight(m_run[0]);
    l_fin[0] *= f0;
#pragma unroll
    for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[0][c][r] *= f0;
#pragma unroll
    for (int ss = 1; ss < KS; ++ss) {
      const float fs = weight(merge_ml[ss][wave][0][0][col]);
      l_fin[0] = __builtin_fmaf(fs, merge_ml[ss][wave][0][1][col], l_fin[0]);
      const unsigned char* theirs = wave == 0 ? kbuf0_s[ss] : wave == 1 ? kbuf1_s[ss] : wave == 2 ? vbuf0_s[ss] : vbuf1_s[ss];
      const float* src = (const float*)theirs;
#pragma unroll
      for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[0][c][r] = __builtin_fmaf(fs, src[(16 * c + r) * 64 + lane], acc[0][c][r]);
    }
    m_run[0] = m_all;
  }

  // ---- epilogue: O = O_acc / l (* v descale), LSE = ln(2) * (m c + log2 l)
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) {
    const float l_row = l_fin[qb];
    if (qrow[qb] < n && p.splits > 1) {
      // partial result of this key chunk: normalised O in fp32 and its LSE,
      // merged by attn_fwd_combine
      const float inv = l_row > 0.f ? p.v_descale / l_row : 0.f;
      const int64_t prow = ((int64_t)chunk * bh_count + bh) * n + qrow[qb];
      float* po = p.part_o + prow * D;
#pragma unroll
      for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(float4*)(po + 32 * c + 8 * j + 4 * half) =
              make_float4(acc[qb][c][4 * j] * inv, acc[qb][c][4 * j + 1] * inv, acc[qb][c][4 * j + 2] * inv,
                          acc[qb][c][4 * j + 3] * inv);
      if (half == 0)
        p.part_lse[prow] = (m_run[qb] == -INFINITY || !(l_row > 0.f))
                               ? -INFINITY
                               : (m_run[qb] * cexp + __builtin_amdgcn_logf(l_row) - kPShift) * kLn2;
    } else if (qrow[qb] < n) {
      const float inv = l_row > 0.f ? p.v_descale / l_row : 0.f;
      constexpr int kOutBytes = 2;
      unsigned char* og = (unsigned char*)p.o +
                          ((int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)qrow[qb] * p.o_ss) * kOutBytes;
#pragma unroll
      for (int c = 0; c < C::kDBlocks; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * c + 8 * j + 4 * half;
          uint2 w;
          w.x = pack2<PIN>(acc[qb][c][4 * j] * inv, acc[qb][c][4 * j + 1] * inv);
          w.y = pack2<PIN>(acc[qb][c][4 * j + 2] * inv, acc[qb][c][4 * j + 3] * inv);
          *(uint2*)(og + d * kOutBytes) = w;
        }
      if (p.lse != nullptr && half == 0) {
        const float lse = (m_run[qb] == -INFINITY || !(l_row > 0.f))
                              ? -INFINITY
                              : (m_run[qb] * cexp + __builtin_amdgcn_logf(l_row) - kPShift) * kLn2;
        p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + qrow[qb]] = lse;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launch
// ---------------------------------------------------------------------------
// Merge of the key chunks' partial results (p.splits > 1): per query row,
// LSE = ln sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s, written in
// the output type; a row no chunk saw keeps O = 0, LSE = -inf.  One thread per
// 4 columns of a row; HBM-bound.
template <In OUT, int D>
__global__ void __launch_bounds__(256) attn_fwd_combine(const FwdParams p) {
  constexpr int kThreadsPerRow = D / 4;
  constexpr int kRowsPerBlock = 256 / kThreadsPerRow;
  const int64_t rows = (int64_t)p.batch * p.heads * p.n;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kThreadsPerRow;
  if (r >= rows) return;
  const int d = (threadIdx.x % kThreadsPerRow) * 4;
  const int row = (int)(r % p.n);
  const int bh = (int)(r / p.n);
  const int b = bh / p.heads, h = bh - b * p.heads;
  const int64_t stride = rows;   // between chunks
  float m = -INFINITY;
  for (int s = 0; s < p.splits; ++s) m = fmaxf(m, p.part_lse[s * stride + r]);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float lse = -INFINITY;
  if (m != -INFINITY) {
    float wsum = 0.f;
    for (int s = 0; s < p.splits; ++s) {
      const float w = __builtin_amdgcn_exp2f((p.part_lse[s * stride + r] - m) * 1.4426950408889634f);
      if (w > 0.f) {
        const float4 x = *(const float4*)(p.part_o + (s * stride + r) * D + d);
        o.x = __builtin_fmaf(w, x.x, o.x);
        o.y = __builtin_fmaf(w, x.y, o.y);
        o.z = __builtin_fmaf(w, x.z, o.z);
        o.w = __builtin_fmaf(w, x.w, o.w);
      }
      wsum += w;
    }
    const float inv = 1.f / wsum;
    o = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    lse = m + __builtin_amdgcn_logf(wsum) * kLn2;
  }
  unsigned char* og = (unsigned char*)p.o + ((int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)row * p.o_ss) * 2;
  uint2 w;
  w.x = pack2<OUT>(o.x, o.y);
  w.y = pack2<OUT>(o.z, o.w);
  *(uint2*)(og + d * 2) = w;
  if (p.lse != nullptr && d == 0) p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + row] = lse;
}

// Scratch of the allocation-free entry point.  Each GPU the library runs on
// holds its own copy for the life of the process; in host code `scratch` is
// only a handle, so kernels receive the address hipGetSymbolAddress reports
// for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(int dev, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t status[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    void* a = nullptr;
    status[dev] = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    addr[dev] = status[dev] == hipSuccess ? a : nullptr;
  });
  *ptr = addr[dev];
  return status[dev];
}

template <In IN, int D, int WAVES, int RB, bool P8, int KS, bool V16 = false>
static hipError_t launch_t(const FwdParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.q_tiles * p.batch * p.heads * p.splits));
  const dim3 block(64 * WAVES * KS);
  hipLaunchKernelGGL((attn_fwd_kernel<IN, D, WAVES, RB, P8, KS, V16>), grid, block, 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  constexpr In OUT = (IN == In::F16) ? In::F16 : In::BF16;
  constexpr int kRowsPerBlock = 256 / (D / 4);
  const int64_t rows = (int64_t)p.batch * p.heads * p.n;
  hipLaunchKernelGGL((attn_fwd_combine<OUT, D>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

// The 16-bit configurations by key streams: row waves per stream, streams.
template <In IN, int D>
static hipError_t launch_16bit(const FwdParams& p, int cfg, hipStream_t stream) {
  switch (cfg) {
    case 0: return launch_t<IN, D, 4, 1, false, 1>(p, stream);
    case 2: return launch_t<IN, D, 4, 1, false, 2>(p, stream);
    // four streams only at d = 64: four times two K and two V slots must fit a CU's LDS
    case 3: if constexpr (D == 64) return launch_t<IN, D, 1, 1, false, 4>(p, stream); else return hipErrorInvalidValue;
    // 64 rows and two streams at d = 64 (at d = 128 its registers would leave one wave per SIMD)
    case 4: if constexpr (D == 64) return launch_t<IN, D, 2, 1, false, 2>(p, stream); else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

// fp8 V widened exactly to bf16 (every e4m3 value is a bf16 value) into
// the copy [B][Hk][N][D]: one thread per 16 stored bytes of a V row.  It is
// bound by HBM (one byte read and two written per element), and lets the
// attention kernel load bf16 V tiles by DMA, as for 16-bit inputs, instead
// of every workgroup widening each V tile it loads through its registers.
template <int D>
__global__ void __launch_bounds__(256) attn_widen_v(const FwdParams p) {
  constexpr int kChunks = D / 16;
  const int hk = p.heads / p.group;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)p.batch * hk * p.n * kChunks) return;
  const int c = (int)(t % kChunks);
  const int64_t r = t / kChunks;                 // copy row: (b Hk + h) N + s
  const int s = (int)(r % p.n);
  const int64_t bh = r / p.n;
  const int h = (int)(bh % hk), b = (int)(bh / hk);
  const unsigned char* src =
      (const unsigned char*)p.v + (int64_t)b * p.v_sb + (int64_t)h * p.v_sh + (int64_t)s * p.v_ss + c * 16;
  uint4 lo, hi;
  fp8x16_to_bf16(*(const uint4*)src, lo, hi);
  uint4* dst = (uint4*)((unsigned char*)p.v_wide + (r * D + c * 16) * 2);
  dst[0] = lo;
  dst[1] = hi;
}

hipError_t launch_fwd(const FwdParams& p, int in_dtype, int d, int cfg, hipStream_t stream) {
  // in_dtype: 1 = f16, 2 = bf16, 3 = fp8 e4m3 (validated by the caller)
  if (in_dtype == 3) {
    if (d != 128) return hipErrorInvalidValue;
    if (cfg == 0 && p.v_wide != nullptr) {
      const int64_t threads = (int64_t)p.batch * (p.heads / p.group) * p.n * (128 / 16);
      hipLaunchKernelGGL((attn_widen_v<128>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      // the attention kernel reads the copy: element strides of [B][Hk][N][D]
      FwdParams pw = p;
      pw.v = p.v_wide;
      pw.v_ss = 128;
      pw.v_sh = (int64_t)p.n * 128;
      pw.v_sb = (int64_t)(p.heads / p.group) * p.n * 128;
      return launch_t<In::FP8, 128, 4, 1, false, 1, true>(pw, stream);
    }
    if (cfg == 0) return launch_t<In::FP8, 128, 4, 1, false, 1>(p, stream);
    if (cfg == 1) return launch_t<In::FP8, 128, 4, 1, true, 1>(p, stream);
    return hipErrorInvalidValue;
  }
  if (in_dtype == 1 && d == 64) return launch_16bit<In::F16, 64>(p, cfg, stream);
  if (in_dtype == 1 && d == 128) return launch_16bit<In::F16, 128>(p, cfg, stream);
  if (in_dtype == 2 && d == 64) return launch_16bit<In::BF16, 64>(p, cfg, stream);
  if (in_dtype == 2 && d == 128) return launch_16bit<In::BF16, 128>(p, cfg, stream);
  return hipErrorInvalidValue;
}

}  // namespace ea
