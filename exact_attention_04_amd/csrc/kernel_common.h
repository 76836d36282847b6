// Device-side building blocks shared by the attention kernels (forward and
// backward) for gfx950: operand types, the swizzled LDS tile layout, MFMA
// and conversion wrappers, range-checked buffer loads and the mask
// classification of blocks of (query, key) pairs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tiles.h"

namespace ea {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr float kLn2 = 0.6931471805599453f;

enum class In { F16, BF16, FP8 };

// ---------------------------------------------------------------------------
// LDS layout: a K or V tile is kBN rows of ROW_BYTES bytes, split into
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

__device__ __forceinline__ f32x16 mfma_fp8(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x16 c) {
  const i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8 bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  // formats 0/0: both operands OCP e4m3; scale exponents 127: no block scaling
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
}

// The same with B scaled by 2^(scale_b - 127) (E8M0 exponent).
__device__ __forceinline__ f32x16 mfma_fp8_scaled(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x16 c, int scale_b) {
  const i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8 bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, scale_b);
}

// Pack two fp32 values into the P operand type (round to nearest even):
// one v_cvt_pk_{bf16,f16}_f32.
template <In IN>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 v = {a, b};
  if constexpr (IN == In::F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
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

// fp8 e4m3 x16 (one uint4) -> bf16 x16 (two uint4), exact (bf16 holds every
// e4m3 value): one packed convert per two values, bytes 0-1 of a dword to
// its first bf16 pair and bytes 2-3 to the second, with scale 1.
__device__ __forceinline__ void fp8x16_to_bf16(uint4 in, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.0f, false));
    o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.0f, true));
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// Buffer resource of `bytes` bytes at `base` (word 3 = 0x00020000: raw,
// untyped access on this GPU family).  Offsets at or past `bytes` read as 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// 16 bytes per lane from global memory straight into LDS: lane L's bytes at
// base + voff land at lds + 16 L (one instruction fills 1 KB).
__device__ __forceinline__ void load_16b_to_lds(const void* base, int bytes, uint32_t voff, unsigned char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_rsrc(base, bytes), (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

// 16 bytes from global memory into registers (0 past `bytes`).
__device__ __forceinline__ uint4 load_16b(const void* base, int bytes, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(base, bytes), voff, 0, 0));
}

// The values of lanes l and l ^ 32 of a wave (the two key halves of one query
// row), both in every lane: one v_permlane32_swap exchanges the upper 32 lanes
// of one copy with the lower 32 lanes of the other, so the two results hold
// {lane l, lane l ^ 32} in some order (no LDS round trip).
struct LanePair {
  float a, b;
};
__device__ __forceinline__ LanePair lane_pair(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return {__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}
// Sum and max over the two lanes of a query row.
__device__ __forceinline__ float pair_sum(float x) {
  const LanePair p = lane_pair(x);
  return p.a + p.b;
}
__device__ __forceinline__ float pair_max(float x) {
  const LanePair p = lane_pair(x);
  return fmaxf(p.a, p.b);
}

// Visible-key range of query rows [q0, q0+qrows) and the mask classification
// of a block of rows x keys.  Key j is visible from query i iff j < n,
// (!causal || j <= i), (wl < 0 || j >= i - wl) and (wr < 0 || j <= i + wr).
struct KeyRange {
  int lo, hi;   // [lo, hi) keys that any of the rows can see
};

__device__ __forceinline__ KeyRange tile_key_range(int q0, int qrows, int n, int causal, int wl, int wr) {
  const int qlast = min(q0 + qrows, n) - 1;
  const int lo = wl >= 0 ? max(0, q0 - wl) : 0;
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

// One 16-key k-step j of the P.V product below (pv_half): 4 packed P pairs
// per row block.
template <In PIN, int D, int RB>
__device__ __forceinline__ void pv_kstep(f32x16 (&acc)[RB][D / 32], const uint32_t (&pk)[RB][4],
                                         const unsigned char* vl, const uint32_t (&va)[2][D / 32], int hb, int j) {
  // the fragment reads of the step are issued together, ahead of its MFMAs,
  // so their latency is paid once per step rather than per MFMA
  const unsigned char* base = vl + (32 * hb + 16 * j) * (2 * D);
  uint4 aop[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + va[0][c]));
    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + va[1][c]));
    const uint2 w0 = __builtin_bit_cast(uint2, t0);
    const uint2 w1 = __builtin_bit_cast(uint2, t1);
    aop[c] = make_uint4(w0.x, w0.y, w1.x, w1.y);
  }
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int qb = 0; qb < RB; ++qb)
      acc[qb][c] = mfma_16bit<PIN>(aop[c], make_uint4(pk[qb][0], pk[qb][1], pk[qb][2], pk[qb][3]), acc[qb][c]);
}

// The V^T fragments of one 16-key k-step j of pv_kstep, read ahead of its
// MFMAs (pv_kstep_with).
template <int D>
__device__ __forceinline__ void pv_frags(uint4 (&aop)[D / 32], const unsigned char* vl, const uint32_t (&va)[2][D / 32],
                                         int hb, int j) {
  const unsigned char* base = vl + (32 * hb + 16 * j) * (2 * D);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const uint2 w0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + va[0][c])));
    const uint2 w1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + va[1][c])));
    aop[c] = make_uint4(w0.x, w0.y, w1.x, w1.y);
  }
}
template <In PIN, int D, int RB>
__device__ __forceinline__ void pv_kstep_with(f32x16 (&acc)[RB][D / 32], const uint32_t (&pk)[RB][8],
                                              const uint4 (&aop)[D / 32], int j) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int qb = 0; qb < RB; ++qb)
      acc[qb][c] = mfma_16bit<PIN>(aop[c], make_uint4(pk[qb][4 * j], pk[qb][4 * j + 1], pk[qb][4 * j + 2], pk[qb][4 * j + 3]),
                                   acc[qb][c]);
}

// O^T += V^T P^T for both row blocks over the 32 keys [32 hb, 32 hb + 32) of a
// staged tile, as two k-steps of 16 keys (pv_kstep, j = 0, 1).  P^T (16-bit,
// B operand) is in the layout the S^T accumulator left it: lane l holds query
// l%32 and, for k-step j, keys 32 hb + 16 j + {4 half + t, 8 + 4 half + t},
// t < 4 (packed pairs pk[4 j .. 4 j + 3]).  The matching V^T fragment (A
// operand: row d = l%32 of a 32-column block, the same 8 keys) is gathered
// with two transposing LDS reads: within each 16-lane group, source lane sl
// points at key base + sl/4, columns 4 (sl%4) .. +3, and lane i receives
// column i of the 4 consecutive keys.  Each fragment feeds both row blocks.
//
// `va[r8][c]` is this lane's byte offset, within a V tile, of its read for
// key row 4 (g/2) + sl/4 + 8 r8 and column block c; moving by 16 or 32 key
// rows leaves the swizzle unchanged, so every other read of the tile is that
// offset plus a constant.
template <In PIN, int D, int RB>
__device__ __forceinline__ void pv_half(f32x16 (&acc)[RB][D / 32], const uint32_t (&pk)[RB][8],
                                        const unsigned char* vl, const uint32_t (&va)[2][D / 32], int hb) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t pj[RB][4];
#pragma unroll
    for (int qb = 0; qb < RB; ++qb)
#pragma unroll
      for (int t = 0; t < 4; ++t) pj[qb][t] = pk[qb][4 * j + t];
    pv_kstep<PIN, D, RB>(acc, pj, vl, va, hb, j);
  }
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};
template <int I>
struct IntTag {
  static constexpr int value = I;
};

// Work order of a grid of `units` x `heads` workgroups, unit 0 the heaviest:
// returns (unit, head) of workgroup w.  Workgroups go to the 8 XCDs round
// robin (w on XCD w % 8); XCD x takes its heads 8 i + x in groups of g and
// runs a group's units, heaviest first, before the next group, so the
// workgroups resident on one XCD read the same few heads' tiles through its
// L2.  The head count must be a multiple of 8 g.  A unit is whatever the
// caller makes of it (a query tile; a query tile of one of a K/V head's
// query heads).
__device__ __forceinline__ int2 xcd_grouped(int w, int units, int g) {
  const int x = w & 7, s = w >> 3, per = g * units;
  return make_int2((s % per) / g, ((s / per) * g + (s % per) % g) * 8 + x);
}

}  // namespace ea
