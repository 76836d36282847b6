// C ABI of the exact-attention forward: argument checks, planning and launch.
// The contract of every entry point is stated in include/ea_attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "ea_attn.h"
#include "bwd_kernel.h"
#include "fwd_kernel.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
bool g_dev_is_gfx950[kMaxDevices];

bool device_is_gfx950(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return false;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    g_dev_is_gfx950[dev] = false;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      // gcnArchName looks like "gfx950:sramecc+:xnack-"
      g_dev_is_gfx950[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                             (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
    }
  });
  return g_dev_is_gfx950[dev];
}

int elem_bytes(int dtype) {
  switch (dtype) {
    case EA_F16:
    case EA_BF16: return 2;
    case EA_FP8_E4M3: return 1;
    case EA_F32: return 4;
    default: return 0;
  }
}

// Largest byte extent accepted for one tensor (128 TiB, beyond any device
// allocation): with it, every offset the kernels form fits in int64 and a
// base pointer plus its extent cannot wrap.
constexpr int64_t kMaxExtentBytes = (int64_t)1 << 47;

// Byte extent of a [B, S, H, D] strided tensor (strides >= 0, sizes >= 1):
// (B-1) sb + (S-1) ss + (H-1) sh + D elements of `esz` bytes.  False when it
// overflows or exceeds kMaxExtentBytes.
bool extent_of(int64_t B, int64_t S, int64_t H, int64_t D, int64_t sb, int64_t ss, int64_t sh, int esz,
               int64_t* bytes) {
  int64_t t0 = 0, t1 = 0, t2 = 0, sum = 0, out = 0;
  if (__builtin_mul_overflow(B - 1, sb, &t0) || __builtin_mul_overflow(S - 1, ss, &t1) ||
      __builtin_mul_overflow(H - 1, sh, &t2) || __builtin_add_overflow(t0, t1, &sum) ||
      __builtin_add_overflow(sum, t2, &sum) || __builtin_add_overflow(sum, D, &sum) ||
      __builtin_mul_overflow(sum, (int64_t)esz, &out) || out > kMaxExtentBytes)
    return false;
  *bytes = out;
  return true;
}

// Byte range [lo, hi) spanned by a tensor whose extent passed extent_of.
struct Span {
  uintptr_t lo, hi;
};
Span span_at(const void* base, int64_t bytes) {
  const uintptr_t lo = (uintptr_t)base;
  return {lo, lo + (uintptr_t)bytes};
}
Span span_of(const void* base, int64_t B, int64_t S, int64_t H, int64_t D, int64_t sb, int64_t ss, int64_t sh,
             int esz) {
  int64_t bytes = 0;
  extent_of(B, S, H, D, sb, ss, sh, esz, &bytes);
  return span_at(base, bytes);
}
bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Span of an fp32 [B, H, N] array with row stride 1.
Span span_rows_f32(const void* base, int64_t B, int64_t H, int64_t N, int64_t sb, int64_t sh) {
  return span_of(base, B, 1, H, N, sb, 0, sh, 4);
}
bool rows_f32_fit(int64_t B, int64_t H, int64_t N, int64_t sb, int64_t sh) {
  int64_t bytes = 0;
  return extent_of(B, 1, H, N, sb, 0, sh, 4, &bytes);
}

// A window bound at or past the sequence length bounds nothing: it is
// treated as -1, which keeps the kernels' row + bound sums within int32.
int32_t effective_window(int32_t w, int64_t n) { return (int64_t)w >= n ? -1 : w; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Checks shared by ea_attn_fwd and ea_attn_plan.  Returns EA_OK, or the error.
// Sets *empty when there is nothing to compute.
// Version-1 sizes of the growing structs: everything before the fields added
// since.
constexpr size_t kArgsV1Size = offsetof(ea_attn_args, workspace);
constexpr size_t kArgsV2Size = offsetof(ea_attn_args, pv_dtype);
constexpr size_t kPlanV1Size = offsetof(ea_attn_plan_info, workspace_bytes);

// The caller's workspace (pointer, bytes), or none when its struct predates it.
void* workspace_of(const ea_attn_args* a, int64_t* bytes) {
  if (a->struct_size < kArgsV2Size || a->workspace == nullptr || a->workspace_bytes <= 0) {
    *bytes = 0;
    return nullptr;
  }
  *bytes = a->workspace_bytes;
  return a->workspace;
}

// pv_dtype, or 0 when the caller's struct predates it.
int32_t pv_dtype_of(const ea_attn_args* a) { return a->struct_size >= sizeof(ea_attn_args) ? a->pv_dtype : 0; }

int validate(const ea_attn_args* a, bool* empty) {
  *empty = false;
  if (a == nullptr || a->struct_size < kArgsV1Size) return EA_EINVAL;
  if (a->batch < 0 || a->seqlen_q < 0 || a->seqlen_k < 0 || a->nheads_q < 1 || a->nheads_k < 1 ||
      a->headdim < 1)
    return EA_EINVAL;
  if (elem_bytes(a->in_dtype) == 0 || elem_bytes(a->out_dtype) == 0) return EA_EINVAL;
  if (!std::isfinite(a->softmax_scale)) return EA_EINVAL;
  const bool fp8 = a->in_dtype == EA_FP8_E4M3;
  const float ds[3] = {a->q_descale, a->k_descale, a->v_descale};
  for (float d : ds) {
    if (!std::isfinite(d) || !(d > 0.f)) return EA_EINVAL;
    if (!fp8 && d != 1.0f) return EA_EINVAL;
  }
  if (a->window_left < -1 || a->window_right < -1) return EA_EINVAL;
  const int32_t pv = pv_dtype_of(a);
  if (pv != 0 && pv != EA_BF16 && pv != EA_FP8_E4M3) return EA_EINVAL;
  if (a->struct_size >= sizeof(ea_attn_args) && a->reserved != 0) return EA_EINVAL;

  // what the kernels implement
  if (a->in_dtype == EA_F32) return EA_EUNSUPPORTED;
  if (!fp8 && pv != 0) return EA_EUNSUPPORTED;
  if (fp8 ? a->out_dtype != EA_BF16 : a->out_dtype != a->in_dtype) return EA_EUNSUPPORTED;
  if (a->headdim != 64 && a->headdim != 128) return EA_EUNSUPPORTED;
  if (fp8 && a->headdim != 128) return EA_EUNSUPPORTED;
  if (a->seqlen_q != a->seqlen_k) return EA_EUNSUPPORTED;
  if (a->nheads_q % a->nheads_k != 0) return EA_EUNSUPPORTED;
  if (!(a->softmax_scale > 0.f)) return EA_EUNSUPPORTED;

  if (a->batch == 0 || a->seqlen_q == 0) {
    *empty = true;
    return EA_OK;
  }
  if (a->q == nullptr || a->k == nullptr || a->v == nullptr || a->o == nullptr) return EA_EINVAL;

  const int64_t B = a->batch, N = a->seqlen_q, H = a->nheads_q, Hk = a->nheads_k, D = a->headdim;
  const int ein = elem_bytes(a->in_dtype), eout = elem_bytes(a->out_dtype);
  const int64_t strides[12] = {a->q_stride_b, a->q_stride_s, a->q_stride_h, a->k_stride_b, a->k_stride_s, a->k_stride_h,
                               a->v_stride_b, a->v_stride_s, a->v_stride_h, a->o_stride_b, a->o_stride_s, a->o_stride_h};
  for (int i = 0; i < 12; ++i) {
    if (strides[i] < 0 || strides[i] > kMaxExtentBytes) return EA_EUNSUPPORTED;
    const int esz = i < 9 ? ein : eout;
    if ((strides[i] * esz) % 16 != 0) return EA_EUNSUPPORTED;
  }
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o)) return EA_EUNSUPPORTED;
  if (a->lse != nullptr) {
    if (((uintptr_t)a->lse & 3u) != 0 || a->lse_stride_b < 0 || a->lse_stride_h < 0) return EA_EUNSUPPORTED;
  }
  // the kernels keep per-head row offsets and tile indices in 32 bits
  const int64_t lim = (int64_t)1 << 31;
  int64_t bh = 0;
  if (N >= lim / 2 || __builtin_mul_overflow(B, H, &bh) || bh >= lim) return EA_EUNSUPPORTED;
  for (int i = 0; i < 4; ++i) {
    // (the first test keeps the products below from overflowing)
    if (strides[3 * i + 1] >= lim || strides[3 * i + 1] * N >= lim) return EA_EUNSUPPORTED;
    // byte offsets within a 64-row K/V tile are 32-bit
    if (strides[3 * i + 1] * 64 * 2 >= lim) return EA_EUNSUPPORTED;
  }

  // every tensor's extent is bounded before any span is formed
  {
    int64_t bytes = 0;
    const int64_t heads[4] = {H, Hk, Hk, H};
    for (int i = 0; i < 4; ++i)
      if (!extent_of(B, N, heads[i], D, strides[3 * i], strides[3 * i + 1], strides[3 * i + 2], i < 3 ? ein : eout,
                     &bytes))
        return EA_EUNSUPPORTED;
    if (a->lse != nullptr && !rows_f32_fit(B, H, N, a->lse_stride_b, a->lse_stride_h)) return EA_EUNSUPPORTED;
    if (a->struct_size >= kArgsV2Size && a->workspace != nullptr && a->workspace_bytes > kMaxExtentBytes)
      return EA_EUNSUPPORTED;
  }
  const Span so = span_of(a->o, B, N, H, D, a->o_stride_b, a->o_stride_s, a->o_stride_h, eout);
  const Span sq = span_of(a->q, B, N, H, D, a->q_stride_b, a->q_stride_s, a->q_stride_h, ein);
  const Span sk = span_of(a->k, B, N, Hk, D, a->k_stride_b, a->k_stride_s, a->k_stride_h, ein);
  const Span sv = span_of(a->v, B, N, Hk, D, a->v_stride_b, a->v_stride_s, a->v_stride_h, ein);
  if (overlaps(so, sq) || overlaps(so, sk) || overlaps(so, sv)) return EA_EINVAL;
  if (a->lse != nullptr) {
    const Span sl = span_rows_f32(a->lse, B, H, N, a->lse_stride_b, a->lse_stride_h);
    if (overlaps(sl, so) || overlaps(sl, sq) || overlaps(sl, sk) || overlaps(sl, sv)) return EA_EINVAL;
  }
  int64_t ws_bytes = 0;
  if (void* ws = workspace_of(a, &ws_bytes)) {
    if (!aligned16(ws)) return EA_EUNSUPPORTED;
    const Span sw{(uintptr_t)ws, (uintptr_t)ws + (uintptr_t)ws_bytes};
    if (overlaps(sw, so) || overlaps(sw, sq) || overlaps(sw, sk) || overlaps(sw, sv)) return EA_EINVAL;
    if (a->lse != nullptr && overlaps(sw, span_rows_f32(a->lse, B, H, N, a->lse_stride_b, a->lse_stride_h)))
      return EA_EINVAL;
  }
  return EA_OK;
}

// Kernel configuration (see fwd_kernel.h).  fp8: 1 for the e4m3 P.V, else
// 0.  16-bit, by the launch's items (query tiles of 128 rows x heads): 0 when
// they give every CU two workgroups; below that key streams, four streams of
// 32 rows at d = 64 with fewer than 128 items, else two streams of 128 rows
// (8 waves, one workgroup per CU: two waves per SIMD).
// Whether the key work of the 128-row query tiles is unbalanced (causal or
// windowed masks): the heaviest tile sees at least 1.5x the average key
// tiles.  O(N / 128) on the host.
bool unbalanced_tiles(const ea_attn_args* a) {
  const int n = (int)a->seqlen_q, bm = 128, bn = ea::tile_bn();
  const int wl = effective_window(a->window_left, n), wr = effective_window(a->window_right, n);
  const int qt = (n + bm - 1) / bm;
  int64_t total = 0;
  int most = 0;
  for (int t = 0; t < qt; ++t) {
    const int q0 = t * bm, qlast = std::min(q0 + bm, n) - 1;
    const int lo = wl >= 0 ? std::max(0, q0 - wl) : 0;
    int hi = n;
    if (a->causal) hi = std::min(hi, qlast + 1);
    if (wr >= 0) hi = std::min(hi, qlast + wr + 1);
    hi = std::max(lo, hi);
    const int c = (hi + bn - 1) / bn - lo / bn;
    total += c;
    most = std::max(most, c);
  }
  return 2 * (int64_t)most * qt >= 3 * total;
}

// Tile configuration (see plan.cpp): the plain 128-row one when the query
// tiles fill two workgroups per CU; otherwise key streams: at d = 64, four
// streams of 32 rows for the fewest tiles, and two streams of 64 rows where
// the tiles' work is unbalanced (twice the workgroups, so the heaviest-first
// order balances them); else two streams of 128 rows.
int choose_cfg(const ea_attn_args* a) {
  if (a->in_dtype == EA_FP8_E4M3) return pv_dtype_of(a) == EA_FP8_E4M3 ? 1 : 0;
  const int64_t items = a->batch * a->nheads_q * ((a->seqlen_q + 127) / 128);
  if (items >= 512) return 0;
  if (a->headdim == 64) {
    if (items < 128) return 3;
    if (unbalanced_tiles(a)) return 4;
  }
  return 2;
}

ea::FwdParams make_params(const ea_attn_args* a, int cfg) {
  ea::FwdParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.batch = (int)a->batch;
  p.heads = (int)a->nheads_q;
  p.group = (int)(a->nheads_q / a->nheads_k);
  p.n = (int)a->seqlen_q;
  p.q_tiles = (p.n + ea::tile_bm(cfg) - 1) / ea::tile_bm(cfg);
  p.q_sb = a->q_stride_b; p.q_ss = a->q_stride_s; p.q_sh = a->q_stride_h;
  p.k_sb = a->k_stride_b; p.k_ss = a->k_stride_s; p.k_sh = a->k_stride_h;
  p.v_sb = a->v_stride_b; p.v_ss = a->v_stride_s; p.v_sh = a->v_stride_h;
  p.o_sb = a->o_stride_b; p.o_ss = a->o_stride_s; p.o_sh = a->o_stride_h;
  p.lse_sb = a->lse_stride_b; p.lse_sh = a->lse_stride_h;
  p.causal = a->causal ? 1 : 0;
  p.wl = effective_window(a->window_left, a->seqlen_q);
  p.wr = effective_window(a->window_right, a->seqlen_q);
  const bool fp8 = a->in_dtype == EA_FP8_E4M3;
  const double c = (double)a->softmax_scale * (fp8 ? (double)a->q_descale * (double)a->k_descale : 1.0) *
                   1.4426950408889634;
  p.c_log2 = (float)c;
  p.v_descale = fp8 ? a->v_descale : 1.0f;
  p.splits = 1;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  p.v_wide = nullptr;
  return p;
}

// Checks of ea_attn_bwd.  Returns EA_OK, or the error; sets *empty when there
// is nothing to compute.
int validate_bwd(const ea_attn_bwd_args* a, bool* empty) {
  *empty = false;
  if (a == nullptr || a->struct_size < sizeof(ea_attn_bwd_args)) return EA_EINVAL;
  if (a->batch < 0 || a->seqlen < 0 || a->nheads_q < 1 || a->nheads_k < 1 || a->headdim < 1) return EA_EINVAL;
  if (elem_bytes(a->dtype) == 0) return EA_EINVAL;
  if (!std::isfinite(a->softmax_scale)) return EA_EINVAL;
  if (a->window_left < -1 || a->window_right < -1) return EA_EINVAL;
  if (a->dtype != EA_F16 && a->dtype != EA_BF16) return EA_EUNSUPPORTED;
  if (a->headdim != 64 && a->headdim != 128) return EA_EUNSUPPORTED;
  if (a->nheads_q % a->nheads_k != 0) return EA_EUNSUPPORTED;
  if (!(a->softmax_scale > 0.f)) return EA_EUNSUPPORTED;
  if (a->batch == 0 || a->seqlen == 0) {
    *empty = true;
    return EA_OK;
  }
  const void* ptrs[10] = {a->q, a->k, a->v, a->o, a->dout, a->lse, a->delta, a->dq, a->dk, a->dv};
  for (int i = 0; i < 10; ++i)
    if (ptrs[i] == nullptr) return EA_EINVAL;

  const int64_t B = a->batch, N = a->seqlen, H = a->nheads_q, Hk = a->nheads_k, D = a->headdim;
  const int64_t strides[24] = {a->q_stride_b,  a->q_stride_s,  a->q_stride_h,  a->k_stride_b,  a->k_stride_s,  a->k_stride_h,
                               a->v_stride_b,  a->v_stride_s,  a->v_stride_h,  a->o_stride_b,  a->o_stride_s,  a->o_stride_h,
                               a->do_stride_b, a->do_stride_s, a->do_stride_h, a->dq_stride_b, a->dq_stride_s, a->dq_stride_h,
                               a->dk_stride_b, a->dk_stride_s, a->dk_stride_h, a->dv_stride_b, a->dv_stride_s, a->dv_stride_h};
  for (int i = 0; i < 24; ++i) {
    if (strides[i] < 0 || strides[i] > kMaxExtentBytes) return EA_EUNSUPPORTED;
    if ((strides[i] * 2) % 16 != 0) return EA_EUNSUPPORTED;
  }
  for (int i = 0; i < 10; ++i) {
    if (i == 5 || i == 6) continue;
    if (!aligned16(ptrs[i])) return EA_EUNSUPPORTED;
  }
  if (((uintptr_t)a->lse & 3u) != 0 || ((uintptr_t)a->delta & 3u) != 0) return EA_EUNSUPPORTED;
  if (a->lse_stride_b < 0 || a->lse_stride_h < 0 || a->delta_stride_b < 0 || a->delta_stride_h < 0)
    return EA_EUNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;
  int64_t bh = 0;
  if (N >= lim / 2 || __builtin_mul_overflow(B, H, &bh) || bh >= lim) return EA_EUNSUPPORTED;
  if ((N + 127) / 128 * bh >= lim / 2) return EA_EUNSUPPORTED;
  for (int i = 0; i < 8; ++i) {
    if (strides[3 * i + 1] >= lim || strides[3 * i + 1] * N >= lim) return EA_EUNSUPPORTED;
    if (strides[3 * i + 1] * 64 * 2 >= lim) return EA_EUNSUPPORTED;
  }
  {
    int64_t bytes = 0;
    const int64_t heads[8] = {H, Hk, Hk, H, H, H, Hk, Hk};
    for (int i = 0; i < 8; ++i)
      if (!extent_of(B, N, heads[i], D, strides[3 * i], strides[3 * i + 1], strides[3 * i + 2], 2, &bytes))
        return EA_EUNSUPPORTED;
    if (!rows_f32_fit(B, H, N, a->lse_stride_b, a->lse_stride_h) ||
        !rows_f32_fit(B, H, N, a->delta_stride_b, a->delta_stride_h))
      return EA_EUNSUPPORTED;
  }
  // outputs (dq, dk, dv, delta) overlap neither each other nor any input
  const Span in[6] = {span_of(a->q, B, N, H, D, a->q_stride_b, a->q_stride_s, a->q_stride_h, 2),
                      span_of(a->k, B, N, Hk, D, a->k_stride_b, a->k_stride_s, a->k_stride_h, 2),
                      span_of(a->v, B, N, Hk, D, a->v_stride_b, a->v_stride_s, a->v_stride_h, 2),
                      span_of(a->o, B, N, H, D, a->o_stride_b, a->o_stride_s, a->o_stride_h, 2),
                      span_of(a->dout, B, N, H, D, a->do_stride_b, a->do_stride_s, a->do_stride_h, 2),
                      span_rows_f32(a->lse, B, H, N, a->lse_stride_b, a->lse_stride_h)};
  const Span out[4] = {span_of(a->dq, B, N, H, D, a->dq_stride_b, a->dq_stride_s, a->dq_stride_h, 2),
                       span_of(a->dk, B, N, Hk, D, a->dk_stride_b, a->dk_stride_s, a->dk_stride_h, 2),
                       span_of(a->dv, B, N, Hk, D, a->dv_stride_b, a->dv_stride_s, a->dv_stride_h, 2),
                       span_rows_f32(a->delta, B, H, N, a->delta_stride_b, a->delta_stride_h)};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i], in[j])) return EA_EINVAL;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out[j])) return EA_EINVAL;
  }
  return EA_OK;
}

ea::BwdParams make_bwd_params(const ea_attn_bwd_args* a) {
  ea::BwdParams p;
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.dout = a->dout;
  p.lse = a->lse; p.delta = a->delta;
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  p.batch = (int)a->batch;
  p.heads = (int)a->nheads_q;
  p.heads_kv = (int)a->nheads_k;
  p.group = (int)(a->nheads_q / a->nheads_k);
  p.n = (int)a->seqlen;
  p.q_tiles = (p.n + 127) / 128;
  p.k_blocks = (p.n + 127) / 128;
  p.q_sb = a->q_stride_b; p.q_ss = a->q_stride_s; p.q_sh = a->q_stride_h;
  p.k_sb = a->k_stride_b; p.k_ss = a->k_stride_s; p.k_sh = a->k_stride_h;
  p.v_sb = a->v_stride_b; p.v_ss = a->v_stride_s; p.v_sh = a->v_stride_h;
  p.o_sb = a->o_stride_b; p.o_ss = a->o_stride_s; p.o_sh = a->o_stride_h;
  p.do_sb = a->do_stride_b; p.do_ss = a->do_stride_s; p.do_sh = a->do_stride_h;
  p.dq_sb = a->dq_stride_b; p.dq_ss = a->dq_stride_s; p.dq_sh = a->dq_stride_h;
  p.dk_sb = a->dk_stride_b; p.dk_ss = a->dk_stride_s; p.dk_sh = a->dk_stride_h;
  p.dv_sb = a->dv_stride_b; p.dv_ss = a->dv_stride_s; p.dv_sh = a->dv_stride_h;
  p.lse_sb = a->lse_stride_b; p.lse_sh = a->lse_stride_h;
  p.delta_sb = a->delta_stride_b; p.delta_sh = a->delta_stride_h;
  p.causal = a->causal ? 1 : 0;
  p.wl = effective_window(a->window_left, a->seqlen);
  p.wr = effective_window(a->window_right, a->seqlen);
  p.scale = a->softmax_scale;
  p.c_log2 = (float)((double)a->softmax_scale * 1.4426950408889634);
  return p;
}

// Key tiles of the query tile with the most (the kernel's visible key range).
int max_kv_tiles(const ea::FwdParams& p, int cfg) {
  const int bm = ea::tile_bm(cfg), bn = ea::tile_bn();
  int best = 0;
  for (int t = 0; t < p.q_tiles; ++t) {
    const int q0 = t * bm;
    const int qlast = std::min(q0 + bm, p.n) - 1;
    const int lo = p.wl >= 0 ? std::max(0, q0 - p.wl) : 0;
    int hi = p.n;
    if (p.causal) hi = std::min(hi, qlast + 1);
    if (p.wr >= 0) hi = std::min(hi, qlast + p.wr + 1);
    hi = std::max(lo, hi);
    best = std::max(best, (hi + bn - 1) / bn - lo / bn);
  }
  return best;
}

// Host-side mirror of the kernel's tile walk, for plan reports only.
void count_tiles(const ea::FwdParams& p, int cfg, int64_t* tiles, int64_t* masked) {
  const int bm = ea::tile_bm(cfg), bn = ea::tile_bn();
  int64_t t_all = 0, t_mask = 0;
  for (int t = 0; t < p.q_tiles; ++t) {
    const int q0 = t * bm;
    const int qlast = std::min(q0 + bm, p.n) - 1;
    int lo = p.wl >= 0 ? std::max(0, q0 - p.wl) : 0;
    int hi = p.n;
    if (p.causal) hi = std::min(hi, qlast + 1);
    if (p.wr >= 0) hi = std::min(hi, qlast + p.wr + 1);
    hi = std::max(lo, hi);
    for (int kt = lo / bn; kt < (hi + bn - 1) / bn; ++kt) {
      const int k0 = kt * bn, k1 = k0 + bn;
      bool full = k1 <= p.n;
      if (p.causal && k1 - 1 > q0) full = false;
      if (p.wl >= 0 && k0 < qlast - p.wl) full = false;
      if (p.wr >= 0 && k1 - 1 > q0 + p.wr) full = false;
      ++t_all;
      if (!full) ++t_mask;
    }
  }
  const int64_t bh = (int64_t)p.batch * p.heads;
  *tiles = t_all * bh;
  *masked = t_mask * bh;
}

// Workspace bytes for the bf16 copy of V that fp8 inputs with bf16 P.V read
// when the caller's workspace holds it (0: no such copy for this call).  The
// copy's rows are 256 bytes, so it is offered only while a head's rows stay
// below 2^31 bytes, as the kernels' 32-bit row offsets need.
int64_t wanted_v_copy(const ea_attn_args* a, int cfg) {
  if (a->in_dtype != EA_FP8_E4M3 || cfg != 0 || a->seqlen_k >= ((int64_t)1 << 23)) return 0;
  return ea::widened_v_bytes(a->batch * a->nheads_k, a->seqlen_k, (int)a->headdim);
}

// Key chunks per query tile this call would use with a large enough workspace,
// and the workspace that takes.
int wanted_splits(const ea::FwdParams& p, int cfg, int d, int64_t* bytes) {
  if (ea::key_streams(cfg) > 1) {   // the streams split the keys within the workgroup
    *bytes = 0;
    return 1;
  }
  int64_t total = 0, masked = 0;
  count_tiles(p, cfg, &total, &masked);
  const int s = ea::choose_splits((int64_t)p.q_tiles * p.batch * p.heads, max_kv_tiles(p, cfg), total);
  *bytes = ea::split_workspace_bytes(s, (int64_t)p.batch * p.heads, p.n, d);
  return s;
}

}  // namespace

extern "C" {

int ea_attn_fwd(const ea_attn_args* args, void* stream) {
  bool empty = false;
  const int st = validate(args, &empty);
  if (st != EA_OK || empty) return st;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return EA_EHIP;
  }
  if (!device_is_gfx950(dev)) return EA_EDEVICE;
  const int cfg = choose_cfg(args);
  ea::FwdParams p = make_params(args, cfg);
  int64_t need = 0, have = 0;
  const int splits = wanted_splits(p, cfg, (int)args->headdim, &need);
  const int64_t vcopy = wanted_v_copy(args, cfg);
  unsigned char* ws = (unsigned char*)workspace_of(args, &have);
  // The workspace holds [V copy | split partials]; a smaller one serves the
  // split first (it decides how well a few-tile launch fills the GPU), then
  // the copy.  Neither changes which values are computed: the copy is exact,
  // the split only reorders the sums.
  if (ws != nullptr) {
    const bool split = splits > 1 && have >= need;
    const bool copy = vcopy > 0 && have >= vcopy + (split ? need : 0);
    if (copy) p.v_wide = ws;
    if (split) {
      p.splits = splits;
      p.part_o = (float*)(ws + (copy ? vcopy : 0));
      p.part_lse = p.part_o + (int64_t)splits * p.batch * p.heads * p.n * args->headdim;
    }
  }
  e = ea::launch_fwd(p, args->in_dtype, (int)args->headdim, cfg, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return EA_EHIP;
  }
  return EA_OK;
}

int ea_attn_fwd_noalloc(const ea_attn_args* args, void* stream) {
  bool empty = false;
  const int st = validate(args, &empty);
  if (st != EA_OK || empty) return st;
  if (args->struct_size >= kArgsV2Size && args->workspace != nullptr) return EA_EINVAL;
  const int cfg = choose_cfg(args);
  ea::FwdParams p = make_params(args, cfg);
  int64_t need = 0;
  const int splits = wanted_splits(p, cfg, (int)args->headdim, &need);
  if (need > ea::kScratchBytes) return EA_ESCRATCH;   // before any device call
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return EA_EHIP;
  }
  if (!device_is_gfx950(dev)) return EA_EDEVICE;
  if (splits > 1) {
    void* scratch = nullptr;
    e = ea::scratch_address(dev, &scratch);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return EA_EHIP;
    }
    p.splits = splits;
    p.part_o = (float*)scratch;
    p.part_lse = p.part_o + (int64_t)splits * p.batch * p.heads * p.n * args->headdim;
  }
  e = ea::launch_fwd(p, args->in_dtype, (int)args->headdim, cfg, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return EA_EHIP;
  }
  return EA_OK;
}

int ea_attn_bwd(const ea_attn_bwd_args* args, void* stream) {
  bool empty = false;
  const int st = validate_bwd(args, &empty);
  if (st != EA_OK || empty) return st;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return EA_EHIP;
  }
  if (!device_is_gfx950(dev)) return EA_EDEVICE;
  const ea::BwdParams p = make_bwd_params(args);
  e = ea::launch_bwd(p, args->dtype, (int)args->headdim, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return EA_EHIP;
  }
  return EA_OK;
}

int ea_attn_plan(const ea_attn_args* args, ea_attn_plan_info* info) {
  if (info == nullptr || info->struct_size < kPlanV1Size) return EA_EINVAL;
  bool empty = false;
  const int st = validate(args, &empty);
  if (st != EA_OK) return st;
  const uint32_t sz = info->struct_size;
  const bool v2 = sz >= sizeof(ea_attn_plan_info);
  std::memset(info, 0, v2 ? sizeof(ea_attn_plan_info) : kPlanV1Size);
  info->struct_size = sz;
  const int cfg = choose_cfg(args);
  info->block_m = ea::tile_bm(cfg);
  info->block_n = ea::tile_bn();
  info->waves = ea::tile_waves(cfg);
  info->lds_bytes = ea::lds_bytes(args->in_dtype, (int)args->headdim, cfg);
  std::strncpy(info->kernel, ea::kernel_name(args->in_dtype, (int)args->headdim, cfg), sizeof(info->kernel) - 1);
  if (empty) return EA_OK;
  const ea::FwdParams p = make_params(args, cfg);
  info->grid = (int64_t)p.q_tiles * p.batch * p.heads;
  count_tiles(p, cfg, &info->kv_tiles, &info->masked_tiles);
  if (v2) {
    int64_t need = 0;
    info->splits = wanted_splits(p, cfg, (int)args->headdim, &need);
    info->workspace_bytes = wanted_v_copy(args, cfg) + need;
  }
  return EA_OK;
}

const char* ea_status_string(int status) {
  switch (status) {
    case EA_OK: return "ok";
    case EA_EINVAL: return "invalid argument";
    case EA_EUNSUPPORTED: return "unsupported argument combination";
    case EA_EDEVICE: return "current device is not gfx950";
    case EA_EHIP: return "HIP runtime error";
    case EA_ESCRATCH: return "the key split needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int ea_last_hip_error(void) { return g_last_hip_error; }

uint32_t ea_abi_version(void) { return EA_ABI_VERSION; }

}  // extern "C"
