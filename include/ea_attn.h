/*
 * ea_attn.h -- C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * The operation is exact scaled-dot-product attention,
 *
 *     O = softmax(Q K^T * scale + mask) V,      LSE_i = ln sum_j exp(s_ij)
 *
 * the "standard attention" of the "Flash Attention | Hermes Skill" page
 * (Workflow 1, Step 2), computed with the IO-aware tiling its Quick start
 * names: tiles live on chip and the softmax is online (running max / running
 * sum), so the N x N score matrix never reaches HBM ("FlashAttention",
 * aiunderstanding.org, sections "Djupdykning" and "Teknisk insikt").  The
 * result equals the materialised definition up to floating-point rounding.
 *
 * Conventions shared by every call:
 *   - Pointers named q, k, v, o, lse are DEVICE pointers on the current HIP
 *     device.  The caller owns every buffer; the library allocates nothing,
 *     keeps no buffer, and never modifies q, k or v.
 *   - Strides are in ELEMENTS.  A tensor is addressed as
 *       base + b*stride_b + s*stride_s + h*stride_h + d      (d contiguous)
 *     which covers [batch, seqlen, nheads, headdim] ("bshd", the flash-attn
 *     layout of the pages' Workflow 2), [batch, heads, seq, dim] ("bhsd", the
 *     SDPA layout of the pages' Quick start) and transposed views of either,
 *     without copies.
 *   - Calls return an ea_status code and never abort, print or throw.
 *   - The library is thread-safe: apart from a once-initialised table of
 *     device properties it holds no mutable global state.
 */
#ifndef EA_ATTN_H
#define EA_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 5: the forward's workspace may also hold the bf16 copy of an fp8 V, and
   ea_attn_plan's workspace_bytes includes it (no struct changed). */
#define EA_ABI_VERSION 5u

/* Status codes. */
enum ea_status {
  EA_OK = 0,
  EA_EINVAL = 1,        /* malformed arguments: see ea_attn_fwd */
  EA_EUNSUPPORTED = 2,  /* well-formed but outside what the kernels implement */
  EA_EDEVICE = 3,       /* the current device is not a gfx950 GPU */
  EA_EHIP = 4,          /* a HIP runtime call failed; see ea_last_hip_error */
  EA_ESCRATCH = 5       /* ea_attn_fwd_noalloc: the launch needs more scratch
                           than the library's static buffer holds */
};

/* Element types. */
enum ea_dtype {
  EA_F16 = 1,           /* IEEE binary16 */
  EA_BF16 = 2,          /* bfloat16 */
  EA_FP8_E4M3 = 3,      /* OCP 8-bit float E4M3 ("fn": no infinities, max 448) */
  EA_F32 = 4            /* accepted by the enum only to be rejected: the pages
                           state that float32 inputs are not supported
                           ("Flash Attention | Hermes Skill", Common issues) */
};

/*
 * Arguments of one forward call.  struct_size is sizeof(ea_attn_args); the
 * sizes of the version-1 struct (everything before `workspace`) and of the
 * version-2 struct (everything before `pv_dtype`) are also accepted and mean
 * workspace == NULL and pv_dtype == 0 as far as they lack them.  The struct
 * may grow at its end in later ABI versions.
 */
typedef struct ea_attn_args {
  uint32_t struct_size;
  int32_t in_dtype;          /* ea_dtype of q, k, v: EA_F16, EA_BF16 or EA_FP8_E4M3 */
  int32_t out_dtype;         /* ea_dtype of o: same as in_dtype for 16-bit inputs,
                                EA_BF16 for EA_FP8_E4M3 inputs */
  int32_t causal;            /* nonzero: key j is visible from query i only if j <= i */
  int32_t window_left;       /* sliding window, inclusive: keys j with */
  int32_t window_right;      /*   i - window_left <= j <= i + window_right;
                                -1 on a side means unbounded on that side
                                (the pages' window_size=(left, right),
                                "Flash Attention | Hermes Skill", Workflow 2) */
  float softmax_scale;       /* finite and > 0; the pages' default is 1/sqrt(headdim) */
  float q_descale;           /* fp8 only: the stored value times the descale is the */
  float k_descale;           /*   real value (per-tensor scales); must be finite and */
  float v_descale;           /*   > 0, and exactly 1.0 for 16-bit inputs */
  int64_t batch;             /* B >= 0 */
  int64_t seqlen_q;          /* Nq >= 0 */
  int64_t seqlen_k;          /* Nk >= 0; this version requires Nq == Nk */
  int64_t nheads_q;          /* Hq >= 1 */
  int64_t nheads_k;          /* Hk >= 1 K/V heads; Hq must be a multiple of Hk.
                                With Hk < Hq the K/V heads are shared (multi-query
                                / grouped-query attention, "Flash Attention |
                                Hermes Skill", Workflow 2, Step 3): query head h
                                reads K/V head h / (Hq / Hk) */
  int64_t headdim;           /* D: 64 or 128 */
  const void* q;             /* [B, Nq, Hq, D] via the strides below */
  const void* k;             /* [B, Nk, Hk, D] */
  const void* v;             /* [B, Nk, Hk, D] (same strides rules as k) */
  void* o;                   /* [B, Nq, Hq, D], written in full */
  float* lse;                /* [B, Hq, Nq] float32, natural log of the scaled,
                                masked scores; NULL = do not write */
  int64_t q_stride_b, q_stride_s, q_stride_h;
  int64_t k_stride_b, k_stride_s, k_stride_h;
  int64_t v_stride_b, v_stride_s, v_stride_h;
  int64_t o_stride_b, o_stride_s, o_stride_h;
  int64_t lse_stride_b, lse_stride_h;   /* LSE rows are contiguous along Nq */
  /* Optional scratch (ea_attn_plan reports the bytes wanted, 0 if none),
     laid out as [V copy | split partials]:
     - fp8 inputs with P.V in bf16: a bf16 copy of V, B x Hk x Nk x D x 2
       bytes rounded up to 256, which a first kernel fills with V widened
       exactly to bf16; the attention kernel then loads V as for 16-bit
       inputs instead of widening each V tile it loads.  Results are
       bitwise the same with or without it.
     - launches with too few query tiles to fill the GPU: the keys of each
       tile are split into chunks whose partial results are merged by a
       second kernel (same results up to rounding).
     NULL runs with neither; fewer bytes than wanted serve the split first
     (when they hold its part), then the copy (when they hold it as well).
     Device memory, 16-byte aligned, owned by the caller; its contents need
     no initialisation and are overwritten; launches that may run at the same
     time need separate workspaces. */
  void* workspace;
  int64_t workspace_bytes;
  /* Number format of P and V in the P.V product, for fp8 inputs ("Flash
     Attention | Hermes Skill", FP8 section: forward attention on e4m3
     inputs; the pages leave the format of P open).  0 or EA_BF16: P rounded
     to bf16 and V widened exactly to bf16, on the 16-bit matrix instructions
     (the default).  EA_FP8_E4M3: P (times 2^3) rounded to e4m3 and V as
     stored, on the 8-bit matrix instructions; a K/V tile that adds more than
     1/8 of some query row's running sum also multiplies the e4m3 rounding
     residual of P, so P keeps about 8 bits there.  For 16-bit inputs: 0. */
  int32_t pv_dtype;
  int32_t reserved;          /* 0 */
} ea_attn_args;

/* What ea_attn_fwd would launch for a given argument set. */
typedef struct ea_attn_plan_info {
  uint32_t struct_size;      /* set by the caller to sizeof(ea_attn_plan_info); the
                                version-1 size (up to `kernel`) is accepted and
                                the fields after it are then not written */
  int32_t block_m;           /* query rows per workgroup */
  int32_t block_n;           /* keys per K/V tile */
  int32_t waves;             /* wavefronts per workgroup */
  int32_t lds_bytes;         /* LDS per workgroup */
  int64_t grid;              /* workgroups of the unsplit launch (the key split
                                launches `splits` times as many, then a merge) */
  int64_t kv_tiles;          /* K/V tiles visited over the whole launch */
  int64_t masked_tiles;      /* of which need per-element masking */
  char kernel[64];           /* name of the kernel instantiation */
  int64_t workspace_bytes;   /* ea_attn_args.workspace size that enables the key split
                                and, for fp8 inputs with bf16 P.V, the copy of V */
  int32_t splits;            /* key chunks per query tile with that workspace (1: none) */
  int32_t reserved;
} ea_attn_plan_info;

/*
 * ea_attn_fwd -- launch the attention forward on `stream` (a hipStream_t;
 * NULL is the default stream).  Asynchronous: returns once the kernel is
 * enqueued; no host synchronisation, no allocation.
 *
 * Checks its arguments and returns without launching anything on failure
 * (o and lse are then untouched); the first failing check decides the code:
 *   EA_EINVAL        args NULL or struct_size too small; a NULL q/k/v/o; a
 *                    negative size; Hq or Hk < 1; a bad dtype enum; a
 *                    non-finite softmax_scale; a descale that is not finite
 *                    and > 0, or != 1 for 16-bit inputs; window bounds < -1;
 *                    pv_dtype not 0, EA_BF16 or EA_FP8_E4M3, or reserved != 0;
 *                    o overlapping q, k or v; lse overlapping o, q, k or v;
 *                    a workspace overlapping any tensor.
 *   EA_EUNSUPPORTED  float32 inputs; headdim not 64 or 128 (fp8: not 128);
 *                    a nonzero pv_dtype with 16-bit inputs;
 *                    Nq != Nk; Hq not a multiple of Hk; softmax_scale <= 0; an output
 *                    dtype other than the one above; a negative stride; a
 *                    base pointer not 16-byte aligned or a b/s/h stride
 *                    whose byte size is not a multiple of 16 (the kernels
 *                    move 16-byte vectors); an lse pointer not 4-byte
 *                    aligned; an index that would overflow 32 bits
 *                    (|stride| * extent >= 2^31 elements).
 *   EA_EDEVICE       the current device is not gfx950.
 *   EA_EHIP          a HIP call or the launch failed.
 * B == 0 or Nq == 0 returns EA_OK without launching once the dtype, size,
 * scale, descale and window checks have passed (the pointers may be NULL).
 */
int ea_attn_fwd(const ea_attn_args* args, void* stream);

/*
 * ea_attn_fwd_noalloc -- ea_attn_fwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, results and checks as ea_attn_fwd, but
 * args->workspace must be NULL: a launch that splits its keys (the plan's
 * splits > 1) keeps the partial results in a static device array of the
 * library, 32 MiB per GPU, which each GPU the library runs on holds until the
 * process ends; fp8 inputs with bf16 P.V widen V per tile inside the kernel
 * (no copy of V).  Nothing is allocated, freed or copied by this call.
 *   EA_EINVAL        as ea_attn_fwd, and a non-NULL workspace.
 *   EA_ESCRATCH      the key split's partial results (the plan's
 *                    workspace_bytes less the fp8 V copy) exceed 32 MiB
 *                    (checked before any device call; ea_attn_fwd with a
 *                    caller workspace, or with none, runs such a problem).
 *   EA_EUNSUPPORTED, EA_EDEVICE, EA_EHIP   as ea_attn_fwd.
 * All calls on one GPU share that GPU's array, and it keeps the last call's
 * contents (every element a launch reads, it first writes, so nothing needs
 * clearing): launches that may overlap on one GPU (different streams, or
 * threads without ordering) race on it and must not be issued that way.
 */
int ea_attn_fwd_noalloc(const ea_attn_args* args, void* stream);

/*
 * ea_attn_plan -- fill *info with the tile configuration and grid that
 * ea_attn_fwd would use for *args.  Runs the same argument checks except the
 * device check, launches nothing and touches no device memory, so it works
 * without a GPU.  info->struct_size must be set by the caller.
 */
int ea_attn_plan(const ea_attn_args* args, ea_attn_plan_info* info);

/*
 * Arguments of one backward call: the gradients of a loss with respect to
 * q, k and v given its gradient dout with respect to the forward's output o.
 * The pages obtain them by recomputation ("Flash Attention | Hermes Skill",
 * Quick start: IO-aware tiling and recomputation; its FP8 section: the 16-bit
 * kernels run forward and backward, fp8 forward only).  With s the scaled,
 * masked scores and P_ij = exp(s_ij - lse_i), the chain rule through the
 * forward's definition gives
 *     dv = P^T dout,   dP = dout v^T,   delta_i = dout_i . o_i,
 *     dS = P o (dP - delta),   dq = scale dS k,   dk = scale dS^T q,
 * with a shared K/V head's gradients summed over the query heads that read it.
 * struct_size must be sizeof(ea_attn_bwd_args).
 */
typedef struct ea_attn_bwd_args {
  uint32_t struct_size;
  int32_t dtype;             /* EA_F16 or EA_BF16: q, k, v, o, dout, dq, dk, dv */
  int32_t causal;            /* mask, as in ea_attn_args */
  int32_t window_left;
  int32_t window_right;
  float softmax_scale;       /* finite and > 0, the forward's scale */
  int64_t batch;             /* B >= 0 */
  int64_t seqlen;            /* N >= 0 (queries and keys) */
  int64_t nheads_q;          /* Hq >= 1 */
  int64_t nheads_k;          /* Hk >= 1, Hq a multiple of Hk (shared K/V heads) */
  int64_t headdim;           /* D: 64 or 128 */
  const void* q;             /* [B, N, Hq, D] via the strides below (read) */
  const void* k;             /* [B, N, Hk, D] (read) */
  const void* v;             /* [B, N, Hk, D] (read) */
  const void* o;             /* [B, N, Hq, D] the forward's output (read) */
  const void* dout;          /* [B, N, Hq, D] gradient with respect to o (read) */
  const float* lse;          /* [B, Hq, N] the forward's log-sum-exp (read) */
  float* delta;              /* [B, Hq, N] written: dout_i . o_i in float32 */
  void* dq;                  /* [B, N, Hq, D] written in full */
  void* dk;                  /* [B, N, Hk, D] written in full */
  void* dv;                  /* [B, N, Hk, D] written in full */
  int64_t q_stride_b, q_stride_s, q_stride_h;
  int64_t k_stride_b, k_stride_s, k_stride_h;
  int64_t v_stride_b, v_stride_s, v_stride_h;
  int64_t o_stride_b, o_stride_s, o_stride_h;
  int64_t do_stride_b, do_stride_s, do_stride_h;
  int64_t dq_stride_b, dq_stride_s, dq_stride_h;
  int64_t dk_stride_b, dk_stride_s, dk_stride_h;
  int64_t dv_stride_b, dv_stride_s, dv_stride_h;
  int64_t lse_stride_b, lse_stride_h;       /* rows contiguous along N */
  int64_t delta_stride_b, delta_stride_h;   /* rows contiguous along N */
} ea_attn_bwd_args;

/*
 * ea_attn_bwd -- launch the backward on `stream` (a hipStream_t; NULL is the
 * default stream).  Asynchronous, no allocation: two kernels in stream order
 * (dq and delta, then dk and dv).  Results do not depend on the order in which
 * workgroups run (no atomics).  All pointers are device pointers owned by the
 * caller.
 *   EA_EINVAL        args NULL or struct_size too small; a NULL pointer; a
 *                    negative size; Hq or Hk < 1; a bad dtype enum; a
 *                    non-finite softmax_scale; window bounds < -1; an output
 *                    (dq, dk, dv, delta) overlapping an input or another
 *                    output.
 *   EA_EUNSUPPORTED  fp8 or float32 dtype; headdim not 64 or 128; Hq not a
 *                    multiple of Hk; softmax_scale <= 0; a negative stride; a
 *                    16-bit tensor's base not 16-byte aligned or a stride
 *                    whose byte size is not a multiple of 16; lse or delta not
 *                    4-byte aligned; an index that would overflow 32 bits.
 *   EA_EDEVICE       the current device is not gfx950.
 *   EA_EHIP          a launch failed.
 * B == 0 or N == 0 returns EA_OK without launching.
 */
int ea_attn_bwd(const ea_attn_bwd_args* args, void* stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char* ea_status_string(int status);

/* The hipError_t of the last EA_EHIP failure on the calling thread (0 if none). */
int ea_last_hip_error(void);

/* EA_ABI_VERSION of the built library. */
uint32_t ea_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EA_ATTN_H */
