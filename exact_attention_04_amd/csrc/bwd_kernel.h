// Internal interface between the C ABI layer and the backward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea {

// Arguments of the backward kernels, already validated by the ABI layer.
// Strides are in elements; every tensor's head dimension is contiguous.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;      // [B, H, N] from the forward (natural log)
  float* delta;          // [B, H, N], written: dO_i . O_i
  void* dq;
  void* dk;
  void* dv;
  int batch, heads, heads_kv, group, n;
  int q_tiles;           // query tiles of 128 rows (dQ kernel)
  int k_blocks;          // key blocks of 128 rows (dK/dV kernel)
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t do_sb, do_ss, do_sh;
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dk_sb, dk_ss, dk_sh;
  int64_t dv_sb, dv_ss, dv_sh;
  int64_t lse_sb, lse_sh;
  int64_t delta_sb, delta_sh;
  int causal, wl, wr;
  float scale;           // softmax scale
  float c_log2;          // scale * log2(e)
};

// in_dtype: 1 = f16, 2 = bf16; d: 64 or 128.  Launches the dQ kernel (which
// also writes delta) and then the dK/dV kernel on `stream`.
hipError_t launch_bwd(const BwdParams& p, int in_dtype, int d, hipStream_t stream);
const char* bwd_kernel_names(int in_dtype, int d);

}  // namespace ea
