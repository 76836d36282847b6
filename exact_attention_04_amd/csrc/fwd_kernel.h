// Internal interface between the C ABI layer and the forward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea {

// Kernel arguments, already validated and converted by the ABI layer.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;            // may be null
  int batch, heads, n, q_tiles;
  int group;             // query heads per K/V head (query head h reads K/V head h / group)
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t lse_sb, lse_sh;
  int causal, wl, wr;
  float c_log2;          // softmax_scale * q_descale * k_descale * log2(e)
  float v_descale;
};

// Tile configuration 0 (the only one): 128 query rows per workgroup (4 waves
// of 32 rows, two waves per SIMD), 64 keys per K/V tile.
int tile_bm(int cfg);
int tile_waves(int cfg);
int tile_bn();
int lds_bytes(int in_dtype, int d);
const char* kernel_name(int in_dtype, int d, int cfg);
hipError_t launch_fwd(const FwdParams& p, int in_dtype, int d, int cfg, hipStream_t stream);

}  // namespace ea
