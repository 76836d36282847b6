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
  // key chunks per query tile (1: no split); with more, the chunks' partial
  // results go to part_o [splits][B H][N][D] and part_lse [splits][B H][N]
  // (fp32) and a second kernel merges them
  int splits;
  float* part_o;
  float* part_lse;
};

// Split of the keys for a launch of `items` query tiles x heads whose tiles
// see at most `max_kv_tiles` key tiles and `total_kv_tiles` over all items:
// 1 when the items already fill the GPU or their work is balanced.
int choose_splits(int64_t items, int max_kv_tiles, int64_t total_kv_tiles);
// Workspace bytes for `splits` chunks (0 for one).
int64_t split_workspace_bytes(int splits, int64_t batch_heads, int64_t n, int d);

// Kernel configurations, both 128 query rows per workgroup (4 waves of 32
// rows, two waves per SIMD) and 64 keys per K/V tile: 0, P.V in 16 bits
// (fp8 V widened exactly to bf16); 1 (fp8 inputs only), P and V in e4m3 on
// the 8-bit matrix instruction.
int tile_bm(int cfg);
int tile_waves(int cfg);
int tile_bn();
int lds_bytes(int in_dtype, int d, int cfg);
const char* kernel_name(int in_dtype, int d, int cfg);
hipError_t launch_fwd(const FwdParams& p, int in_dtype, int d, int cfg, hipStream_t stream);

}  // namespace ea
