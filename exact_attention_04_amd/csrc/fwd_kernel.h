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
  // fp8 inputs with P.V in bf16: null, or a [B][Hk][N][D] bf16 buffer that a
  // first kernel fills with V widened exactly to bf16, which the attention
  // kernel then loads as it loads 16-bit V (null: each workgroup widens the V
  // tiles it loads, through registers)
  void* v_wide;
};

// Split of the keys for a launch of `items` query tiles x heads whose tiles
// see at most `max_kv_tiles` key tiles and `total_kv_tiles` over all items:
// 1 when the items already fill the GPU or their work is balanced.
int choose_splits(int64_t items, int max_kv_tiles, int64_t total_kv_tiles);
// Workspace bytes for `splits` chunks (0 for one).
int64_t split_workspace_bytes(int splits, int64_t batch_heads, int64_t n, int d);
// Bytes of the widened bf16 copy of an fp8 V (FwdParams::v_wide), rounded up
// to 256 so that what follows it in a workspace stays aligned.
int64_t widened_v_bytes(int64_t batch_heads_kv, int64_t n, int d);

// The allocation-free entry point's scratch: a static device array of
// kScratchBytes per GPU holding the key split's partial results (in place of
// a caller's workspace).  scratch_address() returns its device address on
// device `dev`, which must be the current device; the lookup runs once per
// device and its result (or error) is kept.
constexpr int64_t kScratchBytes = (int64_t)32 << 20;
hipError_t scratch_address(int dev, void** ptr);

// Kernel configurations (64 keys per K/V tile, 32 query rows per wave):
//   0: 128 rows per workgroup (4 waves), P.V in 16 bits (fp8 V widened
//      exactly to bf16, by a first kernel into FwdParams::v_wide when that
//      is set, else per tile in the attention kernel); two workgroups per
//      CU, two waves per SIMD;
//   1: as 0 for fp8 inputs with P and V in e4m3 on the 8-bit instruction;
//   2, 3 (16-bit inputs): the workgroup's waves form key streams that split
//      the key tiles and merge in LDS, for launches with few query tiles:
//      2 streams of 4 row waves (128 rows), or 4 streams of 1 (32 rows,
//      d = 64 only).
// tile_bm: query rows per workgroup; key_streams: streams; tile_waves: all
// waves of the workgroup.
int tile_bm(int cfg);
int key_streams(int cfg);
int tile_waves(int cfg);
int tile_bn();
int lds_bytes(int in_dtype, int d, int cfg);
const char* kernel_name(int in_dtype, int d, int cfg);
hipError_t launch_fwd(const FwdParams& p, int in_dtype, int d, int cfg, hipStream_t stream);

}  // namespace ea
