// Host-side planning of the attention launches: tile configurations, the key
// split and kernel names.  No device code; the kernels' launch functions are
// in fwd_kernel.hip and bwd_kernel.hip.
#include <algorithm>
#include <cstdint>

#include "bwd_kernel.h"
#include "fwd_kernel.h"
#include "tiles.h"

namespace ea {

// Kernel configurations: 128 query rows per workgroup (4 waves x 32 rows,
// two workgroups per CU), 64 keys per K/V tile; configuration 1 (fp8 inputs
// only) runs P.V on the e4m3 matrix instruction.
int tile_bm(int /*cfg*/) { return 128; }

// Key split.  Measured on gfx950: a split pays for its merge kernel (a few
// microseconds) only where the query tiles' work is unbalanced (causal or
// windowed masks), by cutting the heaviest tiles; on balanced launches it
// costs.  So: no split when the items fill two workgroups per CU on the 256
// CUs, or when the heaviest tile sees fewer than 1.5x the average key tiles;
// otherwise enough chunks to bring the heaviest tile to about the average,
// within the GPU's two-per-CU capacity, with at least two key tiles per chunk
// and at most 16 chunks.
int choose_splits(int64_t items, int max_kv_tiles, int64_t total_kv_tiles) {
  constexpr int64_t kResident = 2 * 256;
  if (items <= 0 || items >= kResident || total_kv_tiles <= 0) return 1;
  if (2 * (int64_t)max_kv_tiles * items < 3 * total_kv_tiles) return 1;   // balanced
  int64_t s = ((int64_t)max_kv_tiles * items + total_kv_tiles - 1) / total_kv_tiles;
  s = std::min<int64_t>(s, (kResident + items - 1) / items);
  s = std::min<int64_t>(s, max_kv_tiles / 2);
  s = std::min<int64_t>(s, 16);
  return (int)std::max<int64_t>(s, 1);
}

int64_t split_workspace_bytes(int splits, int64_t batch_heads, int64_t n, int d) {
  return splits > 1 ? (int64_t)splits * batch_heads * n * (d + 1) * 4 : 0;
}
int tile_waves(int /*cfg*/) { return 4; }
int tile_bn() { return kBN; }

int lds_bytes(int in_dtype, int d, int cfg) {
  const bool fp8 = in_dtype == 3;
  const int kin = fp8 ? 1 : 2;
  return 2 * (kBN * d * kin + kBN * d * (cfg == 1 ? 1 : 2));
}

const char* kernel_name(int in_dtype, int d, int cfg) {
  static const char* names[3][2] = {{"attn_fwd<f16,d64,bm128,bn64>", "attn_fwd<f16,d128,bm128,bn64>"},
                                    {"attn_fwd<bf16,d64,bm128,bn64>", "attn_fwd<bf16,d128,bm128,bn64>"},
                                    {"none", "attn_fwd<fp8,d128,bm128,bn64>"}};
  if (cfg == 1) return (in_dtype == 3 && d == 128) ? "attn_fwd<fp8,pv8,d128,bm128,bn64>" : "none";
  if (in_dtype < 1 || in_dtype > 3 || (d != 64 && d != 128)) return "none";
  return names[in_dtype - 1][d == 128];
}

const char* bwd_kernel_names(int in_dtype, int d) {
  static const char* names[2][2] = {{"attn_bwd<f16,d64>", "attn_bwd<f16,d128>"}, {"attn_bwd<bf16,d64>", "attn_bwd<bf16,d128>"}};
  if (in_dtype < 1 || in_dtype > 2 || (d != 64 && d != 128)) return "none";
  return names[in_dtype - 1][d == 128];
}

}  // namespace ea
