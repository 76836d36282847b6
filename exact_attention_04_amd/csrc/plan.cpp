// Host-side planning of the attention launches: tile configurations, the key
// split and kernel names.  No device code; the kernels' launch functions are
// in fwd_kernel.hip and bwd_kernel.hip.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "bwd_kernel.h"
#include "fwd_kernel.h"
#include "tiles.h"

namespace ea {

// Kernel configurations.  Each wave owns 32 query rows and K/V tiles hold 64
// keys.  A configuration is (row waves per key stream, key streams):
//   0: 4 x 1 -- 128 rows, two workgroups per CU (two waves per SIMD);
//   1: 4 x 1 with the e4m3 P.V (fp8 inputs only);
//   2: 4 x 2 -- 128 rows, two key streams: 8 waves, one workgroup per CU;
//   3: 1 x 4 -- 32 rows, four key streams: 4 waves (d = 64 only: four
//      streams' slots fit a CU's LDS at d = 64);
//   4: 2 x 2 -- 64 rows, two key streams: 4 waves, two workgroups per CU
//      (d = 64 only).
// Streams split a workgroup's key tiles among themselves and merge in LDS.
// Measured on one MI355X (median kernel time, fp16 d = 64):
//   B1 H8 N512:           config 0 14.6 us, 2 13.7, 3 10.8 (64 rows x 4: 11.7)
//   B2 H8 N2048:          config 0 38.0 us, 2 31.1, 3 59.8 (64 rows x 4: 38.6)
//   B2 H8 N2048 causal:   config 0 (key split) 33.1 us, 2 28.7, 3 44.3
//                         (64 rows x 4: 27.6)
// and, in alternated runs on another box, config 4 against the choice above:
//   B1 H8 N512 11.3 us against 10.7 (config 3); B2 H8 N2048 30.8 against 30.8
//   (config 2); B2 H8 N2048 causal 24.6 against 27.7 (config 2).
namespace {
struct Shape {
  int row_waves, streams;
};
Shape shape_of(int cfg) {
  switch (cfg) {
    case 2: return {4, 2};
    case 3: return {1, 4};
    case 4: return {2, 2};
    default: return {4, 1};
  }
}
}  // namespace

int tile_bm(int cfg) { return 32 * shape_of(cfg).row_waves; }
int key_streams(int cfg) { return shape_of(cfg).streams; }

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

int64_t widened_v_bytes(int64_t batch_heads_kv, int64_t n, int d) {
  return (batch_heads_kv * n * d * 2 + 255) / 256 * 256;
}
int tile_waves(int cfg) { return shape_of(cfg).row_waves * shape_of(cfg).streams; }
int tile_bn() { return kBN; }

int lds_bytes(int in_dtype, int d, int cfg) {
  const bool fp8 = in_dtype == 3;
  const int kin = fp8 ? 1 : 2;
  const Shape sh = shape_of(cfg);
  // per stream: two K slots and two V slots; with streams, each row's maximum
  // and sum per stream for the merge
  const int slots = 2 * (kBN * d * kin + kBN * d * (cfg == 1 ? 1 : 2));
  return sh.streams * slots + (sh.streams > 1 ? sh.streams * sh.row_waves * 2 * 32 * 4 : 0);
}

const char* kernel_name(int in_dtype, int d, int cfg) {
  static char names[8][2][3][48];   // filled once; cfg < 8, d in {64, 128}, dtype 1..3
  static std::once_flag once;
  std::call_once(once, [] {
    const char* ty[3] = {"f16", "bf16", "fp8"};
    for (int c = 0; c < 8; ++c)
      for (int di = 0; di < 2; ++di)
        for (int t = 0; t < 3; ++t) {
          const Shape sh = shape_of(c);
          std::snprintf(names[c][di][t], sizeof(names[c][di][t]), "attn_fwd<%s,%sd%d,bm%d,bn%d%s>", ty[t],
                        c == 1 ? "pv8," : "", di ? 128 : 64, 32 * sh.row_waves, kBN,
                        sh.streams > 1 ? (sh.streams == 2 ? ",ks2" : ",ks4") : "");
        }
  });
  if (in_dtype < 1 || in_dtype > 3 || (d != 64 && d != 128) || cfg < 0 || cfg > 4) return "none";
  if (in_dtype == 3 && (d != 128 || cfg > 1)) return "none";
  if (in_dtype != 3 && (cfg == 1 || (cfg > 2 && d != 64))) return "none";
  return names[cfg][d == 128][in_dtype - 1];
}

const char* bwd_kernel_names(int in_dtype, int d) {
  static const char* names[2][2] = {{"attn_bwd<f16,d64>", "attn_bwd<f16,d128>"}, {"attn_bwd<bf16,d64>", "attn_bwd<bf16,d128>"}};
  if (in_dtype < 1 || in_dtype > 2 || (d != 64 && d != 128)) return "none";
  return names[in_dtype - 1][d == 128];
}

}  // namespace ea
