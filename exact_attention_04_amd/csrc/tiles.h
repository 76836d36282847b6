// Tile constants shared by the kernels and the host-side planner.
#pragma once

namespace ea {

constexpr int kBN = 64;            // keys per K/V tile

}  // namespace ea
