// Block -> output-tile mapping shared by the GEMM kernels.
#pragma once

#include <stdint.h>

namespace cfp32 {

constexpr int kXcds = 8;     // MI355X deals workgroups to its 8 XCDs round-robin
constexpr int kGroupM = 4;   // tile-rows per scheduling group

// Renumber block `bid` of `nbm x nbn` tiles so that the tiles one XCD runs are
// contiguous in the new order (XCD x gets the x-th contiguous share), then
// walk them in groups kGroupM tile-rows high, column by column.  Tiles that
// run together on one XCD then share A row-panels and W column-panels in
// that XCD's L2.  The mapping is a bijection onto [0, nbm) x [0, nbn).
__device__ __forceinline__ void tile_of_block(int64_t bid, int64_t nbm, int64_t nbn, int64_t &tile_m,
                                              int64_t &tile_n)
{
    const int64_t total = nbm * nbn;
    const int64_t q = total / kXcds, r = total % kXcds;
    const int64_t xcd = bid % kXcds, local = bid / kXcds;
    const int64_t b = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
    const int64_t span = (int64_t)kGroupM * nbn;
    const int64_t first_m = (b / span) * kGroupM;
    const int64_t gsize = (nbm - first_m) < kGroupM ? (nbm - first_m) : kGroupM;
    tile_m = first_m + (b % span) % gsize;
    tile_n = (b % span) / gsize;
}

}  // namespace cfp32
