// mmq_tiles.h -- how the MMQ kernels map workgroups to output tiles on the
// eight XCDs of a gfx950 device (each XCD has its own L2).
#ifndef MMQ_TILES_H
#define MMQ_TILES_H

#include <hip/hip_runtime.h>

namespace q4mi {

// Map the linear workgroup id so that the 8 XCDs (which receive workgroups
// round-robin) each own a contiguous run of tiles.
__device__ __forceinline__ int xcd_tile(int pid, int ntiles)
{
    constexpr int kXcd = 8;
    const int per = ntiles / kXcd, rem = ntiles % kXcd;
    const int xcd = pid % kXcd, local = pid / kXcd;
    // the first rem XCDs own per + 1 tiles, the others per
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Tile t of a tiles_m x tiles_n grid (activation-row tiles x weight-row
// tiles) in groups of gm = ceil(tiles_m / 8) activation-row tiles, the m
// index running fastest within a group: one XCD's contiguous run of t then
// covers about gm activation-row tiles, its concurrent workgroups share both
// their activation and weight tiles in its L2, and each XCD reads every
// weight tile once.
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, int &mt, int &nt)
{
    const int gm = (tiles_m + 7) / 8;
    const int g = t / (gm * tiles_n), r = t - g * (gm * tiles_n);
    const int rows = min(gm, tiles_m - g * gm);
    mt = g * gm + r % rows;
    nt = r / rows;
}

}  // namespace q4mi

#endif
