// Output-tile order of a launch: which (pid_m, pid_n) tile workgroup `wg`
// computes.  Shared by the kernels (device) and the planner/ABI (host), so the
// host-side export tests exactly what the kernels run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dtg {

// Workgroups of one launch are handed to the accelerator dies (XCDs) round
// robin: workgroup wg runs on XCD wg % xcds.  This permutation renumbers them
// so that XCD x receives one contiguous range of tile-order positions; with
// the grouped order below, a contiguous range is a band of M tiles sharing
// the same B panels, which then stay in that XCD's own L2.  A bijection on
// [0, grid) for any grid (the first grid % xcds dies get one extra position).
template <typename I>
__host__ __device__ inline I xcd_permute(I wg, I grid, I xcds) {
    if (xcds <= 1) return wg;
    const I per = grid / xcds, rem = grid % xcds;
    const I x = wg % xcds, local = wg / xcds;
    return x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
}

// Grouped tile order (FlagGems "Hygon optimization", section "Grouped
// scheduling: improve L2 data reuse").  Definition: the M tiles form bands of
// group_m consecutive rows of tiles (the last band holds what is left); the
// order visits the bands top to bottom, and inside a band it takes the N tiles
// left to right, for each one every row of the band top to bottom, so
// consecutive workgroups share one K x N panel of B.  Position pos lies in
// band pos / (group_m * num_pid_n) (every band before the last is full);
// inside it, its offset counts whole columns of the band's height first.
// group_m = 1 is plain row-major order.
template <typename I>
__host__ __device__ inline void grouped_tile(I pos, I num_pid_m, I num_pid_n, I group_m,
                                             I* pid_m, I* pid_n) {
    const I full_band = group_m * num_pid_n;          // positions in a band of group_m rows
    const I band = pos / full_band;
    const I top = band * group_m;                     // first M tile of the band
    const I height = (num_pid_m - top < group_m) ? num_pid_m - top : group_m;
    const I off = pos - band * full_band;             // position inside the band
    *pid_n = off / height;                            // a column of the band per `height` positions
    *pid_m = top + off % height;
}

template <typename I>
__host__ __device__ inline void tile_of_workgroup(I wg, I num_pid_m, I num_pid_n, I group_m,
                                                  I xcds, I* pid_m, I* pid_n) {
    const I grid = num_pid_m * num_pid_n;
    grouped_tile<I>(xcd_permute<I>(wg, grid, xcds), num_pid_m, num_pid_n, group_m, pid_m, pid_n);
}

}  // namespace dtg
