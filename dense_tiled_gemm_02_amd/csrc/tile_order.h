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

// Stream-K schedule ("Hopper Support in Triton", the SplitK / stream-K
// slides).  The T x nkt iterations (output tile in grouped order, K step)
// are dealt out to W workgroups as W contiguous ranges: range w is
// [floor(w T nkt / W), floor((w + 1) T nkt / W)).  A range covers the tail
// of one tile, whole tiles and the head of another; each such piece is run
// by the tile body over its K steps.  A tile cut by range starts is summed by
// the K-slice exchange from its parts, numbered from the tile's first K step:
// part 0 belongs to the range that holds that step, part j to the j-th range
// that starts inside the tile.  With every range non-empty (W <= T nkt), the
// number of ranges starting at or before iteration s is
// ceil((s + 1) W / (T nkt)), which gives a part's number and a tile's part
// count without a search.  A range publishes at most one part 0 (its last
// piece) and one part j >= 1 (its first piece): to slots W + w and w of
// 2 W.  32-bit arithmetic: callers keep T nkt W below 2^31.
struct SkPiece {
    uint32_t tile, kt0, kt1;   // K steps [kt0, kt1) of output tile `tile`
    uint32_t part, nparts;     // part `part` of the tile's `nparts` (1: the whole tile)
    uint32_t slot0, slot1;     // workspace slot of part 0, and slot1 + j of part j >= 1
    uint32_t next;             // first iteration after this piece
};

__host__ __device__ inline uint32_t sk_range_start(uint32_t w, uint32_t total, uint32_t W) {
    return w * total / W;
}

// The piece that starts at iteration `it` of a range ending at `end`.
__host__ __device__ inline SkPiece sk_piece(uint32_t it, uint32_t end, uint32_t total, uint32_t nkt, uint32_t W) {
    auto starts_upto = [&](uint32_t s) { return ((s + 1) * W + total - 1) / total; };
    SkPiece q;
    q.tile = it / nkt;
    const uint32_t t0 = q.tile * nkt;
    const uint32_t stop = (end < t0 + nkt) ? end : t0 + nkt;
    const uint32_t c0 = starts_upto(t0);
    q.kt0 = it - t0;
    q.kt1 = stop - t0;
    q.part = starts_upto(it) - c0;
    q.nparts = starts_upto(t0 + nkt - 1) - c0 + 1;
    q.slot0 = W + c0 - 1;   // the last piece of range c0 - 1
    q.slot1 = c0 - 1;       // part j: the first piece of range c0 - 1 + j
    q.next = stop;
    return q;
}

template <typename I>
__host__ __device__ inline void tile_of_workgroup(I wg, I num_pid_m, I num_pid_n, I group_m,
                                                  I xcds, I* pid_m, I* pid_n) {
    const I grid = num_pid_m * num_pid_n;
    grouped_tile<I>(xcd_permute<I>(wg, grid, xcds), num_pid_m, num_pid_n, group_m, pid_m, pid_n);
}

}  // namespace dtg
