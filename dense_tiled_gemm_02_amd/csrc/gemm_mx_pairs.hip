// Variant table of the block-scaled tile kernel (gemm_mx_kernel.h) for the
// pairs the one-width table leaves out: every pair with an FP6 operand (E2M3,
// E3M2) and the pairs of an 8-bit with a 4-bit operand, each operand staged
// in rows of its own width (128 k per K step).  Tiles: 256 x 256 (8 waves, 2
// or 3 stages), 128 x 128 (4 waves, 3 stages), 64 x 64 (4 waves, 3 stages)
// and the decode regime's 32 x 64 slab (2 waves, 4 stages).
#include "gemm_mx_kernel.h"

namespace dtg {
namespace {

// the 20 pairs outside the one-width table, A's format first
#define MX_PAIRS(BM, BN, WM, WN, ST)                                                                            \
    MX_ENTRY(BM, BN, WM, WN, ST, 0, 2), MX_ENTRY(BM, BN, WM, WN, ST, 0, 3), MX_ENTRY(BM, BN, WM, WN, ST, 0, 4),   \
    MX_ENTRY(BM, BN, WM, WN, ST, 1, 2), MX_ENTRY(BM, BN, WM, WN, ST, 1, 3), MX_ENTRY(BM, BN, WM, WN, ST, 1, 4),   \
    MX_ENTRY(BM, BN, WM, WN, ST, 2, 0), MX_ENTRY(BM, BN, WM, WN, ST, 2, 1), MX_ENTRY(BM, BN, WM, WN, ST, 2, 2),   \
    MX_ENTRY(BM, BN, WM, WN, ST, 2, 3), MX_ENTRY(BM, BN, WM, WN, ST, 2, 4), MX_ENTRY(BM, BN, WM, WN, ST, 3, 0),   \
    MX_ENTRY(BM, BN, WM, WN, ST, 3, 1), MX_ENTRY(BM, BN, WM, WN, ST, 3, 2), MX_ENTRY(BM, BN, WM, WN, ST, 3, 3),   \
    MX_ENTRY(BM, BN, WM, WN, ST, 3, 4), MX_ENTRY(BM, BN, WM, WN, ST, 4, 0), MX_ENTRY(BM, BN, WM, WN, ST, 4, 1),   \
    MX_ENTRY(BM, BN, WM, WN, ST, 4, 2), MX_ENTRY(BM, BN, WM, WN, ST, 4, 3)

// 256 x 256 with a 3-deep ring where three stages fit the LDS beside the
// scales (rows of at most 12 bits of element per k: FP6 with FP6 or FP4, 8-bit
// with FP4): FP6 E2M3 4096^3 63.6 -> 61.7 us, E4M3 x E2M1 61.9 -> 60.6 us
// (interleaved, one box), the same bits.  Listed first, so the planner takes
// them for these pairs.
#define MX_DEEP(FA, FB) MX_ENTRY(256, 256, 2, 4, 3, FA, FB)

const MxEntry kMxPairTable[] = {
    MX_DEEP(2, 2), MX_DEEP(2, 3), MX_DEEP(3, 2), MX_DEEP(3, 3), MX_DEEP(2, 4), MX_DEEP(3, 4),
    MX_DEEP(4, 2), MX_DEEP(4, 3), MX_DEEP(0, 4), MX_DEEP(1, 4), MX_DEEP(4, 0), MX_DEEP(4, 1),
    MX_PAIRS(256, 256, 2, 4, 2),
    MX_PAIRS(128, 128, 2, 2, 3),
    MX_PAIRS(64, 64, 2, 2, 3),
    MX_PAIRS(32, 64, 1, 2, 4),
};

}  // namespace

const MxEntry* mx_pair_kernel_table(int* count) {
    *count = static_cast<int>(sizeof(kMxPairTable) / sizeof(kMxPairTable[0]));
    return kMxPairTable;
}

}  // namespace dtg
