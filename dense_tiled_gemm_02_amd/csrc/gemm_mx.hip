// Variant table of the block-scaled tile kernel (gemm_mx_kernel.h) for the
// pairs of one element width: E4M3 and E5M2 in any combination, E2M1 with
// E2M1.
#include "gemm_mx_kernel.h"

namespace dtg {
namespace {

#define MX_FORMATS(BM, BN, WM, WN, ST)                                                                       \
    MX_ENTRY(BM, BN, WM, WN, ST, 0, 0), MX_ENTRY(BM, BN, WM, WN, ST, 1, 1), MX_ENTRY(BM, BN, WM, WN, ST, 0, 1), \
    MX_ENTRY(BM, BN, WM, WN, ST, 1, 0), MX_ENTRY(BM, BN, WM, WN, ST, 4, 4)

const MxEntry kMxTable[] = {
    MX_FORMATS(256, 256, 2, 4, 2),
    MX_FORMATS(256, 128, 4, 2, 3),
    MX_FORMATS(128, 256, 2, 4, 3),
    MX_FORMATS(128, 128, 2, 2, 3),
    MX_FORMATS(64, 64, 2, 2, 3),
    MX_FORMATS(192, 256, 2, 4, 2),
    // decode regime: 32 x 64 slabs of two waves, a 4-deep ring, K slices
    // across workgroups
    MX_FORMATS(32, 64, 1, 2, 4),
};

}  // namespace

const MxEntry* mx_kernel_table(int* count) {
    *count = static_cast<int>(sizeof(kMxTable) / sizeof(kMxTable[0]));
    return kMxTable;
}

}  // namespace dtg
