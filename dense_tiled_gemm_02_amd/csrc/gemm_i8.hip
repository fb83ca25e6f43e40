// Variants of the tile kernel for 8-bit integer operands (gemm_dma_kernel.h,
// gemm_i8_kernel): int8 A (M x K) and B stored N x K, both k contiguous,
// int32 accumulation, C and D.  The planner's ladder tiles with the
// 16 x 16 x 64 instruction, and the 256 x 256 tile with 32 x 32 x 32 for the
// instruction-shape comparison.  BK counts 16-bit units: 64 is 128 k.
#include "gemm_dma_kernel.h"

namespace dtg {
namespace {

const KernelEntry kTable[] = {
    I8_ENTRY(256, 256, 64, 2, 4, 16, 2),
    I8_ENTRY(256, 256, 64, 2, 4, 32, 2),
    I8_ENTRY(256, 128, 64, 4, 2, 16, 3),
    I8_ENTRY(128, 256, 64, 2, 4, 16, 3),
    I8_ENTRY(128, 128, 64, 2, 4, 16, 4),
    I8_ENTRY(128, 128, 64, 2, 4, 16, 2),
    I8_ENTRY(64, 64, 64, 2, 2, 16, 4),
};

}  // namespace

const KernelEntry* i8_kernel_table(int* count) {
    *count = static_cast<int>(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace dtg
