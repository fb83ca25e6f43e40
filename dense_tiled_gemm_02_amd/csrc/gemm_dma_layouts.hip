// Variants of the direct-to-LDS GEMM kernel (gemm_dma_kernel.h), operands stored transposed (A as K x M, B as N x K, or both) for the planner's ladder tiles.
#include "gemm_dma_kernel.h"

namespace dtg {
namespace {

const KernelEntry kTable[] = {
    DMA_LAYOUTS(256, 256, 64, 2, 4, 16, 2),
    DMA_LAYOUTS(256, 128, 64, 4, 2, 16, 2),
    DMA_LAYOUTS(128, 256, 64, 2, 4, 16, 2),
    DMA_LAYOUTS(128, 128, 64, 2, 4, 16, 2),
    DMA_LAYOUTS(256, 128, 64, 4, 2, 16, 3),
    DMA_LAYOUTS(128, 256, 64, 2, 4, 16, 3),
    DMA_LAYOUTS(128, 128, 64, 2, 4, 16, 4),
    DMA_LAYOUTS(64, 64, 64, 2, 2, 16, 4),
};

}  // namespace

const KernelEntry* dma_kernel_table_layouts(int* count) {
    *count = static_cast<int>(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace dtg
