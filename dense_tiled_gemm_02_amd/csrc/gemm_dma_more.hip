// Variants of the direct-to-LDS GEMM kernel (gemm_dma_kernel.h), more row-major tiles (smaller and 4-wave tiles, deeper rings).
#include "gemm_dma_kernel.h"

namespace dtg {
namespace {

const KernelEntry kTable[] = {
    DMA_BOTH(256, 128, 64, 2, 2, 16, 3),
    DMA_BOTH(256, 128, 64, 2, 2, 16, 2),
    DMA_BOTH(128, 256, 64, 2, 2, 16, 2),
    DMA_BOTH(128, 128, 64, 2, 2, 16, 2),
    DMA_BOTH(128, 128, 64, 2, 2, 16, 4),
    DMA_BOTH(128, 128, 64, 2, 2, 32, 2),
    DMA_BOTH(128, 128, 64, 2, 4, 16, 4),
    DMA_BOTH(128, 128, 32, 2, 4, 16, 4),
    DMA_BOTH(192, 256, 64, 2, 4, 16, 2),
};

}  // namespace

const KernelEntry* dma_kernel_table_more(int* count) {
    *count = static_cast<int>(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace dtg
