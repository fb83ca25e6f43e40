// Stream-K variants of the direct-to-LDS GEMM kernel (gemm_dma_kernel.h):
// row-major operands; the (tile, K step) iterations dealt out to a fixed
// number of workgroups, tiles cut by range starts finished by the K-slice
// exchange.  256 x 256 is the planner's; 256 x 128 runs the exchange with
// 64 accumulators per lane.
#include "gemm_dma_kernel.h"

namespace dtg {
namespace {

const KernelEntry kTable[] = {
    DMA_SK_BOTH(256, 256, 64, 2, 4, 16, 2),
    DMA_SK_BOTH(256, 128, 64, 4, 2, 16, 3),
};

}  // namespace

const KernelEntry* dma_kernel_table_sk(int* count) {
    *count = static_cast<int>(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace dtg
