// Stream-K variants of the direct-to-LDS GEMM kernel (gemm_dma_kernel.h):
// row-major operands; the (tile, K step) iterations dealt out to a fixed
// number of workgroups, tiles cut by range starts finished by the K-slice
// exchange.  256 x 256 is the planner's; 256 x 128 runs the exchange with
// 64 accumulators per lane.  Also the streamed-B variants the planner swaps
// in when the grid has one row of tiles.
#include "gemm_dma_kernel.h"

namespace dtg {
namespace {

const KernelEntry kTable[] = {
    DMA_SK_BOTH(256, 256, 64, 2, 4, 16, 2),
    DMA_SK_BOTH(256, 128, 64, 4, 2, 16, 3),
    // streamed B for one row of tiles: the 4-wave 64 x 64 tile of the short,
    // wide problems and of the decode table (32 x 8192 x 8192 29.4 -> 28.6 us,
    // 64 x 8192 x 8192 31.8 -> 31.2, 32 and 64 x 4096 x 4096 12.8 -> 12.6 and
    // 13.5 -> 13.3; the K-sliced 128 x 128 tile lost by it: 48 x 2048 x 8192
    // 20.9 -> 21.9 us, so it has no twin)
    DMA_SB_BOTH(64, 64, 64, 2, 2, 16, 4),
};

}  // namespace

const KernelEntry* dma_kernel_table_sk(int* count) {
    *count = static_cast<int>(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace dtg
