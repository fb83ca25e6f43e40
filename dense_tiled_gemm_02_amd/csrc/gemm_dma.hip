// Variants of the direct-to-LDS GEMM kernel (gemm_dma_kernel.h): the
// planner's ladder tiles and the wide-tile experiments, row-major operands;
// the table the planner sees joins the three variant files.
#include <vector>

#include "gemm_dma_kernel.h"

namespace dtg {
namespace {

const KernelEntry kTable[] = {
    DMA_BOTH(256, 256, 64, 2, 4, 16, 2),
    DMA_BOTH(256, 128, 64, 4, 2, 16, 2),
    DMA_BOTH(128, 256, 64, 2, 4, 16, 2),
    DMA_BOTH(128, 128, 64, 2, 4, 16, 2),
    DMA_BOTH(256, 128, 64, 4, 2, 16, 3),
    DMA_BOTH(128, 256, 64, 2, 4, 16, 3),
    DMA_BOTH(64, 64, 64, 2, 2, 16, 4),
    DMA_BOTH(256, 256, 32, 2, 4, 16, 4),
    DMA_BOTH(256, 256, 64, 2, 4, 32, 2),
    DMA_BOTH(256, 256, 32, 2, 4, 32, 4),
    // one wave per SIMD, 128 x 128 wave tiles, accumulators in AGPRs
    DMA_BOTH(256, 256, 64, 2, 2, 32, 2),
    DMA_BOTH(256, 256, 64, 2, 2, 16, 2),
};

}  // namespace

const KernelEntry* dma_kernel_table_more(int* count);
const KernelEntry* dma_kernel_table_layouts(int* count);
const KernelEntry* dma_kernel_table_sk(int* count);

int64_t dma_workspace_bytes(int64_t tiles, int bm, int bn, int splits) {
    if (splits <= 1) return 0;
    if (tiles > kMaxCounters) return -1;
    return kCounterBytes + tiles * splits * static_cast<int64_t>(bm) * bn * 4;
}

int64_t dma_sk_workspace_bytes(int64_t tiles, int bm, int bn, int64_t workgroups) {
    if (tiles > kMaxCounters) return -1;
    return kCounterBytes + 2 * workgroups * static_cast<int64_t>(bm) * bn * 4;
}

const KernelEntry* dma_kernel_table(int* count) {
    static const std::vector<KernelEntry> all = [] {
        std::vector<KernelEntry> v(kTable, kTable + sizeof(kTable) / sizeof(kTable[0]));
        int n = 0;
        const KernelEntry* t = dma_kernel_table_more(&n);
        v.insert(v.end(), t, t + n);
        t = dma_kernel_table_layouts(&n);
        v.insert(v.end(), t, t + n);
        t = dma_kernel_table_sk(&n);
        v.insert(v.end(), t, t + n);
        return v;
    }();
    *count = static_cast<int>(all.size());
    return all.data();
}

}  // namespace dtg
