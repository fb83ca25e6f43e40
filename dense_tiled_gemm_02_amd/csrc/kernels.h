// Internal interface between the planner / C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dtg {

// Arguments of every GEMM kernel; strides in elements.  A element (m, k) is
// A[m * lda + k * sak], B element (k, n) is B[k * ldb + n * sbn]; C and D are
// row-major with leading strides ldc, ldd.  M, N, K < 2^31 (the planner
// rejects larger).
struct KArgs {
    const uint16_t* A;
    const uint16_t* B;
    const uint16_t* C;   // nullptr unless has_c
    uint16_t* D;
    int32_t M, N, K;
    int32_t num_pid_m, num_pid_n;
    int32_t group_m;
    int32_t xcds;        // 1: no XCD pre-permutation
    int32_t has_c;
    int32_t splits;      // K slices across workgroups (1 = none)
    int64_t lda, ldb, ldc, ldd;
    int64_t sak, sbn;    // 1 for row-major A and B
    void* ws;            // workspace: arrival counters, then fp32 partial tiles
};

// Workspace of every split-K launch: a fixed region of kMaxCounters 32-bit
// arrival counters (one per output slab or tile, left at zero by every
// launch), then the fp32 partial tiles.  The region is the same for every
// plan, so one zero-filled workspace serves any sequence of plans.
constexpr int kMaxCounters = 4096;
constexpr int64_t kCounterBytes = kMaxCounters * 4;

typedef hipError_t (*launch_fn)(const KArgs& args, int64_t grid, hipStream_t stream);

enum KernelFamily { KF_TILE = 1, KF_SKINNY = 2, KF_DMA = 3, KF_DMA_SK = 6 };

// One compiled kernel variant.  vec = 1: 16-byte vector loads (requires
// K % 8 == 0, N % 8 == 0, lda % 8 == 0, ldb % 8 == 0 and 16-byte aligned A, B);
// vec = 0: element loads, any shape.
struct KernelEntry {
    int32_t family;
    int32_t bm, bn, bk, stages, mfma, waves_m, waves_n, splitk;
    int32_t dtype;       // 0 fp16, 1 bf16, 2 int8 operands with int32 C and D
    int32_t vec;
    int32_t threads;
    int64_t lds_bytes;
    launch_fn launch;
    const char* name;
    int32_t layout;      // operands in memory: bit 0 A stored K x M, bit 1 B stored N x K; -1 any strides
    int32_t stream_b;    // 1: B loaded non-temporal, for grids of one row of tiles (each byte of B read once)
};

// Layout code of a problem's A and B (see KernelEntry::layout).
constexpr int kLayTA = 1, kLayTB = 2;

// All compiled variants (tile kernels followed by skinny kernels).
const KernelEntry* tile_kernel_table(int* count);
const KernelEntry* skinny_kernel_table(int* count);
const KernelEntry* dma_kernel_table(int* count);
const KernelEntry* i8_kernel_table(int* count);   // dtype 2: int8 operands, int32 C and D

// Workspace bytes of a skinny launch over nslabs slabs of bm x bn split into
// `splits` K slices (0 when splits == 1, -1 when nslabs is above the fixed
// counter region).
int64_t skinny_workspace_bytes(int64_t nslabs, int bm, int bn, int splits);

// Workspace bytes of a direct-to-LDS launch over `tiles` output tiles of
// bm x bn split into `splits` K slices (0 when splits == 1, -1 when tiles is
// above the counter region).
int64_t dma_workspace_bytes(int64_t tiles, int bm, int bn, int splits);

// Workspace bytes of a stream-K launch of `workgroups` workgroups over
// `tiles` output tiles of bm x bn (-1 when tiles is above the counter region).
int64_t dma_sk_workspace_bytes(int64_t tiles, int bm, int bn, int64_t workgroups);

// Enqueue a kernel that writes zeros to nwords 32-bit words at p.
hipError_t zero_words(void* p, int64_t nwords, hipStream_t stream);

}  // namespace dtg
