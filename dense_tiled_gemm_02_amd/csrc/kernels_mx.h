// Internal interface between the block-scaled (MX) planner / C ABI and its
// HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dtg {

// Arguments of the MX kernels.  A: M rows of lda bytes (k along the row),
// B: N rows of ldb bytes (column j of B, k along the row), SA / SB: M / N rows
// of ldsa / ldsb bytes of E8M0 scales, one per 32 k.  C, D: row-major M x N
// of the output type, leading strides ldc, ldd in elements.
struct MxArgs {
    const uint8_t* A;
    const uint8_t* B;
    const uint8_t* SA;
    const uint8_t* SB;
    const void* C;       // nullptr unless has_c
    void* D;
    int32_t M, N, K;     // K in elements
    int32_t num_pid_m, num_pid_n;
    int32_t group_m;
    int32_t xcds;        // 1: no XCD pre-permutation
    int32_t has_c;
    int32_t out;         // output type: 0 fp16, 1 bf16, 2 fp32
    int64_t lda, ldb, ldsa, ldsb;
    int64_t ldc, ldd;
    int32_t splits;      // K slices across workgroups (1 = none)
    void* ws;            // workspace of the K slices (same layout as the 16-bit kernels')
};

typedef hipError_t (*mx_launch_fn)(const MxArgs& args, int64_t grid, hipStream_t stream);

// Element format codes (the matrix instruction's own operand-type codes).
constexpr int kMxE4M3 = 0, kMxE5M2 = 1, kMxE2M3 = 2, kMxE3M2 = 3, kMxE2M1 = 4;

// gemm_config.kernel values of the two block-scaled kernels: the LDS-staged
// tile kernel (gemm_mx_kernel.h; every pair of formats, its variants in
// gemm_mx.hip for pairs of one width and gemm_mx_pairs.hip for the others)
// and the register-direct kernel (gemm_mx_direct.hip; every pair).
constexpr int kMxKernelTile = 4, kMxKernelDirect = 5;

// One compiled MX kernel variant.
struct MxEntry {
    int32_t bm, bn;
    int32_t bk;          // k per K step (elements): 128 bytes of k per row
    int32_t stages, mfma, waves_m, waves_n;
    int32_t fmt_a, fmt_b;
    int32_t splitk;      // most K slices the variant takes (1: none)
    int32_t threads;
    int64_t lds_bytes;
    mx_launch_fn launch;
    const char* name;
    int32_t kind;        // kMxKernelTile or kMxKernelDirect
};

const MxEntry* mx_kernel_table(int* count);
const MxEntry* mx_pair_kernel_table(int* count);
const MxEntry* mx_direct_kernel_table(int* count);

}  // namespace dtg
