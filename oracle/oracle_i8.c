/*
 * CPU oracle for the integer matrix multiply  D = A x B (+ C):  8-bit integer
 * inputs, 32-bit integer accumulation and output.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code with the HIP library.
 *
 * What it computes (sources, by page title and section):
 *  - FlagGems "Hygon optimization", section "DUMMA matrix instruction shapes":
 *    the matrix unit takes integer inputs as well as floating-point ones, the
 *    lower precision covering more k per instruction, and one operation
 *    computes D = A x B + C;
 *  - "DCU K100 节点初探" section 5.2 (MatMulAdd): D[i][j] = sum_k A[i][k] B[k][j]
 *    + C[i][j], D a separate output and C an addend.
 *
 * Definition evaluated here, for i < M, j < N:
 *     exact[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]  (+ C[i][j])   in int64,
 *     D[i][j]     = exact[i][j] reduced modulo 2^32 to a two's-complement int32.
 * Every product is at most 2^14 in magnitude, so the int64 sum is exact for
 * any K below 2^48; an int32 accumulator that wraps on overflow reaches the
 * same residue in any order of addition, which is why D (not a saturated
 * value) is the result.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (see build.py).
 */
#include <stdint.h>
#include <stdlib.h>

/* x modulo 2^32 as a two's-complement int32: the unsigned residue of the low
 * 32 bits, read back as signed. */
int32_t oracle_wrap_i32(int64_t x) {
    const uint32_t low = (uint32_t)((uint64_t)x & 0xffffffffu);
    return low < 0x80000000u ? (int32_t)low : (int32_t)((int64_t)low - 0x100000000LL);
}

/*
 * Loop order i, k, j (B read by rows); rows of the output spread over OpenMP
 * threads.  A element (i, k) is A[i * sa_m + k * sa_k], B element (k, j) is
 * B[k * sb_k + j * sb_n], C element (i, j) is C[i * sc_m + j * sc_n] (C may
 * be NULL).  exact (may be NULL) and D are row-major M x N.  Returns 0, or 1
 * on a negative size, 2 when out of memory.
 */
int oracle_gemm_i8(int64_t M, int64_t N, int64_t K,
                   const int8_t* A, int64_t sa_m, int64_t sa_k,
                   const int8_t* B, int64_t sb_k, int64_t sb_n,
                   const int32_t* C, int64_t sc_m, int64_t sc_n,
                   int64_t* exact, int32_t* D) {
    if (M < 0 || N < 0 || K < 0) return 1;
    if (M == 0 || N == 0) return 0;
    int failed = 0;
#pragma omp parallel
    {
        int64_t* acc = (int64_t*)malloc((size_t)N * sizeof(int64_t));
        if (!acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            if (!acc) continue;
            for (int64_t j = 0; j < N; ++j) acc[j] = 0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t a = A[i * sa_m + k * sa_k];
                for (int64_t j = 0; j < N; ++j) acc[j] += a * (int64_t)B[k * sb_k + j * sb_n];
            }
            if (C)
                for (int64_t j = 0; j < N; ++j) acc[j] += C[i * sc_m + j * sc_n];
            for (int64_t j = 0; j < N; ++j) {
                if (exact) exact[i * N + j] = acc[j];
                D[i * N + j] = oracle_wrap_i32(acc[j]);
            }
        }
        free(acc);
    }
    return failed ? 2 : 0;
}
