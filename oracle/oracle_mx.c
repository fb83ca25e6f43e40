/*
 * CPU oracle for the block-scaled ("microscaled") matrix multiply
 *     D = A x B (+ C)
 * on MX operands: 8-bit or 4-bit floating-point elements, each run of 32
 * consecutive k of a row of A (of a column of B) sharing one power-of-two
 * scale.
 *
 * TEST INFRASTRUCTURE ONLY, like oracle.c: nothing on the product path links,
 * loads or calls this file, and it shares no code, header, table or helper with
 * the HIP library.
 *
 * What it computes.  "Tuning Triton kernels", section 6 (Gluon): gfx950 adds a
 * scaled matrix instruction as the way to the microscaled data types (there is
 * no gfx942 counterpart), and the FP4 x FP4 GEMM kernel tuned in the same
 * section ("Tuning someone else's Gluon kernel") runs on them.  The pages name
 * the types but do not define them; the plain reading is the OCP Microscaling
 * (MX) formats, v1.0:
 *   - a block is 32 consecutive elements along the reduction (k) index, with
 *     one shared scale X = 2^(e - 127) stored as an 8-bit exponent e (E8M0;
 *     e = 255 is NaN);
 *   - elements are FP8 E4M3 (bias 7, 3 fraction bits, no infinities, NaN is
 *     S.1111.111), FP8 E5M2 (bias 15, 2 fraction bits, IEEE-style infinities
 *     and NaNs), FP6 E2M3 (bias 1, 3 fraction bits) or E3M2 (bias 3, 2
 *     fraction bits), or FP4 E2M1 (bias 1, 1 fraction bit); the FP6 and FP4
 *     formats have no infinities or NaNs;
 *   - the dot product of two MX vectors is the sum over blocks of
 *     X_a * X_b * sum_i (a_i * b_i), i.e. the sum over k of the scaled
 *     element products.
 * So, for A of M x K elements with scales SA (M x ceil(K/32)) and B given
 * column by column (N x K elements, scales SB, N x ceil(K/32)):
 *     ref[i][j] = sum_{k ascending} (a_ik X^A_{i,k/32}) (b_jk X^B_{j,k/32})  (+ c_ij),
 *     S[i][j]   = sum_k |(a_ik X^A) (b_jk X^B)|.
 * Every scaled element is exact in binary64 (at most 4 significand bits times a
 * power of two between 2^-127 and 2^127) and so is every product (at most 8
 * bits, exponents well inside binary64's range); the only rounding is the
 * binary64 summation, bounded by K * 2^-53 * S.
 *
 * Acceptance rule (oracle_mx_tol_check).  The pages fix no precision for the
 * microscaled product, so the bound is derived from the arithmetic of the
 * instruction that computes it, as measured by a single-instruction probe:
 * the scaled matrix instruction adds each run of 8 consecutive products after
 * aligning them to the largest, keeping 13 bits below that product's leading
 * bit (a product 2^14 below the largest of its run is lost, one 2^13 below is
 * kept); the run sums are then accumulated in binary32.  A run's error is
 * below 8 * 2^(floor(log2 max|p|) - 13) <= 2^-10 * max|p|, so with
 *     S8[i][j] = sum over runs k = 8q .. 8q + 7 of max_k |(a X^A)(b X^B)|
 * a computed output g is accepted when g is finite and
 *     |g - ref| <= ulp_out(ref) + 2^-20 * S + 2^-10 * S8
 * (2^-20 S is the binary32 accumulation term of the 16-bit contract).
 *
 * Storage (the library's convention, restated here independently): elements
 * of an 8-bit format are one byte each, element k of row i at byte
 * A[i * lda + k]; FP4 elements are packed two per byte, element k at byte
 * A[i * lda + k / 2], in the low nibble for even k and the high nibble for odd
 * k; FP6 elements are packed four per three bytes, the row read as one
 * little-endian bit string with element k in bits 6k .. 6k + 5 (element k
 * starts in byte 6k / 8).  The scale of block t of row i is byte
 * SA[i * ldsa + t].  B is stored the
 * same way with its columns as rows: element (k, j) at B[j * ldb + k] (FP8).
 *
 * Build: compiled into liboracle.so together with oracle.c (build.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* element format codes of this file's entry points */
#define MX_E4M3 0
#define MX_E5M2 1
#define MX_E2M3 2
#define MX_E3M2 3
#define MX_E2M1 4

/* FP8 E4M3: sign, 4 exponent bits (bias 7), 3 fraction bits.  Exponent field
 * 0 is subnormal (m/8 * 2^-6); exponent 15 with fraction 7 is NaN, and every
 * other pattern, exponent 15 included, is a finite normal number. */
double oracle_decode_e4m3(uint8_t c) {
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = ldexp((double)m, -9);            /* m/8 * 2^-6 */
    else v = ldexp((double)(8 + m), e - 10);              /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* FP8 E5M2: sign, 5 exponent bits (bias 15), 2 fraction bits, IEEE-style:
 * exponent 31 is infinity (fraction 0) or NaN. */
double oracle_decode_e5m2(uint8_t c) {
    int s = (c >> 7) & 1, e = (c >> 2) & 31, m = c & 3;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -16);           /* m/4 * 2^-14 */
    else v = ldexp((double)(4 + m), e - 17);              /* (1 + m/4) * 2^(e-15) */
    return s ? -v : v;
}

/* FP4 E2M1 (the low 4 bits of c): sign, 2 exponent bits (bias 1), 1 fraction
 * bit; exponent 0 is subnormal (m/2), no infinities or NaNs. */
double oracle_decode_e2m1(uint8_t c) {
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v;
    if (e == 0) v = 0.5 * m;
    else v = ldexp((double)(2 + m), e - 2);               /* (1 + m/2) * 2^(e-1) */
    return s ? -v : v;
}

/* FP6 E2M3 (the low 6 bits of c): sign, 2 exponent bits (bias 1), 3 fraction
 * bits; exponent 0 is subnormal (m/8), no infinities or NaNs (largest 7.5). */
double oracle_decode_e2m3(uint8_t c) {
    int s = (c >> 5) & 1, e = (c >> 3) & 3, m = c & 7;
    double v;
    if (e == 0) v = ldexp((double)m, -3);                 /* m/8 */
    else v = ldexp((double)(8 + m), e - 4);               /* (1 + m/8) * 2^(e-1) */
    return s ? -v : v;
}

/* FP6 E3M2 (the low 6 bits of c): sign, 3 exponent bits (bias 3), 2 fraction
 * bits; exponent 0 is subnormal (m/4 * 2^-2), no infinities or NaNs (largest 28). */
double oracle_decode_e3m2(uint8_t c) {
    int s = (c >> 5) & 1, e = (c >> 2) & 7, m = c & 3;
    double v;
    if (e == 0) v = ldexp((double)m, -4);                 /* m/4 * 2^-2 */
    else v = ldexp((double)(4 + m), e - 5);               /* (1 + m/4) * 2^(e-3) */
    return s ? -v : v;
}

/* E8M0 scale: 2^(c - 127); c = 255 is NaN. */
double oracle_decode_e8m0(uint8_t c) {
    return c == 255 ? NAN : ldexp(1.0, (int)c - 127);
}

/* Code of FP6 element k of a stored row: the row's bytes read as one
 * little-endian bit string, element k in bits 6k .. 6k + 5. */
uint8_t oracle_fp6_code(const uint8_t* row, int64_t k) {
    const int64_t bit = 6 * k;
    const int64_t byte = bit / 8;
    const int off = (int)(bit % 8);
    unsigned v = row[byte] >> off;
    if (off > 2) v |= (unsigned)row[byte + 1] << (8 - off);   /* the code continues in the next byte */
    return (uint8_t)(v & 63u);
}

/* Element k of one stored row. */
static double mx_element(const uint8_t* row, int64_t k, int fmt) {
    if (fmt == MX_E2M1) {
        const uint8_t b = row[k >> 1];
        return oracle_decode_e2m1((k & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15));
    }
    if (fmt == MX_E2M3) return oracle_decode_e2m3(oracle_fp6_code(row, k));
    if (fmt == MX_E3M2) return oracle_decode_e3m2(oracle_fp6_code(row, k));
    return fmt == MX_E4M3 ? oracle_decode_e4m3(row[k]) : oracle_decode_e5m2(row[k]);
}

static int fmt_ok(int fmt) {
    return fmt == MX_E4M3 || fmt == MX_E5M2 || fmt == MX_E2M3 || fmt == MX_E3M2 || fmt == MX_E2M1;
}

/* Scaled values of one stored row: out[k] = element k * its block's scale. */
static void scaled_row(const uint8_t* row, const uint8_t* srow, int64_t K, int fmt, double* out) {
    for (int64_t k = 0; k < K; ++k) out[k] = mx_element(row, k, fmt) * oracle_decode_e8m0(srow[k / 32]);
}

/*
 * Full product.  A: M rows of lda bytes, SA: M rows of ldsa bytes; B: N rows
 * (the columns of B) of ldb bytes, SB: N rows of ldsb bytes; C (may be NULL):
 * binary64 values, element (i, j) at C[i * ldc_m + j * ldc_n].  ref and S are
 * dense row-major M x N.  Rows of the output are spread over OpenMP threads.
 */
int oracle_mx_gemm_f64(int64_t M, int64_t N, int64_t K, int fmt_a, int fmt_b,
                       const uint8_t* A, int64_t lda, const uint8_t* SA, int64_t ldsa,
                       const uint8_t* B, int64_t ldb, const uint8_t* SB, int64_t ldsb,
                       const double* C, int64_t ldc_m, int64_t ldc_n, double* ref, double* S, double* S8) {
    if (M < 0 || N < 0 || K < 0 || !fmt_ok(fmt_a) || !fmt_ok(fmt_b)) return 1;
    if (M == 0 || N == 0) return 0;
    const size_t KK = (size_t)(K > 0 ? K : 1);
    double* Bv = (double*)malloc(KK * (size_t)N * sizeof(double));
    if (!Bv) return 2;
    for (int64_t j = 0; j < N; ++j) scaled_row(B + j * ldb, SB + j * ldsb, K, fmt_b, Bv + (size_t)j * KK);
    int failed = 0;
#pragma omp parallel
    {
        double* arow = (double*)malloc(KK * sizeof(double));
        if (!arow) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            if (!arow) continue;
            scaled_row(A + i * lda, SA + i * ldsa, K, fmt_a, arow);
            for (int64_t j = 0; j < N; ++j) {
                const double* b = Bv + (size_t)j * KK;
                double r = 0.0, s = 0.0, s8 = 0.0, run_max = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const double prod = arow[k] * b[k];    /* exact */
                    r += prod;
                    s += fabs(prod);
                    if (fabs(prod) > run_max) run_max = fabs(prod);
                    if (k % 8 == 7 || k == K - 1) { s8 += run_max; run_max = 0.0; }
                }
                if (C) r += C[i * ldc_m + j * ldc_n];
                ref[i * N + j] = r;
                S[i * N + j] = s;
                if (S8) S8[i * N + j] = s8;
            }
        }
        free(arow);
    }
    free(Bv);
    return failed ? 2 : 0;
}

/* The same definition at the listed output positions (ii[t], jj[t]). */
int oracle_mx_gemm_f64_at(int64_t K, int fmt_a, int fmt_b,
                          const uint8_t* A, int64_t lda, const uint8_t* SA, int64_t ldsa,
                          const uint8_t* B, int64_t ldb, const uint8_t* SB, int64_t ldsb,
                          const double* C, int64_t ldc_m, int64_t ldc_n,
                          int64_t npts, const int64_t* ii, const int64_t* jj, double* ref, double* S,
                          double* S8) {
    if (K < 0 || npts < 0 || !fmt_ok(fmt_a) || !fmt_ok(fmt_b)) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < npts; ++t) {
        const int64_t i = ii[t], j = jj[t];
        double r = 0.0, s = 0.0, s8 = 0.0, run_max = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = mx_element(A + i * lda, k, fmt_a) * oracle_decode_e8m0(SA[i * ldsa + k / 32]);
            const double b = mx_element(B + j * ldb, k, fmt_b) * oracle_decode_e8m0(SB[j * ldsb + k / 32]);
            r += a * b;
            s += fabs(a * b);
            if (fabs(a * b) > run_max) run_max = fabs(a * b);
            if (k % 8 == 7 || k == K - 1) { s8 += run_max; run_max = 0.0; }
        }
        if (C) r += C[i * ldc_m + j * ldc_n];
        ref[t] = r;
        S[t] = s;
        if (S8) S8[t] = s8;
    }
    return 0;
}

/* One unit in the last place of binary32 at x, in the binade of |x| (the
 * subnormal quantum 2^-149 below 2^-126): 2^(max(floor(log2|x|), -126) - 23). */
double oracle_ulp_f32(double x) {
    int e = -126;
    if (x != 0.0 && isfinite(x)) {
        int E;
        frexp(x, &E);
        e = E - 1;
        if (e < -126) e = -126;
    }
    return ldexp(1.0, e - 23);
}

/* Acceptance check of binary32 outputs: g finite and
 * |g - ref| <= ulp_f32(ref) + 2^-20 S.  Same contract as oracle_tol_check. */
int64_t oracle_tol_check_f32(int64_t n, const float* got, const double* ref, const double* S,
                             double* worst, int64_t* first_bad) {
    int64_t fails = 0, first = -1;
    double w = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        const double g = (double)got[t];
        const double bound = oracle_ulp_f32(ref[t]) + ldexp(S[t], -20);
        double ratio;
        int bad;
        if (!isfinite(g)) { ratio = INFINITY; bad = 1; }
        else {
            const double err = fabs(g - ref[t]);
            ratio = err / bound;
            bad = err > bound;
        }
        if (ratio > w) w = ratio;
        if (bad) { if (first < 0) first = t; ++fails; }
    }
    if (worst) *worst = w;
    if (first_bad) *first_bad = first;
    return fails;
}

/* Decoded output value: kind 0 fp16, 1 bf16 (bit patterns), 2 binary32. */
static double out_value(const void* got, int64_t t, int kind) {
    if (kind == 2) return (double)((const float*)got)[t];
    const uint16_t h = ((const uint16_t*)got)[t];
    if (kind == 1) {
        uint32_t w = (uint32_t)h << 16;
        float f;
        memcpy(&f, &w, 4);
        return (double)f;
    }
    int sg = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v = e == 0 ? ldexp((double)m, -24) : e == 31 ? (m ? NAN : INFINITY) : ldexp((double)(1024 + m), e - 25);
    return sg ? -v : v;
}

/* One ulp of the output type at x, in the binade of |x| (subnormal quantum at
 * least): precision p and minimum exponent of fp16 (11, -14), bf16 (8, -126)
 * or binary32 (24, -126). */
static double out_ulp(double x, int kind) {
    const int p = kind == 0 ? 11 : kind == 1 ? 8 : 24;
    const int emin = kind == 0 ? -14 : -126;
    int e = emin;
    if (x != 0.0 && isfinite(x)) {
        int E;
        frexp(x, &E);
        e = E - 1 < emin ? emin : E - 1;
    }
    return ldexp(1.0, e - p + 1);
}

/* The MX acceptance rule above for n outputs of type `kind` (0 fp16, 1 bf16,
 * 2 binary32).  S8 may be NULL (term dropped).  Returns the number of
 * failures; *worst is the largest |g - ref| / bound (infinity for a
 * non-finite g), *first_bad the first failing index or -1. */
int64_t oracle_mx_tol_check(int64_t n, const void* got, int kind, const double* ref, const double* S,
                            const double* S8, double* worst, int64_t* first_bad) {
    int64_t fails = 0, first = -1;
    double w = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        const double g = out_value(got, t, kind);
        const double bound = out_ulp(ref[t], kind) + ldexp(S[t], -20) + (S8 ? ldexp(S8[t], -10) : 0.0);
        double ratio;
        int bad;
        if (!isfinite(g)) { ratio = INFINITY; bad = 1; }
        else {
            const double err = fabs(g - ref[t]);
            ratio = err / bound;
            bad = err > bound;
        }
        if (ratio > w) w = ratio;
        if (bad) { if (first < 0) first = t; ++fails; }
    }
    if (worst) *worst = w;
    if (first_bad) *first_bad = first;
    return fails;
}
