/*
 * CPU oracle for the dense matrix multiply  D = A x B (+ C).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or helper with the HIP
 * library; it is written from the IEEE 754 definitions and the plain
 * definition of a matrix product.
 *
 * What it computes (sources, by page title and section):
 *  - "DCU K100 节点初探" section 5.2 (MatMulAdd): D[i][j] = sum_k A[i][k]*B[k][j] + C[i][j],
 *    with D a separate output and C an addend.
 *  - FlagGems "Hygon optimization", section "DUMMA matrix instruction shapes":
 *    one matrix operation computes D = A x B + C.
 *  - "Hopper Support in Triton", slides 6-7: fp16 inputs, an fp32 accumulator,
 *    a K loop of tile products, and a truncation of the fp32 result to the
 *    input type before the store.
 *
 * The oracle evaluates the exact sum in IEEE binary64 from the exact values of
 * the stored fp16/bf16 inputs:
 *     ref[i][j] = sum_{k=0}^{K-1} a_ik * b_kj  (+ c_ij),   k ascending,
 *     S[i][j]   = sum_k |a_ik * b_kj|.
 * Every fp16 x fp16 or bf16 x bf16 product is exact in binary64 (at most 22
 * significant bits), so the only rounding is the fp64 summation, bounded by
 * K * 2^-53 * S.
 *
 * The acceptance rule for a computed output g (the library's documented
 * tolerance):  g finite and |g - ref| <= ulp_out(ref) + 2^-20 * S.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (see build.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes used by this file's entry points */
#define ORACLE_F16 0
#define ORACLE_BF16 1

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);                 /* subnormal: m/2^10 * 2^-14 */
    } else if (e == 31) {
        v = m ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/2^10) * 2^(e-15) */
    }
    return s ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_decode_bf16(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int m = h & 0x7f;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -133);                /* subnormal: m/2^7 * 2^-126 */
    } else if (e == 255) {
        v = m ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + m), e - 134);     /* (1 + m/2^7) * 2^(e-127) */
    }
    return s ? -v : v;
}

static double decode(uint16_t h, int dtype) {
    return dtype == ORACLE_BF16 ? oracle_decode_bf16(h) : oracle_decode_f16(h);
}

/* Format parameters: precision p (significand bits incl. the implicit one),
 * minimum normal exponent emin, maximum exponent emax. */
static void fmt_params(int dtype, int* p, int* emin, int* emax) {
    if (dtype == ORACLE_BF16) { *p = 8; *emin = -126; *emax = 127; }
    else                      { *p = 11; *emin = -14; *emax = 15; }
}

/* Exponent of the leading bit of a finite, nonzero |x|: floor(log2|x|). */
static int ilog2_abs(double x) {
    int E;
    frexp(x, &E);          /* |x| = f * 2^E, f in [0.5, 1) */
    return E - 1;
}

/* One unit in the last place of the output format at x, taken in the binade of
 * |x| (clamped to the subnormal quantum): 2^(max(floor(log2|x|), emin) - p + 1).
 * At x = 0 this is the smallest subnormal. */
double oracle_ulp_out(double x, int dtype) {
    int p, emin, emax;
    fmt_params(dtype, &p, &emin, &emax);
    int e = (x == 0.0) ? emin : ilog2_abs(x);
    if (e < emin) e = emin;
    return ldexp(1.0, e - p + 1);
}

/* Round a binary64 value to the nearest fp16/bf16 value, ties to even, and
 * return its bit pattern.  Values at or beyond the overflow threshold become
 * infinities; NaN becomes the canonical quiet NaN. */
uint16_t oracle_encode_rne(double x, int dtype) {
    int p, emin, emax;
    fmt_params(dtype, &p, &emin, &emax);
    int ebits = (dtype == ORACLE_BF16) ? 8 : 5;
    int fbits = p - 1;
    int bias = (1 << (ebits - 1)) - 1;
    uint16_t sign = signbit(x) ? (uint16_t)(1u << 15) : 0;
    uint16_t inf_bits = (uint16_t)(((1u << ebits) - 1) << fbits);
    if (isnan(x)) return (uint16_t)(inf_bits | (1u << (fbits - 1)));
    double a = fabs(x);
    if (isinf(a)) return sign | inf_bits;
    if (a == 0.0) return sign;
    int e = ilog2_abs(a);
    if (e < emin) e = emin;
    int q = e - fbits;                      /* exponent of the quantum at a */
    double r = ldexp(a, -q);                /* exact: power-of-two scaling */
    double n = rint(r);                     /* default mode: nearest, ties to even */
    double v = ldexp(n, q);                 /* the rounded magnitude */
    if (v >= ldexp(1.0, emax + 1)) return sign | inf_bits;
    if (v < ldexp(1.0, emin)) {
        /* subnormal (or rounded up to the smallest normal: n == 2^fbits gives
         * exponent field 1, fraction 0, the same bit pattern) */
        return sign | (uint16_t)n;
    }
    int ev = ilog2_abs(v);
    uint32_t frac = (uint32_t)(ldexp(v, fbits - ev) - ldexp(1.0, fbits));
    return sign | (uint16_t)(((uint32_t)(ev + bias) << fbits) | frac);
}

void oracle_decode_array(const uint16_t* src, double* dst, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) dst[i] = decode(src[i], dtype);
}

void oracle_encode_array(const double* src, uint16_t* dst, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_encode_rne(src[i], dtype);
}

double oracle_ulp_array(const double* src, double* dst, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_ulp_out(src[i], dtype);
    return n ? dst[0] : 0.0;
}

/*
 * Full product.  A is M x K with element strides (sa_m, sa_k), B is K x N with
 * (sb_k, sb_n), C (may be NULL) is M x N with (sc_m, sc_n).  ref and S are
 * dense row-major M x N binary64 arrays.
 *
 * Loop order i, k, j with k ascending: for each (i, j) the terms are added in
 * the same order as in the textbook i, j, k loop, so the result is the same;
 * this order only reads B by rows.  Rows of the output are independent and
 * are spread over OpenMP threads.
 */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K, int dtype,
                    const uint16_t* A, int64_t sa_m, int64_t sa_k,
                    const uint16_t* B, int64_t sb_k, int64_t sb_n,
                    const uint16_t* C, int64_t sc_m, int64_t sc_n,
                    double* ref, double* S) {
    if (M < 0 || N < 0 || K < 0) return 1;
    if (M == 0 || N == 0) return 0;
    /* exact values of B, decoded once, row-major K x N */
    double* Bv = (double*)malloc((size_t)(K > 0 ? K : 1) * (size_t)N * sizeof(double));
    if (!Bv) return 2;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            Bv[k * N + j] = decode(B[k * sb_k + j * sb_n], dtype);
    int failed = 0;
#pragma omp parallel
    {
        double* arow = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
        if (!arow) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            if (!arow) continue;
            double* r = ref + i * N;
            double* s = S + i * N;
            for (int64_t j = 0; j < N; ++j) { r[j] = 0.0; s[j] = 0.0; }
            for (int64_t k = 0; k < K; ++k) arow[k] = decode(A[i * sa_m + k * sa_k], dtype);
            for (int64_t k = 0; k < K; ++k) {
                const double a = arow[k];
                const double* b = Bv + k * N;
                for (int64_t j = 0; j < N; ++j) {
                    const double prod = a * b[j];     /* exact */
                    r[j] += prod;
                    s[j] += fabs(prod);
                }
            }
            if (C)
                for (int64_t j = 0; j < N; ++j) r[j] += decode(C[i * sc_m + j * sc_n], dtype);
        }
        free(arow);
    }
    free(Bv);
    return failed ? 2 : 0;
}

/*
 * The same definition evaluated only at the listed output positions
 * (ii[t], jj[t]), t < npts: a dot product over k ascending plus c.  Used where
 * the full product is too large for the CPU.
 */
int oracle_gemm_f64_at(int64_t K, int dtype,
                       const uint16_t* A, int64_t sa_m, int64_t sa_k,
                       const uint16_t* B, int64_t sb_k, int64_t sb_n,
                       const uint16_t* C, int64_t sc_m, int64_t sc_n,
                       int64_t npts, const int64_t* ii, const int64_t* jj,
                       double* ref, double* S) {
    if (K < 0 || npts < 0) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < npts; ++t) {
        const int64_t i = ii[t], j = jj[t];
        double r = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double prod = decode(A[i * sa_m + k * sa_k], dtype) *
                                decode(B[k * sb_k + j * sb_n], dtype);
            r += prod;
            s += fabs(prod);
        }
        if (C) r += decode(C[i * sc_m + j * sc_n], dtype);
        ref[t] = r;
        S[t] = s;
    }
    return 0;
}

/*
 * Acceptance check of computed outputs against ref and S.  got[t] is the bit
 * pattern of output t (n values, in the same order as ref and S).  Returns the
 * number of failures; *worst is the largest |g - ref| / (ulp_out(ref) + 2^-20 S)
 * (infinity for a non-finite g), *first_bad the index of the first failure or -1.
 */
int64_t oracle_tol_check(int64_t n, const uint16_t* got, const double* ref, const double* S,
                         int dtype, double* worst, int64_t* first_bad) {
    int64_t fails = 0, first = -1;
    double w = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        const double g = decode(got[t], dtype);
        const double bound = oracle_ulp_out(ref[t], dtype) + ldexp(S[t], -20);
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

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
