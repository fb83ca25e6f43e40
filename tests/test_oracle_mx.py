"""Pins of the block-scaled (MX) oracle against facts independent of it (CPU only).

The element and scale decoders are checked exhaustively against PyTorch's own
float8 / E8M0 conversions and against bit-field embeddings into IEEE binary32;
the scaled product against BLAS in float64 on the expanded (dequantized)
operands and against closed forms that fix the block size, the block index,
the nibble order of packed 4-bit elements and the orientation of B.  The last
test plants plausible mistakes into calls of the oracle and checks that the
closed-form pins reject each one.
"""
import numpy as np
import pytest
import torch

import oracle

CODES = np.arange(256, dtype=np.uint8)


def _torch_decode(codes, dt):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(dt).to(torch.float64).numpy()


def _same(got, want):
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


# ---------------------------------------------------------------- decoding


def test_e4m3_decode_exhaustive_matches_torch():
    got = oracle.mx_decode(CODES, "e4m3")
    _same(got, _torch_decode(CODES, torch.float8_e4m3fn))
    # no infinities in this format; NaN only at S.1111.111
    assert not np.isinf(got).any()
    assert set(np.flatnonzero(np.isnan(got))) == {0x7F, 0xFF}
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e5m2_decode_exhaustive_matches_torch():
    got = oracle.mx_decode(CODES, "e5m2")
    _same(got, _torch_decode(CODES, torch.float8_e5m2))
    assert got[0x7C] == np.inf and got[0xFC] == -np.inf
    assert got[0x7B] == 57344.0 and got[0x01] == 2.0 ** -16


def test_e8m0_decode_exhaustive_matches_torch_and_binary32_exponent():
    got = oracle.e8m0_decode(CODES)
    _same(got, _torch_decode(CODES, torch.float8_e8m0fnu))
    # code c is the biased exponent field of binary32: 2^(c - 127)
    c = np.arange(1, 255, dtype=np.uint32)
    assert np.array_equal(got[1:255], (c << 23).view(np.float32).astype(np.float64))
    assert got[0] == np.ldexp(1.0, -127) and np.isnan(got[255])


def test_e2m1_decode_matches_binary32_embedding():
    """A normal E2M1 code (s, e, m) has the value of the binary32 number with the
    same sign, exponent field e - 1 + 127 and leading fraction bit m; the two
    subnormal codes are 0 and half the smallest normal (1.0)."""
    codes = np.arange(16, dtype=np.uint8)
    got = oracle.mx_decode(codes, "e2m1")
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0:
            want = 0.5 * m
        else:
            want = float(np.uint32((e + 126) << 23 | m << 22).view(np.float32))
        assert got[c] == (-want if s else want), c
    # only the low nibble is an element
    assert np.array_equal(oracle.mx_decode(codes | 0xF0, "e2m1"), got)
    assert got[7] == 6.0 and got.max() == 6.0


# ---------------------------------------------------------------- products

FMTS = ["e4m3", "e5m2", "e2m1"]


def _rand_codes(rng, rows, K, fmt, full_range=False):
    """Random finite element codes, packed as the format stores them.  Unless
    full_range, the exponent field stays in a band of 8 binades (2^-4 .. 2^4)
    so that every sum below is exact in binary64."""
    if fmt == "e2m1":
        nib = rng.integers(0, 16, (rows, K + (K & 1)), dtype=np.uint8)
        return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    c = rng.integers(0, 256, (rows, K), dtype=np.uint8)
    if full_range:
        bad = (c & 0x7F) == 0x7F if fmt == "e4m3" else (c & 0x7C) == 0x7C
        c[bad] &= 0xBF           # clear an exponent bit: finite
        return c
    sign = c & 0x80
    if fmt == "e4m3":            # exponent field 3..10 (bias 7), 3 fraction bits
        return (sign | ((3 + (c & 7)) << 3) | ((c >> 3) & 7)).astype(np.uint8)
    return (sign | ((11 + (c & 7)) << 2) | ((c >> 3) & 3)).astype(np.uint8)   # bias 15


def _values(codes, K, fmt):
    """Element values by an independent route: torch's float8 decoders, or the
    binary32 embedding of E2M1 pinned above."""
    if fmt == "e2m1":
        nib = np.empty((codes.shape[0], 2 * codes.shape[1]), dtype=np.uint8)
        nib[:, 0::2] = codes & 15
        nib[:, 1::2] = codes >> 4
        table = oracle.mx_decode(np.arange(16, dtype=np.uint8), "e2m1")
        return table[nib[:, :K]]
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    return _torch_decode(codes[:, :K], dt)


def _expanded_scales(S, K):
    return np.repeat(np.ldexp(1.0, S.astype(np.int64) - 127), 32, axis=1)[:, :K]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(5, 7, 32), (9, 6, 80), (17, 12, 200)])
def test_scaled_product_equals_blas_on_dequantized_operands(fmt, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N + K)
    A = _rand_codes(rng, M, K, fmt)
    B = _rand_codes(rng, N, K, fmt)
    nb = (K + 31) // 32
    SA = rng.integers(120, 135, (M, nb), dtype=np.uint8)
    SB = rng.integers(120, 135, (N, nb), dtype=np.uint8)
    ref, S = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt)
    Av = _values(A, K, fmt) * _expanded_scales(SA, K)
    Bv = _values(B, K, fmt) * _expanded_scales(SB, K)
    # every product and partial sum is exact in binary64 at these ranges
    assert np.array_equal(ref, Av @ Bv.T)
    assert np.array_equal(S, np.abs(Av) @ np.abs(Bv).T)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_full_range_codes_within_binary64_summation_bound(fmt):
    """Over the whole finite range the products still are exact; only the
    binary64 sum rounds, by at most K * 2^-53 * S."""
    rng = np.random.default_rng(77)
    M, N, K = 7, 9, 150
    A, B = _rand_codes(rng, M, K, fmt, True), _rand_codes(rng, N, K, fmt, True)
    SA = rng.integers(110, 145, (M, 5), dtype=np.uint8)
    SB = rng.integers(110, 145, (N, 5), dtype=np.uint8)
    ref, S = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt)
    Av = _values(A, K, fmt) * _expanded_scales(SA, K)
    Bv = _values(B, K, fmt) * _expanded_scales(SB, K)
    assert np.all(np.abs(ref - Av @ Bv.T) <= 2 * K * 2.0 ** -53 * S)


def test_mixed_formats_and_addend():
    rng = np.random.default_rng(5)
    M, N, K = 6, 5, 96
    A = _rand_codes(rng, M, K, "e4m3")
    B = _rand_codes(rng, N, K, "e5m2")
    SA = rng.integers(124, 131, (M, 3), dtype=np.uint8)
    SB = rng.integers(124, 131, (N, 3), dtype=np.uint8)
    C = rng.integers(-50, 50, (M, N)).astype(np.float64)
    ref, _ = oracle.mx_gemm_f64(A, SA, B, SB, K, "e4m3", "e5m2", C)
    Av = _values(A, K, "e4m3") * _expanded_scales(SA, K)
    Bv = _values(B, K, "e5m2") * _expanded_scales(SB, K)
    assert np.array_equal(ref, Av @ Bv.T + C)


ONE = {"e4m3": 0x38, "e5m2": 0x3C, "e2m1": 0x22}   # 1.0 (e2m1: two per byte)


def _ones(rows, K, fmt):
    w = (K + 1) // 2 if fmt == "e2m1" else K
    return np.full((rows, w), ONE[fmt], dtype=np.uint8)


@pytest.mark.parametrize("fmt", FMTS)
def test_closed_form_one_scaled_block(fmt):
    """All elements 1.0 and all scales 2^0 give K; doubling the scale of block t
    of row i (of column j) adds exactly the number of k in that block."""
    M, N, K = 4, 3, 100                  # blocks of 32, 32, 32 and a tail of 4
    nb = 4
    A, B = _ones(M, K, fmt), _ones(N, K, fmt)
    SA = np.full((M, nb), 127, dtype=np.uint8)
    SB = np.full((N, nb), 127, dtype=np.uint8)
    ref, S = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt)
    assert np.array_equal(ref, np.full((M, N), float(K))) and np.array_equal(S, ref)
    for t, size in enumerate([32, 32, 32, 4]):
        SA2 = SA.copy()
        SA2[2, t] = 128
        ref, _ = oracle.mx_gemm_f64(A, SA2, B, SB, K, fmt, fmt)
        want = np.full((M, N), float(K))
        want[2, :] += size
        assert np.array_equal(ref, want), t
        SB2 = SB.copy()
        SB2[1, t] = 125                   # 2^-2: the block counts a quarter
        ref, _ = oracle.mx_gemm_f64(A, SA, B, SB2, K, fmt, fmt)
        want = np.full((M, N), float(K))
        want[:, 1] -= 0.75 * size
        assert np.array_equal(ref, want), t


def test_e2m1_nibble_order():
    """Element 2t sits in the low nibble of byte t: with A's bytes 0x21 (low
    nibble 0.5, high nibble 1.0) and B = 1.0 at even k and 0 at odd k, every
    output is (K/2) * 0.5."""
    K = 64
    A = np.full((2, K // 2), 0x21, dtype=np.uint8)
    B = np.full((3, K // 2), 0x02, dtype=np.uint8)
    S1 = np.full((2, 2), 127, dtype=np.uint8)
    S2 = np.full((3, 2), 127, dtype=np.uint8)
    ref, _ = oracle.mx_gemm_f64(A, S1, B, S2, K, "e2m1", "e2m1")
    assert np.array_equal(ref, np.full((2, 3), K / 2 * 0.5))


def test_b_is_given_column_by_column():
    """B's rows are its columns: B row j holding 1.0 only at k = j makes the
    product pick column j of A."""
    rng = np.random.default_rng(9)
    M, N, K = 5, 4, 32
    A = _rand_codes(rng, M, K, "e4m3")
    B = np.zeros((N, K), dtype=np.uint8)
    B[np.arange(N), np.arange(N)] = ONE["e4m3"]
    SA = np.full((M, 1), 127, dtype=np.uint8)
    SB = np.full((N, 1), 127, dtype=np.uint8)
    ref, _ = oracle.mx_gemm_f64(A, SA, B, SB, K, "e4m3", "e4m3")
    assert np.array_equal(ref, _values(A, K, "e4m3")[:, :N])


def test_nan_scale_poisons_only_its_rows():
    M, N, K = 3, 2, 64
    A, B = _ones(M, K, "e4m3"), _ones(N, K, "e4m3")
    SA = np.full((M, 2), 127, dtype=np.uint8)
    SB = np.full((N, 2), 127, dtype=np.uint8)
    SA[1, 1] = 255
    ref, _ = oracle.mx_gemm_f64(A, SA, B, SB, K, "e4m3", "e4m3")
    assert np.isnan(ref[1]).all() and np.array_equal(ref[[0, 2]], np.full((2, N), 64.0))


def test_sampled_positions_equal_full_product():
    rng = np.random.default_rng(11)
    M, N, K = 13, 11, 160
    for fmt in FMTS:
        A, B = _rand_codes(rng, M, K, fmt), _rand_codes(rng, N, K, fmt)
        SA = rng.integers(118, 137, (M, 5), dtype=np.uint8)
        SB = rng.integers(118, 137, (N, 5), dtype=np.uint8)
        C = rng.standard_normal((M, N))
        ref, S = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt, C)
        ii = rng.integers(0, M, 40)
        jj = rng.integers(0, N, 40)
        r2, s2 = oracle.mx_gemm_f64_at(A, SA, B, SB, K, fmt, fmt, C, ii, jj)
        assert np.array_equal(r2, ref[ii, jj]) and np.array_equal(s2, S[ii, jj])


def test_empty_dimensions():
    z = np.zeros((0, 4), dtype=np.uint8)
    s = np.zeros((0, 1), dtype=np.uint8)
    ref, S = oracle.mx_gemm_f64(z, s, _ones(3, 4, "e4m3"), np.full((3, 1), 127, np.uint8), 4, "e4m3", "e4m3")
    assert ref.shape == (0, 3)
    ref, S = oracle.mx_gemm_f64(np.zeros((2, 0), np.uint8), np.zeros((2, 0), np.uint8),
                                np.zeros((3, 0), np.uint8), np.zeros((3, 0), np.uint8), 0, "e4m3", "e4m3")
    assert np.array_equal(ref, np.zeros((2, 3)))


# ---------------------------------------------------------------- binary32 acceptance


def test_ulp_f32_matches_numpy_spacing():
    rng = np.random.default_rng(3)
    x = np.ldexp(rng.uniform(1, 2, 500), rng.integers(-120, 120, 500)).astype(np.float32)
    got = oracle.ulp_f32(x.astype(np.float64))
    assert np.array_equal(got, np.spacing(np.abs(x)).astype(np.float64))
    assert oracle.ulp_f32(np.array([0.0]))[0] == 2.0 ** -149


def test_tol_check_f32_accepts_rounded_and_rejects_outside():
    rng = np.random.default_rng(4)
    ref = rng.standard_normal(1000) * 3
    S = np.abs(ref) * 4
    got = ref.astype(np.float32)
    n, worst, _ = oracle.tol_check_f32(got, ref, S)
    assert n == 0 and worst <= 1.0
    bound = oracle.ulp_f32(ref) + np.ldexp(S, -20)
    bad = (ref + 3 * bound).astype(np.float32)
    n, worst, first = oracle.tol_check_f32(bad, ref, S)
    assert n == 1000 and first == 0
    g = got.copy()
    g[7] = np.nan
    n, worst, first = oracle.tol_check_f32(g, ref, S)
    assert n == 1 and first == 7 and worst == np.inf


# ---------------------------------------------------------------- planted mistakes


def _mx_pins_pass(gemm):
    """The closed-form pins above, against a candidate `gemm(A, SA, B, SB, K, fmt)`."""
    try:
        for fmt in FMTS:
            M, N, K = 4, 3, 100
            A, B = _ones(M, K, fmt), _ones(N, K, fmt)
            SA = np.full((M, 4), 127, dtype=np.uint8)
            SB = np.full((N, 4), 127, dtype=np.uint8)
            for t, size in enumerate([32, 32, 32, 4]):
                SA2 = SA.copy()
                SA2[2, t] = 128
                want = np.full((M, N), float(K))
                want[2, :] += size
                if not np.array_equal(gemm(A, SA2, B, SB, K, fmt), want):
                    return False
                SB2 = SB.copy()
                SB2[1, t] = 125
                want = np.full((M, N), float(K))
                want[:, 1] -= 0.75 * size
                if not np.array_equal(gemm(A, SA, B, SB2, K, fmt), want):
                    return False
        K = 64
        A = np.full((2, K // 2), 0x21, dtype=np.uint8)
        B = np.full((3, K // 2), 0x02, dtype=np.uint8)
        if not np.array_equal(gemm(A, np.full((2, 2), 127, np.uint8), B, np.full((3, 2), 127, np.uint8), K, "e2m1"),
                              np.full((2, 3), K / 2 * 0.5)):
            return False
        rng = np.random.default_rng(9)
        M, N, K = 5, 4, 32
        A = _rand_codes(rng, M, K, "e4m3")
        B = np.zeros((N, K), dtype=np.uint8)
        B[np.arange(N), np.arange(N)] = ONE["e4m3"]
        if not np.array_equal(gemm(A, np.full((M, 1), 127, np.uint8), B, np.full((N, 1), 127, np.uint8), K, "e4m3"),
                              _values(A, K, "e4m3")[:, :N]):
            return False
    except (ValueError, IndexError):
        return False
    return True


def test_mx_pins_reject_planted_mistakes():
    def good(A, SA, B, SB, K, f):
        return oracle.mx_gemm_f64(A, SA, B, SB, K, f, f)[0]

    def block_of_16(A, SA, B, SB, K, f):        # scale index k / 16 instead of k / 32
        nb = (K + 15) // 16
        ex = lambda S: np.ascontiguousarray(np.repeat(S, 2, axis=1)[:, :nb])
        return np.array([[sum(  # brute force with the wrong block size
            oracle.mx_decode(np.array([A[i, k] if f != "e2m1" else (A[i, k // 2] >> (4 * (k & 1))) & 15], np.uint8), f)[0]
            * oracle.mx_decode(np.array([B[j, k] if f != "e2m1" else (B[j, k // 2] >> (4 * (k & 1))) & 15], np.uint8), f)[0]
            * 2.0 ** (int(SA[i, k // 16 if k // 16 < SA.shape[1] else -1]) - 127)
            * 2.0 ** (int(SB[j, k // 16 if k // 16 < SB.shape[1] else -1]) - 127)
            for k in range(K)) for j in range(B.shape[0])] for i in range(A.shape[0])]) if ex else None

    def scales_swapped(A, SA, B, SB, K, f):     # A's scales used for B's columns and back
        if SA.shape[0] != SB.shape[0]:
            n = min(SA.shape[0], SB.shape[0])
            SA, SB = SA.copy(), SB.copy()
            SA[:n], SB[:n] = SB[:n].copy(), SA[:n].copy()
            return oracle.mx_gemm_f64(A, SA, B, SB, K, f, f)[0]
        return oracle.mx_gemm_f64(A, SB, B, SA, K, f, f)[0]

    def block_shifted(A, SA, B, SB, K, f):      # off-by-one block index
        return oracle.mx_gemm_f64(A, np.ascontiguousarray(np.roll(SA, 1, axis=1)), B, SB, K, f, f)[0]

    def nibbles_swapped(A, SA, B, SB, K, f):
        if f == "e2m1":
            A = ((A >> 4) | (A << 4)).astype(np.uint8)
        return oracle.mx_gemm_f64(A, SA, B, SB, K, f, f)[0]

    def last_block_dropped(A, SA, B, SB, K, f):
        return oracle.mx_gemm_f64(A, SA, B, SB, 32 * ((K - 1) // 32), f, f)[0]

    def b_transposed(A, SA, B, SB, K, f):       # B read as K x N, rows of k
        N = B.shape[0]
        w = B.shape[1]
        Bt = np.ascontiguousarray(B.T.reshape(N, w)) if f != "e2m1" else np.ascontiguousarray(B[::-1])
        return oracle.mx_gemm_f64(A, SA, Bt, SB, K, f, f)[0]

    def scale_unbiased(A, SA, B, SB, K, f):     # 2^e instead of 2^(e - 127), rescaled by a constant
        return oracle.mx_gemm_f64(A, SA, B, SB, K, f, f)[0] * 2.0 ** (127 - 127 + 1)

    assert _mx_pins_pass(good)
    for bad in (block_of_16, scales_swapped, block_shifted, nibbles_swapped, last_block_dropped,
                b_transposed, scale_unbiased):
        assert not _mx_pins_pass(bad), bad.__name__


# ---------------------------------------------------------------- MX acceptance rule


def test_run_sums_closed_forms():
    """S8 = sum over runs of 8 consecutive k of the largest |product|."""
    for K in (64, 100):                     # 100: a last run of 4
        A, B = _ones(3, K, "e4m3"), _ones(2, K, "e4m3")
        SA = np.full((3, 4), 127, np.uint8)
        SB = np.full((2, 4), 127, np.uint8)
        ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, "e4m3", "e4m3", runs=True)
        assert np.array_equal(S8, np.full((3, 2), float(-(-K // 8))))
        # one product of 2 (code 0x40) at the start of every run: each run's max is 2
        A2 = A.copy()
        A2[:, 0::8] = 0x40
        ref, S, S8 = oracle.mx_gemm_f64(A2, SA, B, SB, K, "e4m3", "e4m3", runs=True)
        assert np.array_equal(S8, np.full((3, 2), 2.0 * -(-K // 8)))
        assert np.array_equal(S, np.full((3, 2), float(K + -(-K // 8))))


def test_run_sums_bounds_and_sampled_positions():
    rng = np.random.default_rng(12)
    M, N, K = 9, 7, 200
    for fmt in FMTS:
        A, B = _rand_codes(rng, M, K, fmt), _rand_codes(rng, N, K, fmt)
        SA = rng.integers(120, 135, (M, 7), dtype=np.uint8)
        SB = rng.integers(120, 135, (N, 7), dtype=np.uint8)
        ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt, runs=True)
        assert np.all(S8 <= S) and np.all(8 * S8 >= S)
        Av = _values(A, K, fmt) * _expanded_scales(SA, K)
        Bv = _values(B, K, fmt) * _expanded_scales(SB, K)
        P = np.abs(Av[:, None, :] * Bv[None, :, :])
        want = sum(P[:, :, 8 * q:8 * q + 8].max(axis=2) for q in range(K // 8))
        assert np.array_equal(S8, want)
        ii, jj = rng.integers(0, M, 20), rng.integers(0, N, 20)
        r2, s2, s82 = oracle.mx_gemm_f64_at(A, SA, B, SB, K, fmt, fmt, None, ii, jj, runs=True)
        assert np.array_equal(s82, S8[ii, jj]) and np.array_equal(r2, ref[ii, jj])


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
def test_mx_rule_bound_is_the_sum_of_its_three_terms(out):
    rng = np.random.default_rng(8)
    ref = rng.standard_normal(500) * 4
    S = np.abs(ref) * 8
    S8 = S / 3
    if out == "f32":
        ulp = oracle.ulp_f32(ref)
    else:
        ulp = oracle.ulp_out(ref, out)
    bound = ulp + np.ldexp(S, -20) + np.ldexp(S8, -10)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out]

    def enc(x):
        t = torch.from_numpy(x).to(dt)
        return t.numpy() if out == "f32" else t.view(torch.int16).numpy().view(np.uint16)

    inside = ref + 0.9 * bound * np.sign(rng.standard_normal(500))
    g = enc(inside)
    # the stored value may round past the bound only by the rounding of the output type
    back = g.astype(np.float64) if out == "f32" else oracle.decode(g, out)
    ok = np.abs(back - ref) <= bound
    n, worst, _ = oracle.mx_tol_check(g, out, ref, S, S8)
    assert n == int((~ok).sum())
    outside = enc(ref + 4 * bound)
    n, worst, first = oracle.mx_tol_check(outside, out, ref, S, S8)
    assert n == 500 and first == 0 and worst > 1
    # without the run term the rule is the 16-bit contract
    if out != "f32":
        g2 = enc(ref)
        assert oracle.mx_tol_check(g2, out, ref, S, None)[0] == oracle.tol_check(g2, ref, S, out)[0] == 0


def test_mx_rule_rejects_one_misscaled_block():
    """The run term is loose enough for the instruction and tight enough to
    catch a wrong scale on a single 32-k block of one row."""
    rng = np.random.default_rng(13)
    M, N, K = 16, 16, 1024
    for fmt in ("e4m3", "e5m2", "e2m1"):
        A, B = _rand_codes(rng, M, K, fmt, fmt != "e2m1"), _rand_codes(rng, N, K, fmt, fmt != "e2m1")
        SA = rng.integers(122, 127, (M, 32), dtype=np.uint8)
        SB = rng.integers(122, 127, (N, 32), dtype=np.uint8)
        ref, S, S8 = oracle.mx_gemm_f64(A, SA, B, SB, K, fmt, fmt, runs=True)
        SA2 = SA.copy()
        SA2[5, 17] += 1                     # block 17 of row 5 counted twice
        bad, _ = oracle.mx_gemm_f64(A, SA2, B, SB, K, fmt, fmt)
        g = torch.from_numpy(bad.astype(np.float32)).numpy()
        n, _, _ = oracle.mx_tol_check(g, "f32", ref, S, S8)
        rows = np.unique(np.argwhere(np.abs(bad - ref) > 0)[:, 0])
        assert list(rows) == [5]
        assert n >= 8, (fmt, n)             # at least half of row 5's 16 outputs are caught


# ---------------------------------------------------------------- FP6 elements and mixed widths

FP6 = {"e2m3": (2, 3, 1), "e3m2": (3, 2, 3)}   # exponent bits, fraction bits, bias


def _fp6_embedding(c, fmt):
    """Value of a 6-bit code through binary32: a normal code (s, e, m) is the
    binary32 number with exponent field e - bias + 127 and the fraction bits
    m at the top of its fraction; a subnormal one is m units of the smallest
    subnormal, 2^(1 - bias - fraction bits)."""
    eb, mb, bias = FP6[fmt]
    s, e, m = c >> 5, (c >> mb) & ((1 << eb) - 1), c & ((1 << mb) - 1)
    if e == 0:
        v = m * 2.0 ** (1 - bias - mb)
    else:
        v = float(np.uint32((e - bias + 127) << 23 | m << (23 - mb)).view(np.float32))
    return -v if s else v


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_decode_matches_binary32_embedding_and_fp8_subsets(fmt):
    codes = np.arange(64, dtype=np.uint8)
    got = oracle.mx_decode(codes, fmt)
    for c in range(64):
        assert got[c] == _fp6_embedding(c, fmt), (fmt, c)
    assert np.array_equal(oracle.mx_decode(codes | 0xC0, fmt), got)    # only the low 6 bits
    # OCP MX extremes: E2M3 max 7.5, min normal 1, min subnormal 1/8;
    # E3M2 max 28, min normal 1/4, min subnormal 1/16; no infinities or NaNs
    pos = np.sort(got[:32])
    want = {"e2m3": (7.5, 1.0, 0.125), "e3m2": (28.0, 0.25, 0.0625)}[fmt]
    assert (pos[-1], pos[1]) == (want[0], want[2]) and np.isfinite(got).all()
    assert np.min(np.abs(got[(codes & 31) >= (8 if fmt == "e2m3" else 4)])) == want[1]
    assert len(set(pos.tolist())) == 32 and np.all(np.diff(got[:32]) > 0)   # increasing in the code
    assert np.array_equal(got[32:], -got[:32])
    # every E2M3 value is a float8 E4M3 value and every E3M2 one a float8 E5M2
    # value: torch's float8 conversion returns each exactly
    dt = torch.float8_e4m3fn if fmt == "e2m3" else torch.float8_e5m2
    t = torch.from_numpy(got.astype(np.float32)).to(dt).to(torch.float64).numpy()
    assert np.array_equal(t, got)


def _unpack6(row, K):
    """FP6 codes of a stored row by a route of the test's own: the bytes as
    one big little-endian integer, 6 bits at a time."""
    big = int.from_bytes(bytes(row.tolist()), "little")
    return np.array([(big >> (6 * k)) & 63 for k in range(K)], dtype=np.uint8)


def test_fp6_packing_worked_example_and_round_trip():
    import gemm_inputs
    # bytes 0xC1 0x0F 0x40: bits (low first) 100000 111111 000000 000010
    row = np.array([0xC1, 0x0F, 0x40], np.uint8)
    assert list(oracle.fp6_codes(row, 4)) == [1, 63, 0, 16]
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 64, (5, 96)).astype(np.uint8)
    packed = gemm_inputs.pack_fp6(codes)
    assert packed.shape == (5, 72)
    for i in range(5):
        assert np.array_equal(oracle.fp6_codes(packed[i], 96), codes[i])
        assert np.array_equal(_unpack6(packed[i], 96), codes[i])


def _codes_any(rng, rows, K, fmt):
    """Random codes of any supported format, packed as it is stored."""
    import gemm_inputs
    if fmt in FP6:
        return gemm_inputs.pack_fp6(rng.integers(0, 64, (rows, K)).astype(np.uint8))
    return _rand_codes(rng, rows, K, fmt)


def _values_any(codes, K, fmt):
    if fmt in FP6:
        table = np.array([_fp6_embedding(c, fmt) for c in range(64)])
        return np.stack([table[_unpack6(r, K)] for r in codes])
    return _values(codes, K, fmt)


@pytest.mark.parametrize("fa,fb", [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2"), ("e4m3", "e2m1"),
                                   ("e2m1", "e5m2"), ("e3m2", "e2m1"), ("e4m3", "e2m3")])
def test_fp6_and_mixed_width_products_equal_blas(fa, fb):
    """Products of FP6 operands and of operands of different widths against
    BLAS on operands dequantized by the test's own route (its own unpacking
    and binary32 embedding, torch's float8 decoders); every sum is exact."""
    rng = np.random.default_rng(len(fa) * 7 + len(fb) + ord(fa[1]) + 3 * ord(fb[3]))
    M, N, K = 9, 11, 160
    A, B = _codes_any(rng, M, K, fa), _codes_any(rng, N, K, fb)
    SA = rng.integers(120, 135, (M, 5), dtype=np.uint8)
    SB = rng.integers(120, 135, (N, 5), dtype=np.uint8)
    ref, S = oracle.mx_gemm_f64(A, SA, B, SB, K, fa, fb)
    Av = _values_any(A, K, fa) * _expanded_scales(SA, K)
    Bv = _values_any(B, K, fb) * _expanded_scales(SB, K)
    assert np.array_equal(ref, Av @ Bv.T)
    assert np.array_equal(S, np.abs(Av) @ np.abs(Bv).T)
