"""Pins of the CPU oracle against facts independent of it (CPU only).

Each test checks the oracle against something other than itself: exhaustive
library conversions, exact rational arithmetic, BLAS in float64, and closed
forms of the matrix product (identity, permutation, rank-1, integer inputs).
The last test plants plausible mistakes into calls of the oracle and checks
that the closed-form pins reject every one of them.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

# ---------------------------------------------------------------- decoding


def test_decode_f16_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "f16")
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zero survives
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_bf16_exhaustive_matches_fp32_top_half():
    # bfloat16 is by definition the upper 16 bits of an IEEE binary32
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        want = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = oracle.decode(bits.astype(np.uint16), "bf16")
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    # and torch agrees
    t = torch.from_numpy(bits.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    tw = t.to(torch.float64).numpy()
    assert np.array_equal(got[~nan], tw[~nan])


def test_decode_special_values():
    assert oracle.decode(np.array([0x0001], np.uint16), "f16")[0] == 2.0 ** -24
    assert oracle.decode(np.array([0x03FF], np.uint16), "f16")[0] == 1023 * 2.0 ** -24
    assert oracle.decode(np.array([0x0400], np.uint16), "f16")[0] == 2.0 ** -14
    assert oracle.decode(np.array([0x7BFF], np.uint16), "f16")[0] == 65504.0
    assert oracle.decode(np.array([0x3C00], np.uint16), "f16")[0] == 1.0
    assert oracle.decode(np.array([0x3F80], np.uint16), "bf16")[0] == 1.0
    assert oracle.decode(np.array([0x0001], np.uint16), "bf16")[0] == 2.0 ** -133
    assert math.isinf(oracle.decode(np.array([0xFC00], np.uint16), "f16")[0])


# ---------------------------------------------------------------- encoding


def _f16_values():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)       # all finite non-negative fp16
    return bits.view(np.float16).astype(np.float64)


def test_encode_f16_matches_numpy_on_values_and_midpoints():
    v = _f16_values()
    mids = (v[:-1] + v[1:]) / 2.0                        # exact in binary64
    eps = np.abs(mids) * 2.0 ** -40 + 2.0 ** -60
    xs = np.concatenate([v, mids, mids + eps, mids - eps, [65504.0, 65519.99, 65520.0, 1e6]])
    xs = np.concatenate([xs, -xs])
    got = oracle.encode_rne(xs, "f16")
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)   # numpy rounds binary64 -> binary16 RNE
    assert np.array_equal(got, want)


def test_encode_bf16_matches_torch_on_fp32_representable_inputs():
    rng = np.random.default_rng(7)
    b = rng.integers(0, 0x7F80, size=20000).astype(np.uint32)
    vals = (b << 16).view(np.float32).astype(np.float64)
    nxt = ((b + 1) << 16).view(np.float32).astype(np.float64)
    mids = (vals + nxt) / 2.0                            # 9 significant bits: exact in fp32
    rand32 = rng.standard_normal(20000).astype(np.float32).astype(np.float64)
    xs = np.concatenate([vals, mids, rand32, -mids])
    got = oracle.encode_rne(xs, "bf16")
    want = torch.from_numpy(xs.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got, want.view(np.uint16))


def test_encode_decode_round_trip_exhaustive():
    for dt, top in (("f16", 0x7C00), ("bf16", 0x7F80)):
        bits = np.arange(0, top, dtype=np.uint32).astype(np.uint16)
        allb = np.concatenate([bits, bits | 0x8000])
        assert np.array_equal(oracle.encode_rne(oracle.decode(allb, dt), dt), allb)


# ---------------------------------------------------------------- ulp


def test_ulp_out_worked_values():
    f16 = {1.0: 2.0 ** -10, 0.75: 2.0 ** -11, 0.0: 2.0 ** -24, 2.0 ** -20: 2.0 ** -24,
           65504.0: 32.0, -3.0: 2.0 ** -9, 1024.0: 1.0, 2.0 ** -14: 2.0 ** -24}
    for x, u in f16.items():
        assert oracle.ulp_out(np.array([x]), "f16")[0] == u, x
    bf16 = {1.0: 2.0 ** -7, 0.0: 2.0 ** -133, 3.0: 2.0 ** -6, 2.0 ** -130: 2.0 ** -133}
    for x, u in bf16.items():
        assert oracle.ulp_out(np.array([x]), "bf16")[0] == u, x


def test_ulp_out_f16_matches_numpy_spacing():
    v = _f16_values()[:-1]                               # spacing of the max is inf
    want = np.spacing(v.astype(np.float16)).astype(np.float64)
    assert np.array_equal(oracle.ulp_out(v, "f16"), want)


# ---------------------------------------------------------------- small exact products

F16_SET = [-2.0, -1.0, -0.5, -(2.0 ** -24), 0.0, 2.0 ** -24, 0.5, 1.0, 2.0, 1.5, -0.75]
BF16_SET = [-2.0, -1.0, -0.5, -(2.0 ** -20), 0.0, 2.0 ** -20, 0.5, 1.0, 2.0, 1.5, -0.75]


def _bits_of(vals, dt):
    return oracle.encode_rne(np.asarray(vals, dtype=np.float64), dt)


def _exact(Av, Bv, Cv=None):
    M, K = Av.shape
    N = Bv.shape[1]
    ref = np.empty((M, N), dtype=object)
    S = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            terms = [Fraction(float(Av[i, k])) * Fraction(float(Bv[k, j])) for k in range(K)]
            r = sum(terms, Fraction(0))
            if Cv is not None:
                r += Fraction(float(Cv[i, j]))
            ref[i, j] = r
            S[i, j] = sum((abs(t) for t in terms), Fraction(0))
    return ref, S


@pytest.mark.parametrize("dt,vals", [("f16", F16_SET), ("bf16", BF16_SET)])
def test_brute_force_tiny_shapes_are_exact(dt, vals):
    rng = np.random.default_rng(11)
    for M, N, K in itertools.product((1, 2, 3), repeat=3):
        for with_c in (False, True):
            Av = rng.choice(vals, size=(M, K))
            Bv = rng.choice(vals, size=(K, N))
            Cv = rng.choice(vals, size=(M, N)) if with_c else None
            A, B = _bits_of(Av, dt), _bits_of(Bv, dt)
            C = _bits_of(Cv, dt) if with_c else None
            ref, S = oracle.gemm_f64(A, B, C, dt)
            eref, eS = _exact(Av, Bv, Cv)
            for i in range(M):
                for j in range(N):
                    # dyadic values spanning < 53 bits: the fp64 sum is exact
                    assert Fraction(ref[i, j]) == eref[i, j], (M, N, K, i, j)
                    assert Fraction(S[i, j]) == eS[i, j]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_random_values_within_fp64_summation_bound(dt):
    rng = np.random.default_rng(12)
    M, N, K = 5, 7, 19
    A = _bits_of(rng.uniform(-1, 1, (M, K)), dt)
    B = _bits_of(rng.uniform(-1, 1, (K, N)), dt)
    C = _bits_of(rng.uniform(-1, 1, (M, N)), dt)
    ref, S = oracle.gemm_f64(A, B, C, dt)
    eref, eS = _exact(oracle.decode(A, dt), oracle.decode(B, dt), oracle.decode(C, dt))
    for i in range(M):
        for j in range(N):
            bound = Fraction((K + 1) * 2.0 ** -53) * (eS[i, j] + 1)
            assert abs(Fraction(ref[i, j]) - eref[i, j]) <= bound


@pytest.mark.parametrize("shape", [(64, 48, 80), (257, 129, 300)])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_matches_blas_float64(shape, dt):
    M, N, K = shape
    rng = np.random.default_rng(13)
    A = _bits_of(rng.uniform(-1, 1, (M, K)), dt)
    B = _bits_of(rng.uniform(-1, 1, (K, N)), dt)
    ref, S = oracle.gemm_f64(A, B, None, dt)
    blas = oracle.decode(A, dt) @ oracle.decode(B, dt)
    assert np.all(np.abs(ref - blas) <= 2 * K * 2.0 ** -53 * S + 1e-300)
    absS = np.abs(oracle.decode(A, dt)) @ np.abs(oracle.decode(B, dt))
    assert np.allclose(S, absS, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- closed forms


def _rand_bits(rng, shape, dt, subnormals=False):
    x = rng.uniform(-1, 1, shape)
    if subnormals:
        tiny = 2.0 ** -20 if dt == "f16" else 2.0 ** -130
        mask = rng.random(shape) < 0.2
        x[mask] *= tiny
    return _bits_of(x, dt)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_identity_left_and_right(dt):
    rng = np.random.default_rng(14)
    M, N = 37, 23
    B = _rand_bits(rng, (M, N), dt, subnormals=True)
    I_m = _bits_of(np.eye(M), dt)
    ref, _ = oracle.gemm_f64(I_m, B, None, dt)
    assert np.array_equal(ref, oracle.decode(B, dt))
    A = _rand_bits(rng, (M, N), dt, subnormals=True)
    I_n = _bits_of(np.eye(N), dt)
    ref, _ = oracle.gemm_f64(A, I_n, None, dt)
    assert np.array_equal(ref, oracle.decode(A, dt))
    C = _rand_bits(rng, (M, N), dt)
    ref, _ = oracle.gemm_f64(I_m, B, C, dt)
    assert np.array_equal(ref, oracle.decode(B, dt) + oracle.decode(C, dt))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_permutations(dt):
    rng = np.random.default_rng(15)
    M, K, N = 29, 31, 17
    p = rng.permutation(K)
    P = np.zeros((M, K))
    P[np.arange(M), p[:M]] = 1.0                          # row i picks row p[i] of B
    B = _rand_bits(rng, (K, N), dt)
    ref, _ = oracle.gemm_f64(_bits_of(P, dt), B, None, dt)
    assert np.array_equal(ref, oracle.decode(B, dt)[p[:M]])
    q = rng.permutation(K)
    Q = np.zeros((K, N))
    Q[q[:N], np.arange(N)] = 1.0                          # column j picks column q[j] of A
    A = _rand_bits(rng, (M, K), dt)
    ref, _ = oracle.gemm_f64(A, _bits_of(Q, dt), None, dt)
    assert np.array_equal(ref, oracle.decode(A, dt)[:, q[:N]])


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_rank_one_closed_form(dt):
    rng = np.random.default_rng(16)
    M, N, K = 13, 11, 40
    u = 2.0 ** rng.integers(-6, 3, M) * rng.choice([-1, 1], M)
    v = 2.0 ** rng.integers(-6, 3, N) * rng.choice([-1, 1], N)
    A = _bits_of(np.repeat(u[:, None], K, axis=1), dt)
    B = _bits_of(np.repeat(v[None, :], K, axis=0), dt)
    ref, S = oracle.gemm_f64(A, B, None, dt)
    assert np.array_equal(ref, K * np.outer(u, v))
    assert np.array_equal(S, K * np.abs(np.outer(u, v)))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_integer_inputs_exact(dt):
    rng = np.random.default_rng(17)
    M, N, K = 33, 45, 28          # |D| <= 9*28 = 252 <= 256: exact in bf16 and fp16
    Ai = rng.integers(-3, 4, (M, K))
    Bi = rng.integers(-3, 4, (K, N))
    Ci = rng.integers(-3, 4, (M, N))
    ref, _ = oracle.gemm_f64(_bits_of(Ai, dt), _bits_of(Bi, dt), _bits_of(Ci, dt), dt)
    assert np.array_equal(ref, (Ai @ Bi + Ci).astype(np.float64))


def test_strided_operands_equal_contiguous_copies():
    rng = np.random.default_rng(18)
    big = _rand_bits(rng, (40, 60), "f16")
    A = big[:17, ::3]                    # 17 x 20, column stride 3
    B = big[1:21, 2:30].T.copy().T       # Fortran-ordered 20 x 28
    C = big[::2, :28][:17]
    ref, S = oracle.gemm_f64(A, B, C, "f16")
    ref2, S2 = oracle.gemm_f64(np.ascontiguousarray(A), np.ascontiguousarray(B),
                               np.ascontiguousarray(C), "f16")
    assert np.array_equal(ref, ref2) and np.array_equal(S, S2)


def test_sampled_positions_equal_full_product():
    rng = np.random.default_rng(19)
    M, N, K = 70, 50, 90
    A = _rand_bits(rng, (M, K), "bf16")
    B = _rand_bits(rng, (K, N), "bf16")
    C = _rand_bits(rng, (M, N), "bf16")
    ref, S = oracle.gemm_f64(A, B, C, "bf16")
    ii = rng.integers(0, M, 300)
    jj = rng.integers(0, N, 300)
    r2, s2 = oracle.gemm_f64_at(A, B, C, ii, jj, "bf16")
    assert np.array_equal(r2, ref[ii, jj]) and np.array_equal(s2, S[ii, jj])


def test_empty_dimensions():
    A = np.zeros((3, 0), np.uint16)
    B = np.zeros((0, 4), np.uint16)
    ref, S = oracle.gemm_f64(A, B, None, "f16")
    assert ref.shape == (3, 4) and np.all(ref == 0) and np.all(S == 0)
    C = _bits_of(np.full((3, 4), 0.5), "f16")
    ref, _ = oracle.gemm_f64(A, B, C, "f16")
    assert np.all(ref == 0.5)
    ref, _ = oracle.gemm_f64(np.zeros((0, 5), np.uint16), np.zeros((5, 2), np.uint16), None, "f16")
    assert ref.shape == (0, 2)


# ---------------------------------------------------------------- acceptance rule


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_tol_check_accepts_rounded_and_rejects_outside(dt):
    rng = np.random.default_rng(20)
    M, N, K = 40, 30, 64
    A = _rand_bits(rng, (M, K), dt)
    B = _rand_bits(rng, (K, N), dt)
    ref, S = oracle.gemm_f64(A, B, None, dt)
    good = oracle.encode_rne(ref, dt)
    n, worst, first = oracle.tol_check(good, ref, S, dt)
    assert n == 0 and worst <= 0.5 + 1e-12 and first == -1
    u = oracle.ulp_out(ref, dt)
    for sign in (1.0, -1.0):
        off = ref + sign * (2 * u + S * 2.0 ** -19)
        bad = oracle.encode_rne(off, dt)
        n, worst, first = oracle.tol_check(bad, ref, S, dt)
        assert n == M * N and worst > 1.0 and first == 0
    nanb = good.copy()
    nanb[3, 4] = 0x7E00 if dt == "f16" else 0x7FC0
    n, worst, first = oracle.tol_check(nanb, ref, S, dt)
    assert n == 1 and math.isinf(worst) and first == 3 * N + 4


def test_tol_check_bound_is_inclusive():
    ref = np.array([1.0])
    S = np.array([0.0])
    at = oracle.encode_rne(np.array([1.0 + 2.0 ** -10]), "f16")      # exactly 1 ulp away
    assert oracle.tol_check(at, ref, S, "f16")[0] == 0
    past = oracle.encode_rne(np.array([1.0 + 2.0 ** -9]), "f16")
    assert oracle.tol_check(past, ref, S, "f16")[0] == 1


# ---------------------------------------------------------------- grouped order


def test_grouped_order_hand_worked_case():
    # 5 M tiles, 3 N tiles, groups of 2: bands {0,1}, {2,3}, {4}
    got = oracle.grouped_order(5, 3, 2)
    want = [(0, 0), (1, 0), (0, 1), (1, 1), (0, 2), (1, 2),
            (2, 0), (3, 0), (2, 1), (3, 1), (2, 2), (3, 2),
            (4, 0), (4, 1), (4, 2)]
    assert got == want


def test_grouped_order_group_one_is_row_major():
    assert oracle.grouped_order(3, 4, 1) == [(m, n) for m in range(3) for n in range(4)]


# ---------------------------------------------------------------- planted mistakes


def _closed_form_pins_pass(gemm):
    """Run the identity / permutation / rank-1 / integer / addend pins against a
    candidate oracle `gemm(A, B, C, dt) -> ref`.  Returns False on the first
    mismatch."""
    rng = np.random.default_rng(21)
    dt = "f16"
    M, K, N = 9, 12, 7
    # non-symmetric, non-square operands so a transposition or swap shows
    Ai = rng.integers(-3, 4, (M, K))
    Bi = rng.integers(-3, 4, (K, N))
    Ci = rng.integers(-3, 4, (M, N))
    try:
        if not np.array_equal(gemm(_bits_of(Ai, dt), _bits_of(Bi, dt), _bits_of(Ci, dt), dt),
                              (Ai @ Bi + Ci).astype(np.float64)):
            return False
        p = rng.permutation(K)
        P = np.zeros((M, K))
        P[np.arange(M), p[:M]] = 1
        B = _rand_bits(rng, (K, N), dt)
        if not np.array_equal(gemm(_bits_of(P, dt), B, None, dt), oracle.decode(B, dt)[p[:M]]):
            return False
        u = 2.0 ** rng.integers(-3, 3, M)
        v = -(2.0 ** rng.integers(-3, 3, N))
        A1 = _bits_of(np.repeat(u[:, None], K, 1), dt)
        B1 = _bits_of(np.repeat(v[None, :], K, 0), dt)
        if not np.array_equal(gemm(A1, B1, None, dt), K * np.outer(u, v)):
            return False
    except (ValueError, IndexError):
        return False
    return True


def test_pins_reject_planted_mistakes():
    def good(A, B, C, dt):
        return oracle.gemm_f64(A, B, C, dt)[0]

    def dropped_last_term(A, B, C, dt):
        return oracle.gemm_f64(A[:, :-1], B[:-1], C, dt)[0]

    def addend_ignored(A, B, C, dt):
        return oracle.gemm_f64(A, B, None, dt)[0]

    def addend_subtracted(A, B, C, dt):
        r = oracle.gemm_f64(A, B, None, dt)[0]
        return r - oracle.decode(C, dt) if C is not None else r

    def rows_shifted(A, B, C, dt):
        return oracle.gemm_f64(np.roll(A, 1, axis=0), B, C, dt)[0]

    def k_misaligned(A, B, C, dt):
        return oracle.gemm_f64(A, np.roll(B, 1, axis=0), C, dt)[0]

    def b_read_transposed(A, B, C, dt):
        Bt = np.ascontiguousarray(B.T)
        K, N = B.shape
        # a transposed read of B, same element count, reinterpreted as K x N
        return oracle.gemm_f64(A, Bt.reshape(K, N), C, dt)[0]

    def negated(A, B, C, dt):
        return -oracle.gemm_f64(A, B, C, dt)[0]

    assert _closed_form_pins_pass(good)
    for bad in (dropped_last_term, addend_ignored, addend_subtracted, rows_shifted,
                k_misaligned, b_read_transposed, negated):
        assert not _closed_form_pins_pass(bad), bad.__name__
