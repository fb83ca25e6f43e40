"""Pins of the integer oracle (CPU): oracle.gemm_i8 against what the mathematics
fixes, not against a retyping of its own loop.

* brute force with Python's unbounded integers on every tiny shape;
* numpy's int64 matrix product (a library routine) on random operands;
* closed forms: all-equal entries, identity, permutation, rank one, the
  extreme codes -128 x -128;
* the residue modulo 2^32 (an int32 accumulator wraps; it does not
  saturate), checked against a worked value computed here by hand;
* an addend, and strided operands (B stored N x K passed as a view);
* a planted-mistake test: wrong variants of the product (a dropped k term,
  a saturating accumulator, B read transposed, the addend ignored, the sign of
  the int8 codes lost) each fail one of these pins.
"""
import itertools

import numpy as np
import pytest

import oracle

CODES = np.array([-128, -127, -64, -1, 0, 1, 2, 63, 126, 127], np.int8)


def _residue(x):
    """x mod 2^32 as a signed 32-bit value, by Python arithmetic."""
    r = int(x) % (1 << 32)
    return r - (1 << 32) if r >= (1 << 31) else r


def _brute(A, B, C):
    M, K = A.shape
    N = B.shape[1]
    ex = [[sum(int(A[i, k]) * int(B[k, j]) for k in range(K)) + (int(C[i, j]) if C is not None else 0)
           for j in range(N)] for i in range(M)]
    return ex


def _pins(gemm):
    """Every pin on one implementation `gemm(A, B, C) -> (D int32, exact int64)`;
    returns the names of the failing pins."""
    bad = []
    rng = np.random.default_rng(7)
    # brute force on every tiny shape
    for M, N, K in itertools.product((1, 2, 3), repeat=3):
        A = rng.choice(CODES, (M, K))
        B = rng.choice(CODES, (K, N))
        C = rng.integers(-2 ** 31, 2 ** 31, (M, N)).astype(np.int32)
        D, ex = gemm(A, B, C)
        want = _brute(A, B, C)
        if [[int(v) for v in r] for r in ex] != want or \
                [[int(v) for v in r] for r in D] != [[_residue(v) for v in r] for r in want]:
            bad.append("brute %dx%dx%d" % (M, N, K))
            break
    # numpy's int64 product
    for M, N, K in ((64, 48, 80), (37, 129, 300)):
        A = rng.integers(-128, 128, (M, K)).astype(np.int8)
        B = rng.integers(-128, 128, (K, N)).astype(np.int8)
        D, ex = gemm(A, B, None)
        if not np.array_equal(ex, A.astype(np.int64) @ B.astype(np.int64)):
            bad.append("numpy %dx%dx%d" % (M, N, K))
    # closed forms
    K = 48
    D, ex = gemm(np.full((3, K), -128, np.int8), np.full((K, 5), -128, np.int8), None)
    if not (ex == K * 16384).all():
        bad.append("extreme codes")
    D, ex = gemm(np.ones((4, K), np.int8), np.ones((K, 6), np.int8), None)
    if not (D == K).all():
        bad.append("all ones")
    B = rng.integers(-128, 128, (K, 7)).astype(np.int8)
    D, ex = gemm(np.eye(K, dtype=np.int8), B, None)
    if not np.array_equal(D, B.astype(np.int32)):
        bad.append("identity")
    perm = rng.permutation(K)
    P = np.zeros((K, K), np.int8)
    P[np.arange(K), perm] = 1
    D, ex = gemm(P, B, None)
    if not np.array_equal(D, B[perm].astype(np.int32)):
        bad.append("permutation")
    u = rng.integers(-128, 128, 5).astype(np.int8)
    v = rng.integers(-128, 128, 9).astype(np.int8)
    D, ex = gemm(np.repeat(u[:, None], K, 1), np.repeat(v[None, :], K, 0), None)
    if not np.array_equal(ex, K * np.outer(u.astype(np.int64), v.astype(np.int64))):
        bad.append("rank one")
    # the residue: 127 * 127 * 140000 = 2258060000 = 2^32 - 2036907296
    D, ex = gemm(np.full((1, 140000), 127, np.int8), np.full((140000, 2), 127, np.int8), None)
    if int(ex[0, 0]) != 2258060000 or int(D[0, 0]) != -2036907296 or int(D[0, 1]) != -2036907296:
        bad.append("wrap")
    # the addend wraps too: (2^31 - 1) + 1 -> -2^31
    D, ex = gemm(np.ones((1, 1), np.int8), np.ones((1, 1), np.int8), np.full((1, 1), 2 ** 31 - 1, np.int32))
    if int(D[0, 0]) != -2 ** 31:
        bad.append("addend wrap")
    # strided B: stored N x K, passed as its transposed view
    Bt = rng.integers(-128, 128, (11, K)).astype(np.int8)
    A = rng.integers(-128, 128, (6, K)).astype(np.int8)
    D1, _ = gemm(A, Bt.T, None)
    D2, _ = gemm(A, np.ascontiguousarray(Bt.T), None)
    if not np.array_equal(D1, D2) or not np.array_equal(D1, (A.astype(np.int64) @ Bt.T.astype(np.int64))):
        bad.append("strided")
    return bad


def test_oracle_passes_every_pin():
    assert _pins(oracle.gemm_i8) == []


def test_wrap_of_single_values():
    for x, want in ((0, 0), (2 ** 31 - 1, 2 ** 31 - 1), (2 ** 31, -2 ** 31), (-2 ** 31 - 1, 2 ** 31 - 1),
                    (2 ** 32, 0), (-1, -1), (5 * 2 ** 32 + 7, 7)):
        assert oracle.wrap_i32(x) == want


def test_empty_shapes():
    D, ex = oracle.gemm_i8(np.zeros((0, 4), np.int8), np.zeros((4, 3), np.int8))
    assert D.shape == (0, 3)
    C = np.arange(6, dtype=np.int32).reshape(2, 3)
    D, ex = oracle.gemm_i8(np.zeros((2, 0), np.int8), np.zeros((0, 3), np.int8), C)
    assert np.array_equal(D, C)


def _variant(kind):
    def gemm(A, B, C):
        A64, B64 = A.astype(np.int64), B.astype(np.int64)
        if kind == "drop last k":
            ex = A64[:, :-1] @ B64[:-1, :] if A.shape[1] > 1 else np.zeros((A.shape[0], B.shape[1]), np.int64)
        elif kind == "transposed B":
            ex = A64 @ (B64.T if B.shape[0] == B.shape[1] else B64[::-1])
        elif kind == "unsigned codes":
            ex = A.view(np.uint8).astype(np.int64) @ B.view(np.uint8).astype(np.int64)
        else:
            ex = A64 @ B64
        if C is not None and kind != "ignore C":
            ex = ex + C.astype(np.int64)
        if kind == "saturate":
            D = np.clip(ex, -2 ** 31, 2 ** 31 - 1).astype(np.int32)
        else:
            D = np.array([[_residue(v) for v in r] for r in ex], np.int64).reshape(ex.shape).astype(np.int32)
        return D, ex
    return gemm


@pytest.mark.parametrize("kind", ["drop last k", "transposed B", "unsigned codes", "ignore C", "saturate"])
def test_planted_mistakes_fail_a_pin(kind):
    assert _pins(_variant(kind)), kind
    assert _pins(_variant("none")) == []     # the reference variant itself passes
