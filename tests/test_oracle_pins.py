"""Pins for the CPU oracle, against facts that do not come from the oracle.

The pages print no numeric C for any input, so the oracle is pinned by the
mathematics of the problem they all state (C = alpha*A@B + beta*C, e.g. "Warp
Tiling: A Third Level of Tiling", section "The Kernel", epilogue): exact
rational brute force on tiny shapes, closed forms (identity, all-ones,
rank-1), linearity in alpha and beta, the transpose identity, a float64
library product, and the untouched-memory rule.  Each pin is chosen so that a
plausible slip in the oracle (a dropped or doubled term, a sign, a swapped
index or operand, a wrong leading dimension, a missing alpha or beta) fails.
"""
from fractions import Fraction

import numpy as np
import pytest

from fp32_gemm_amd import inputs

pytestmark = pytest.mark.filterwarnings("ignore")


def _exact(A, B, C, alpha, beta):
    M, K = A.shape
    N = B.shape[1]
    out = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
            out[i][j] = Fraction(float(alpha)) * s + Fraction(float(beta)) * Fraction(float(C[i, j]))
    return out


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_exact_rational(oracle_mod, seed):
    """fp64 oracle vs exact rationals for every M, N, K in {1,2,3,5,7}."""
    rng = np.random.default_rng(100 + seed)
    sizes = (1, 2, 3, 5, 7)
    for M in sizes:
        for N in sizes:
            for K in sizes:
                A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
                B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
                C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
                alpha = np.float32(rng.uniform(-2, 2))
                beta = np.float32(rng.uniform(-2, 2))
                C32, C64 = oracle_mod.sgemm(A, B, C, float(alpha), float(beta))
                ex = _exact(A, B, C, alpha, beta)
                for i in range(M):
                    for j in range(N):
                        scale = abs(float(alpha)) * float(np.abs(A[i].astype(np.float64)) @ np.abs(B[:, j].astype(np.float64))) \
                            + abs(float(beta) * float(C[i, j]))
                        bound = (K + 3) * 2.0 ** -52 * scale + 1e-300
                        assert abs(Fraction(float(C64[i, j])) - ex[i][j]) <= Fraction(bound), (M, N, K, i, j)
                        assert C32[i, j] == np.float32(C64[i, j])


def test_padded_leading_dimensions_and_canary(oracle_mod):
    """Padded lda/ldb/ldc: same values as tight, and every byte outside the
    M x N window of C (padding columns, guard rows before and after) keeps
    its canary bit pattern."""
    M, N, K = 13, 11, 9
    A, B, C = inputs.make_random(M, N, K, seed=7)
    ref32, _ = oracle_mod.sgemm(A, B, C, 0.75, -1.25)
    lda, ldb, ldc = K + 3, N + 5, N + 64
    guard = 4
    canary = np.uint32(0x7FC0DEAD)
    Ab = np.full(M * lda, 99.0, np.float32); Ab.reshape(M, lda)[:, :K] = A
    Bb = np.full(K * ldb, -99.0, np.float32); Bb.reshape(K, ldb)[:, :N] = B
    Cbuf = np.full((guard + M + guard) * ldc, canary, dtype=np.uint32)
    Cview = Cbuf.view(np.float32)
    body = Cview[guard * ldc:(guard + M) * ldc]
    body.reshape(M, ldc)[:, :N] = C
    rc, _ = oracle_mod.sgemm_raw(M, N, K, 0.75, Ab, lda, Bb, ldb, -1.25, body, ldc)
    assert rc == 0
    got = body.reshape(M, ldc)[:, :N]
    assert np.array_equal(got.view(np.uint32), ref32.view(np.uint32))
    mask = np.ones(Cbuf.shape, bool)
    mask[guard * ldc:(guard + M) * ldc] = np.tile(np.r_[np.zeros(N, bool), np.ones(ldc - N, bool)], M)
    assert np.all(Cbuf[mask] == canary)


@pytest.mark.parametrize("M,N", [(64, 64), (77, 150)])
def test_identity_gives_B_bit_exact(oracle_mod, M, N):
    K = M
    rng = np.random.default_rng(3)
    A = np.eye(M, dtype=np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = np.zeros((M, N), np.float32)
    C32, _ = oracle_mod.sgemm(A, B, C, 1.0, 0.0)
    assert np.array_equal(C32.view(np.uint32), B.view(np.uint32))


@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.5, 0.0), (1.0, 1.0), (0.5, 3.0), (1.0, 3.0)])
def test_all_ones_gives_K(oracle_mod, alpha, beta):
    M, N, K = 19, 23, 777
    A = np.ones((M, K), np.float32)
    B = np.ones((K, N), np.float32)
    C = np.random.default_rng(5).integers(-4, 5, (M, N)).astype(np.float32)
    C32, _ = oracle_mod.sgemm(A, B, C, alpha, beta)
    expect = (alpha * K + beta * C.astype(np.float64)).astype(np.float32)
    assert np.array_equal(C32, expect)


def test_rank1_outer_product_is_correctly_rounded(oracle_mod):
    """K = 1: each output is one product, correctly rounded to fp32 (numpy's
    float32 multiply is IEEE round-to-nearest-even)."""
    rng = np.random.default_rng(11)
    a = rng.uniform(-1, 1, (37, 1)).astype(np.float32)
    b = rng.uniform(-1, 1, (1, 41)).astype(np.float32)
    C32, _ = oracle_mod.sgemm(a, b, np.zeros((37, 41), np.float32), 1.0, 0.0)
    assert np.array_equal(C32, a * b)


def test_rank1_integer_columns(oracle_mod):
    """A = u 1^T, B = 1 v^T with small integers: C = K u_i v_j exactly."""
    M, N, K = 21, 17, 300
    rng = np.random.default_rng(12)
    u = rng.integers(-4, 5, M).astype(np.float32)
    v = rng.integers(-4, 5, N).astype(np.float32)
    A = np.repeat(u[:, None], K, axis=1)
    B = np.repeat(v[None, :], K, axis=0)
    C32, _ = oracle_mod.sgemm(A, B, np.zeros((M, N), np.float32), 1.0, 0.0)
    assert np.array_equal(C32, (K * np.outer(u, v)).astype(np.float32))


def test_alpha_beta_linearity(oracle_mod):
    M, N, K = 33, 29, 65
    A, B, C = inputs.make_random(M, N, K, seed=21)
    _, P = oracle_mod.sgemm(A, B, np.zeros_like(C), 1.0, 0.0)   # P = A@B in fp64
    for alpha, beta in [(0.5, 3.0), (-2.0, 0.25), (1.0, -1.0)]:
        _, C64 = oracle_mod.sgemm(A, B, C, alpha, beta)
        want = alpha * P + beta * C.astype(np.float64)
        assert np.max(np.abs(C64 - want)) <= 1e-13 * K
    C32, _ = oracle_mod.sgemm(A, B, C, 0.0, 3.0)
    assert np.array_equal(C32, (np.float64(3.0) * C.astype(np.float64)).astype(np.float32))


def test_transpose_identity_bit_exact(oracle_mod):
    M, N, K = 31, 47, 53
    A, B, C = inputs.make_random(M, N, K, seed=31)
    C1, _ = oracle_mod.sgemm(A, B, np.zeros((M, N), np.float32), 1.0, 0.0)
    C2, _ = oracle_mod.sgemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T),
                             np.zeros((N, M), np.float32), 1.0, 0.0)
    assert np.array_equal(C1.view(np.uint32), np.ascontiguousarray(C2.T).view(np.uint32))


def test_against_float64_library_product(oracle_mod):
    w = inputs.WORKLOADS["sq256"]
    A, B, C = inputs.make(w)
    _, C64 = oracle_mod.sgemm(A, B, C, w.alpha, w.beta)
    ref = w.alpha * (A.astype(np.float64) @ B.astype(np.float64)) + w.beta * C.astype(np.float64)
    assert np.max(np.abs(C64 - ref)) <= 1e-12 * w.K * np.abs(A).max() * np.abs(B).max()


def test_K_zero_is_beta_times_C(oracle_mod):
    M, N = 9, 10
    C = np.random.default_rng(2).uniform(-1, 1, (M, N)).astype(np.float32)
    buf = C.copy()
    rc, _ = oracle_mod.sgemm_raw(M, N, 0, 0.5, None, 1, None, N, 3.0, buf, N)
    assert rc == 0
    assert np.array_equal(buf, (3.0 * C.astype(np.float64)).astype(np.float32))


def test_argument_codes(oracle_mod):
    a = np.zeros(64, np.float32)
    f = oracle_mod.sgemm_raw
    assert f(-1, 2, 2, 1, a, 2, a, 2, 0, a, 2)[0] == -1
    assert f(2, -1, 2, 1, a, 2, a, 2, 0, a, 2)[0] == -2
    assert f(2, 2, -1, 1, a, 2, a, 2, 0, a, 2)[0] == -3
    assert f(2, 2, 2, 1, None, 2, a, 2, 0, a, 2)[0] == -5
    assert f(2, 2, 3, 1, a, 2, a, 2, 0, a, 2)[0] == -6
    assert f(2, 2, 2, 1, a, 2, None, 2, 0, a, 2)[0] == -7
    assert f(2, 3, 2, 1, a, 3, a, 2, 0, a, 3)[0] == -8
    assert f(2, 2, 2, 1, a, 2, a, 2, 0, None, 2)[0] == -10
    assert f(2, 3, 2, 1, a, 2, a, 3, 0, a, 2)[0] == -11
    assert f(0, 0, 0, 1, None, 1, None, 1, 0, None, 1)[0] == 0


def test_thread_count_does_not_change_bits(oracle_mod):
    A, B, C = inputs.make_random(70, 90, 130, seed=41)
    n0 = oracle_mod.max_threads()
    try:
        oracle_mod.set_threads(1)
        c1, _ = oracle_mod.sgemm(A, B, C, 0.5, 3.0)
        oracle_mod.set_threads(max(2, n0))
        c2, _ = oracle_mod.sgemm(A, B, C, 0.5, 3.0)
    finally:
        oracle_mod.set_threads(n0)
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))


def test_entries_match_full_product_bit_exact(oracle_mod):
    """The i-k-j row loop and the textbook per-entry dot product add the same
    terms in the same order, so they agree bit-for-bit."""
    M, N, K = 45, 67, 129
    A, B, C = inputs.make_random(M, N, K, seed=51)
    full32, full64 = oracle_mod.sgemm(A, B, C, 0.5, 3.0)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    e32, e64 = oracle_mod.entries(ii.ravel(), jj.ravel(), A, B, C, 0.5, 3.0)
    assert np.array_equal(e64.view(np.uint64), full64.ravel().view(np.uint64))
    assert np.array_equal(e32.view(np.uint32), full32.ravel().view(np.uint32))


def _fp32_sequential(A, B, tile_k=None, drop_tile=None):
    """Plain fp32 accumulation over k (what a correct GPU kernel may do), with
    an optional dropped K-tile (what a broken one might do)."""
    acc = np.zeros((A.shape[0], B.shape[1]), np.float32)
    for k in range(A.shape[1]):
        if drop_tile is not None and k // tile_k == drop_tile:
            continue
        acc = acc + np.outer(A[:, k], B[k, :]).astype(np.float32)
    return acc


def test_tolerance_separates_fp32_rounding_from_a_dropped_tile(oracle_mod):
    """The parity bar max|C-C64|/(K max|A| max|B|) <= 1e-6 accepts plain fp32
    accumulation and rejects a kernel that skips one 16-wide K-tile."""
    M, N, K = 48, 40, 777
    A, B, _ = inputs.make_random(M, N, K, seed=61)
    _, C64 = oracle_mod.sgemm(A, B, np.zeros((M, N), np.float32), 1.0, 0.0)
    den = (K, np.abs(A).max(), np.abs(B).max())
    good = oracle_mod.rel_error(_fp32_sequential(A, B), C64, *den)
    bad = oracle_mod.rel_error(_fp32_sequential(A, B, 16, 7), C64, *den)
    assert good < 1e-7
    assert bad > 1e-4
