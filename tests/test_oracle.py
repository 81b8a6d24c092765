"""Pins for the CPU oracle: it is checked against facts that do not come from itself.

Each test pins the oracle to something independent of its own code: closed
forms (identity, all-ones, W = 0), exact integer arithmetic, exact rational
arithmetic on tiny shapes, a library routine in a different summation order
(numpy float64 matmul, numpy's binary16 decoder), the worked 4x4 tile example
(page "第5章-基础Kernel", section 3.2), and invariants (ragged rows, blocking,
thread count, leading dimensions). Non-square shapes everywhere, so that a
transposed operand or swapped index fails.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def rand_f32(*shape, lo=-1.0, hi=1.0):
    return RNG.uniform(lo, hi, size=shape).astype(np.float32)


def rand_int(*shape, lo=-2, hi=2, dtype=np.float32):
    return RNG.integers(lo, hi + 1, size=shape).astype(dtype)


# ---- closed forms --------------------------------------------------------

def test_identity_left_and_right():
    K, N = 37, 53
    B = rand_f32(K, N)
    R, T = oracle.gemm(np.eye(K, dtype=np.float32), B)
    assert np.array_equal(R, B.astype(np.float64))
    assert np.array_equal(T, np.abs(B).astype(np.float64))
    A = rand_f32(29, K)
    R, _ = oracle.gemm(A, np.eye(K, dtype=np.float32))
    assert np.array_equal(R, A.astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (17, 70, 129), (1, 1, 4096)])
def test_all_ones_gives_k(M, N, K):
    R, T = oracle.gemm(np.ones((M, K), np.float32), np.ones((K, N), np.float32))
    assert np.all(R == K) and np.all(T == K)


def test_sign_and_scale_closed_form():
    # alpha = -1 on the all-ones product gives -K; beta*C with alpha = 0 gives beta*C.
    M, N, K = 4, 6, 9
    C = rand_f32(M, N)
    R, _ = oracle.gemm(np.ones((M, K), np.float32), np.ones((K, N), np.float32), alpha=-1.0)
    assert np.all(R == -K)
    R, T = oracle.gemm(rand_f32(M, K), rand_f32(K, N), alpha=0.0, beta=-0.25, C=C)
    assert np.array_equal(R, -0.25 * C.astype(np.float64))
    assert np.all(T == 0)


# ---- exact integer arithmetic -------------------------------------------

@pytest.mark.parametrize("M,N,K", [(7, 11, 13), (65, 130, 33), (128, 96, 300)])
def test_integer_matrices_exact(M, N, K):
    A = rand_int(M, K)
    B = rand_int(K, N)
    exact = A.astype(np.int64) @ B.astype(np.int64)
    R, T = oracle.gemm(A, B)
    assert np.array_equal(R, exact.astype(np.float64))
    assert np.array_equal(T, (np.abs(A.astype(np.int64)) @ np.abs(B.astype(np.int64))).astype(np.float64))


def test_integer_alpha_beta_exact():
    M, N, K = 33, 47, 65
    A, B, C = rand_int(M, K), rand_int(K, N), rand_int(M, N, lo=-4, hi=4)
    exact = [[Fraction(3, 2) * int(v) for v in row] for row in (A.astype(np.int64) @ B.astype(np.int64))]
    R, _ = oracle.gemm(A, B, alpha=1.5, beta=0.5, C=C)
    for m in range(M):
        for n in range(N):
            assert Fraction(R[m, n]) == exact[m][n] + Fraction(1, 2) * int(C[m, n])


def test_f16_integer_exact():
    M, N, K = 40, 24, 200
    A = rand_int(M, K, lo=-8, hi=8).astype(np.float16)
    B = rand_int(K, N, lo=-8, hi=8).astype(np.float16)
    exact = A.astype(np.int64) @ B.astype(np.int64)
    R, _ = oracle.gemm(A.view(np.uint16), B.view(np.uint16))
    assert np.array_equal(R, exact.astype(np.float64))


def test_linear_integer_exact():
    M, N, K = 31, 45, 77
    X, W, b = rand_int(M, K), rand_int(K, N), rand_int(N, lo=-4, hi=4)
    y = X.astype(np.int64) @ W.astype(np.int64) + b.astype(np.int64)
    R, _ = oracle.linear(X, W, b, act=1)
    assert np.array_equal(R, np.maximum(y, 0).astype(np.float64))
    R, _ = oracle.linear(X, W, b, act=0)
    assert np.array_equal(R, y.astype(np.float64))
    R, _ = oracle.linear(X, W, None, act=0)
    assert np.array_equal(R, (y - b.astype(np.int64)).astype(np.float64))


# ---- the worked example from the pages ----------------------------------

def test_worked_4x4_tile_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_4x4.json")))
    A = np.array(g["A"], np.float32)
    B = np.array(g["B"], np.float32)
    t = g["tile"]
    # the fixture's hand-worked values against plain integer arithmetic
    Ai = [[int(v) for v in r] for r in g["A"]]
    Bi = [[int(v) for v in r] for r in g["B"]]
    brute = [[sum(Ai[m][k] * Bi[k][n] for k in range(4)) for n in range(4)] for m in range(4)]
    assert brute == g["C"]
    # the oracle against the fixture
    R, _ = oracle.gemm(A, B)
    assert np.array_equal(R, np.array(g["C"], np.float64))
    # the page's tile relation C00 = A00*B00 + A01*B10, each term an oracle call
    p0, _ = oracle.gemm(A[:t, :t], B[:t, :t])
    p1, _ = oracle.gemm(A[:t, t:], B[t:, :t])
    assert np.array_equal(p0, np.array(g["A00_B00"], np.float64))
    assert np.array_equal(p1, np.array(g["A01_B10"], np.float64))
    assert np.array_equal(p0 + p1, R[:t, :t])
    assert np.array_equal(R[:t, :t], np.array(g["C00"], np.float64))
    ab = g["alpha_beta_case"]
    C = np.full((4, 4), ab["C_in_all"], np.float32)
    R2, _ = oracle.gemm(A, B, alpha=ab["alpha"], beta=ab["beta"], C=C)
    assert R2[0, 0] == ab["C00_value"]


# ---- exact rational arithmetic on tiny shapes ----------------------------

@pytest.mark.parametrize("M", [0, 1, 2, 4])
@pytest.mark.parametrize("N", [0, 1, 3])
@pytest.mark.parametrize("K", [0, 1, 2, 4])
def test_tiny_shapes_against_fractions(M, N, K):
    A, B, C = rand_f32(M, K), rand_f32(K, N), rand_f32(M, N)
    alpha, beta = -1.25, 0.75
    R, T = oracle.gemm(A, B, alpha=alpha, beta=beta, C=C)
    assert R.shape == (M, N)
    for m in range(M):
        for n in range(N):
            s = sum((Fraction(float(A[m, k])) * Fraction(float(B[k, n])) for k in range(K)), Fraction(0))
            exact = Fraction(alpha) * s + Fraction(beta) * Fraction(float(C[m, n]))
            tt = sum((abs(Fraction(float(A[m, k])) * Fraction(float(B[k, n]))) for k in range(K)), Fraction(0))
            bound = (K + 2) * 2.0 ** -52 * (abs(alpha) * float(tt) + abs(beta * float(C[m, n])))
            assert abs(float(Fraction(R[m, n]) - exact)) <= bound
            assert abs(T[m, n] - float(tt)) <= K * 2.0 ** -52 * float(tt)


@pytest.mark.parametrize("M,N,K", [(0, 3, 2), (2, 0, 3), (2, 3, 0)])
def test_linear_tiny_against_fractions(M, N, K):
    X, W, b = rand_f32(M, K), rand_f32(K, N), rand_f32(N)
    R, _ = oracle.linear(X, W, b, act=0)
    assert R.shape == (M, N)
    if K == 0:
        assert np.array_equal(R, np.broadcast_to(b.astype(np.float64), (M, N)))


# ---- library cross-check in another summation order ----------------------

@pytest.mark.parametrize("M,N,K", [(37, 53, 129), (64, 200, 1000)])
def test_against_numpy_float64(M, N, K):
    A, B = rand_f32(M, K), rand_f32(K, N)
    R, T = oracle.gemm(A, B)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    assert np.all(np.abs(R - ref) <= 2 * K * 2.0 ** -52 * T)
    Tref = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    assert np.all(np.abs(T - Tref) <= 2 * K * 2.0 ** -52 * Tref)


def test_f16_against_numpy_float64():
    M, N, K = 30, 41, 500
    A = rand_f32(M, K).astype(np.float16)
    B = rand_f32(K, N).astype(np.float16)
    R, T = oracle.gemm(A.view(np.uint16), B.view(np.uint16))
    ref = A.astype(np.float64) @ B.astype(np.float64)
    assert np.all(np.abs(R - ref) <= 2 * K * 2.0 ** -52 * T)


def test_bf16_decoder_all_patterns():
    # pinned to torch's bfloat16 -> float64 conversion on all 65536 patterns
    import torch
    bits = np.arange(65536, dtype=np.int64)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_integer_exact_and_numpy():
    import torch
    M, N, K = 36, 28, 300
    Ai = rand_int(M, K, lo=-8, hi=8)
    Bi = rand_int(K, N, lo=-8, hi=8)
    A = torch.from_numpy(Ai).to(torch.bfloat16)
    B = torch.from_numpy(Bi).to(torch.bfloat16)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    R, _ = oracle.gemm(bits(A), bits(B), bf16=True)
    assert np.array_equal(R, (Ai.astype(np.int64) @ Bi.astype(np.int64)).astype(np.float64))
    Af = torch.from_numpy(rand_f32(M, K)).to(torch.bfloat16)
    Bf = torch.from_numpy(rand_f32(K, N)).to(torch.bfloat16)
    R, T = oracle.gemm(bits(Af), bits(Bf), bf16=True)
    ref = Af.double().numpy() @ Bf.double().numpy()
    assert np.all(np.abs(R - ref) <= 2 * K * 2.0 ** -52 * T)
    # the same bits read as binary16 give a different product: the flag matters
    R16, _ = oracle.gemm(bits(Af), bits(Bf))
    assert not np.allclose(R16, R)


def test_half_decoder_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ---- epilogue semantics --------------------------------------------------

def test_beta_zero_does_not_read_c():
    M, N, K = 5, 6, 7
    C = np.full((M, N), np.nan, np.float32)
    A, B = rand_f32(M, K), rand_f32(K, N)
    # beta == 0: C is not passed at all to the routine
    R, _ = oracle.gemm(A, B, alpha=2.0, beta=0.0, C=C)
    assert np.all(np.isfinite(R))
    R1, _ = oracle.gemm(A, B)
    assert np.array_equal(R, 2.0 * R1)


def test_k_zero_gives_beta_c():
    C = rand_f32(4, 5)
    R, T = oracle.gemm(np.zeros((4, 0), np.float32), np.zeros((0, 5), np.float32), alpha=3.0, beta=0.5, C=C)
    assert np.array_equal(R, 0.5 * C.astype(np.float64)) and np.all(T == 0)
    R, _ = oracle.gemm(np.zeros((4, 0), np.float32), np.zeros((0, 5), np.float32))
    assert np.all(R == 0)


def test_linear_closed_forms():
    M, N, K = 9, 70, 33
    X, b = rand_f32(M, K), rand_f32(N, lo=-0.1, hi=0.1)
    R, _ = oracle.linear(X, np.zeros((K, N), np.float32), b, act=1)
    assert np.array_equal(R, np.broadcast_to(np.maximum(b.astype(np.float64), 0.0), (M, N)))
    assert not np.any(np.signbit(R))  # ReLU gives +0.0, never -0.0
    R, _ = oracle.linear(X, np.zeros((K, N), np.float32), b, act=0)
    assert np.array_equal(R, np.broadcast_to(b.astype(np.float64), (M, N)))
    W = rand_f32(K, N)
    R, _ = oracle.linear(X, W, None, act=0)
    G, _ = oracle.gemm(X, W)
    assert np.array_equal(R, G)


def test_relu_signed_zero_on_negative_outputs():
    X = -np.ones((2, 3), np.float32)
    W = np.ones((3, 4), np.float32)
    R, _ = oracle.linear(X, W, np.zeros(4, np.float32), act=1)
    assert np.all(R == 0) and not np.any(np.signbit(R))


# ---- invariants -----------------------------------------------------------

def test_ragged_rows_are_a_prefix():
    K, N = 96, 80
    A, B = rand_f32(128, K), rand_f32(K, N)
    R128, _ = oracle.gemm(A, B)
    R127, _ = oracle.gemm(A[:127], B)
    assert np.array_equal(R127, R128[:127])
    b = rand_f32(N, lo=-0.1, hi=0.1)
    L128, _ = oracle.linear(A, B, b)
    L127, _ = oracle.linear(A[:127], B, b)
    assert np.array_equal(L127, L128[:127])


@pytest.mark.parametrize("K", [77, 600])
@pytest.mark.parametrize("kind", ["f32", "f16", "bf16", "linear"])
def test_blocked_equals_per_element_loop(kind, K):
    # several row and column blocks, ragged both ways; K = 600 spans three k
    # chunks of the blocked loop, the last one partial
    M, N = 40, 150
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    rows, cols = rows.ravel(), cols.ravel()
    if kind == "linear":
        X, W, b = rand_f32(M, K), rand_f32(K, N), rand_f32(N)
        R, T = oracle.linear(X, W, b, act=1)
        r, t = oracle.linear_at(X, W, rows, cols, b, act=1)
    else:
        A, B, C = rand_f32(M, K), rand_f32(K, N), rand_f32(M, N)
        if kind == "f16":
            A, B = A.astype(np.float16).view(np.uint16), B.astype(np.float16).view(np.uint16)
        if kind == "bf16":   # upper halves of fp32 patterns are valid bfloat16 patterns
            A, B = (A.view(np.uint32) >> 16).astype(np.uint16), (B.view(np.uint32) >> 16).astype(np.uint16)
        bf = kind == "bf16"
        R, T = oracle.gemm(A, B, alpha=1.5, beta=0.5, C=C, bf16=bf)
        r, t = oracle.gemm_at(A, B, rows, cols, alpha=1.5, beta=0.5, C=C, bf16=bf)
    assert np.array_equal(R.ravel(), r) and np.array_equal(T.ravel(), t)


def test_thread_count_does_not_change_bits():
    A, B = rand_f32(70, 300), rand_f32(300, 90)
    R1, T1 = oracle.gemm(A, B, nthreads=1)
    R8, T8 = oracle.gemm(A, B, nthreads=max(2, oracle.max_threads()))
    assert np.array_equal(R1, R8) and np.array_equal(T1, T8)


def test_leading_dimensions():
    M, N, K = 20, 30, 40
    bigA, bigB, bigC = rand_f32(M, K + 9), rand_f32(K, N + 5), rand_f32(M, N + 3)
    A, B, C = bigA[:, :K], bigB[:, :N], bigC[:, :N]
    R, T = oracle.gemm(A, B, alpha=0.5, beta=2.0, C=C)
    Rc, Tc = oracle.gemm(A.copy(), B.copy(), alpha=0.5, beta=2.0, C=C.copy())
    assert np.array_equal(R, Rc) and np.array_equal(T, Tc)


# ---- transposed B (B given N-by-K) ------------------------------------------

@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_b_transposed_equals_explicit_transpose(fmt):
    # A*B^T with B stored N-by-K equals A*(B^T stored K-by-N), bit for bit
    M, N, K = 37, 45, 150
    A, Bt, C = rand_f32(M, K), rand_f32(N, K), rand_f32(M, N)
    kw = {}
    if fmt == "f16":
        A, Bt = A.astype(np.float16).view(np.uint16), Bt.astype(np.float16).view(np.uint16)
    elif fmt == "bf16":
        A, Bt = (A.view(np.uint32) >> 16).astype(np.uint16), (Bt.view(np.uint32) >> 16).astype(np.uint16)
        kw["bf16"] = True
    R, T = oracle.gemm(A, Bt, 1.5, 0.5, C, b_trans=True, **kw)
    R2, T2 = oracle.gemm(A, np.ascontiguousarray(Bt.T), 1.5, 0.5, C, **kw)
    assert np.array_equal(R, R2) and np.array_equal(T, T2)
    rows, cols = np.arange(M).repeat(N), np.tile(np.arange(N), M)
    r, t = oracle.gemm_at(A, Bt, rows, cols, 1.5, 0.5, C, b_trans=True, **kw)
    assert np.array_equal(r, R.ravel()) and np.array_equal(t, T.ravel())


def test_b_transposed_integer_exact():
    M, N, K = 31, 23, 90
    A, Bt = rand_int(M, K), rand_int(N, K)
    R, _ = oracle.gemm(A, Bt, b_trans=True)
    assert np.array_equal(R, (A.astype(np.int64) @ Bt.astype(np.int64).T).astype(np.float64))
    # a non-square transposed operand read the wrong way round is caught
    with pytest.raises(ValueError):
        oracle.gemm(A, Bt)


def test_linear_w_transposed():
    M, N, K = 19, 41, 66
    X, Wt, b = rand_int(M, K), rand_int(N, K), rand_int(N, lo=-4, hi=4)
    R, _ = oracle.linear(X, Wt, b, act=1, w_trans=True)
    y = X.astype(np.int64) @ Wt.astype(np.int64).T + b.astype(np.int64)
    assert np.array_equal(R, np.maximum(y, 0).astype(np.float64))
    rows, cols = np.arange(M).repeat(N), np.tile(np.arange(N), M)
    r, _ = oracle.linear_at(X, Wt, rows, cols, b, act=1, w_trans=True)
    assert np.array_equal(r, R.ravel())


# ---- batched (strided) products -------------------------------------------

def test_batched_integer_exact_against_int64_matmul():
    # distinct, non-square items: a batch index taken from the wrong operand or
    # item, or one item's result written to another, changes the exact result
    nb, M, N, K = 5, 7, 11, 13
    A, B, C = rand_int(nb, M, K), rand_int(nb, K, N), rand_int(nb, M, N, lo=-4, hi=4)
    R, _ = oracle.gemm_batched(A, B, 1.5, 0.5, C)
    want = 1.5 * np.matmul(A.astype(np.int64), B.astype(np.int64)) + 0.5 * C.astype(np.float64)
    assert np.array_equal(R, want)
    Rt, _ = oracle.gemm_batched(A, np.ascontiguousarray(B.transpose(0, 2, 1)), b_trans=True)
    assert np.array_equal(Rt, np.matmul(A.astype(np.int64), B.astype(np.int64)).astype(np.float64))


def test_batched_16bit_integer_exact():
    nb, M, N, K = 3, 9, 6, 40
    A, B = rand_int(nb, M, K, lo=-8, hi=8), rand_int(nb, K, N, lo=-8, hi=8)
    want = np.matmul(A.astype(np.int64), B.astype(np.int64)).astype(np.float64)
    Rh, _ = oracle.gemm_batched(A.astype(np.float16).view(np.uint16), B.astype(np.float16).view(np.uint16))
    bf = lambda x: (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    Rb, _ = oracle.gemm_batched(bf(A), bf(B), bf16=True)
    assert np.array_equal(Rh, want) and np.array_equal(Rb, want)


def test_batched_shared_operand_stride_zero():
    # one B for every item (batch stride 0) equals the per-item products
    nb, M, N, K = 4, 6, 8, 10
    A, B = rand_f32(nb, M, K), rand_f32(K, N)
    R, T = oracle.gemm_batched(A, np.broadcast_to(B, (nb, K, N)))
    for i in range(nb):
        Ri, Ti = oracle.gemm(A[i], B)
        assert np.array_equal(R[i], Ri) and np.array_equal(T[i], Ti)
    np.testing.assert_allclose(R, np.matmul(A.astype(np.float64), B.astype(np.float64)), rtol=0,
                               atol=1e-12)


def test_batched_empty_and_single():
    R, T = oracle.gemm_batched(np.zeros((0, 3, 4), np.float32), np.zeros((0, 4, 5), np.float32))
    assert R.shape == (0, 3, 5) and T.shape == (0, 3, 5)
    A, B = rand_f32(1, 5, 6), rand_f32(1, 6, 7)
    R, _ = oracle.gemm_batched(A, B)
    assert np.array_equal(R[0], oracle.gemm(A[0], B[0])[0])


def test_sampled_rejects_out_of_range():
    with pytest.raises(IndexError):
        oracle.gemm_at(rand_f32(3, 4), rand_f32(4, 5), [3], [0])
