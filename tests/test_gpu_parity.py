"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Tolerance (floating point): |C_gpu - r| <= 1e-4 * t + ulp_fp32(r)/2 element by
element, where r is the oracle's float64 result and t = sum_k |A[m,k]*B[k,n]|.
The half-ulp term covers the single fp32 rounding of the stored result when t
is tiny (e.g. alpha == 0 or a zero row). Integer-valued inputs must give the
oracle's result bit for bit (every partial sum is an exact fp32 integer).

Sizes: small cases span several tiles of every tile shape with ragged tails
in M, N and K and are compared in full; the full-size workloads are run in
the launch configuration the bench times (the automatic plan) and every
output element is compared with the full oracle, their integer-valued
variants bit for bit.
"""
import numpy as np
import pytest

import linear_layer_amd as ll
import oracle
from linear_layer_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32, F16 = ll.DTYPE_F32, ll.DTYPE_F16
# every tile shape the library offers, each forced in turn
T32 = list(range(ll.num_tiles(F32)))
T16 = list(range(ll.num_tiles(F16)))


@pytest.fixture(autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def np32(t):
    return t.detach().cpu().numpy()


def bits16(t):
    return wl.half_bits(t.detach().cpu())


def assert_close(gpu, R, T, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    half_ulp = np.spacing(np.abs(R).astype(np.float32)).astype(np.float64) / 2
    bound = 1e-4 * T + half_ulp
    err = np.abs(gpu - R)
    bad = ~(err <= bound)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside bound; first at flat {i}: "
                             f"gpu={gpu.ravel()[i]!r} oracle={R.ravel()[i]!r} t={T.ravel()[i]!r}")
    return float(np.max(err / np.maximum(T, 1e-300))) if err.size else 0.0


def assert_exact(gpu, R, what=""):
    want = R.astype(np.float32)
    gpu = np.asarray(gpu, dtype=np.float32)
    bad = gpu != want
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} differ; first at flat {i}: "
                             f"gpu={gpu.ravel()[i]!r} want={want.ravel()[i]!r}")


@pytest.fixture
def tile():
    """Force a tile shape for one test, restore the automatic choice after."""
    forced = []

    def force(dtype, t):
        ll.set_tile(dtype, t)
        forced.append(dtype)

    yield force
    for d in forced:
        ll.set_tile(d, -1)


@pytest.fixture
def split():
    """Force the K-split count for one test, restore the automatic choice after."""
    yield ll.set_split_k
    ll.set_split_k(-1)


@pytest.fixture
def stream_k():
    """Force stream-K on or off for one test, restore the automatic choice after."""
    yield ll.set_stream_k
    ll.set_stream_k(-1)


def run_gemm_f32(A, B, alpha=1.0, beta=0.0, C=None):
    Ad, Bd = A.to(DEV), B.to(DEV)
    Cd = (C.clone() if C is not None else torch.full((A.shape[0], B.shape[1]), float("nan"))).to(DEV)
    ll.gemm_f32(Ad, Bd, Cd, alpha, beta)
    torch.cuda.synchronize()
    return np32(Cd)


def run_gemm_f16(A, B, alpha=1.0, beta=0.0, C=None):
    Ad, Bd = A.to(DEV), B.to(DEV)
    Cd = (C.clone() if C is not None else torch.full((A.shape[0], B.shape[1]), float("nan"))).to(DEV)
    ll.gemm_f16f32(Ad, Bd, Cd, alpha, beta)
    torch.cuda.synchronize()
    return np32(Cd)


def run_gemm_bf16(A, B, alpha=1.0, beta=0.0, C=None):
    Ad, Bd = A.to(DEV), B.to(DEV)
    Cd = (C.clone() if C is not None else torch.full((A.shape[0], B.shape[1]), float("nan"))).to(DEV)
    ll.gemm_bf16f32(Ad, Bd, Cd, alpha, beta)
    torch.cuda.synchronize()
    return np32(Cd)


def run_linear(X, W, b, act):
    Xd, Wd = X.to(DEV), W.to(DEV)
    bd = b.to(DEV) if b is not None else None
    Yd = torch.full((X.shape[0], W.shape[1]), float("nan"), device=DEV)
    ll.linear_bias_act(Xd, Wd, bd, act, Yd)
    torch.cuda.synchronize()
    return np32(Yd)


def run_nt(fn, A, B, alpha=1.0, beta=0.0, C=None):
    """C = alpha*A*B^T + beta*C through one of the _nt entry points (B is N-by-K)."""
    Ad, Bd = A.to(DEV), B.to(DEV)
    Cd = (C.clone() if C is not None else torch.full((A.shape[0], B.shape[0]), float("nan"))).to(DEV)
    fn(Ad, Bd, Cd, alpha, beta)
    torch.cuda.synchronize()
    return np32(Cd)


def run_linear_nt(X, W, b, act):
    Xd, Wd = X.to(DEV), W.to(DEV)
    bd = b.to(DEV) if b is not None else None
    Yd = torch.full((X.shape[0], W.shape[0]), float("nan"), device=DEV)
    ll.linear_bias_act_nt(Xd, Wd, bd, act, Yd)
    torch.cuda.synchronize()
    return np32(Yd)


def rand(shape, seed, scale=1.0):
    return wl.uniform(shape, seed, scale)


# ---- small shapes, every tile, ragged tails ----------------------------------

SMALL = [(600, 520, 200), (257, 300, 64), (33, 70, 36), (1, 1, 4), (130, 1, 12), (1, 260, 20)]


@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_f32_small(t, M, N, K, tile):
    tile(F32, t)
    A, B = rand((M, K), 1), rand((K, N), 2)
    R, T = oracle.gemm(np32(A), np32(B))
    assert_close(run_gemm_f32(A, B), R, T, f"f32 tile {t} {M}x{N}x{K}")


@pytest.mark.parametrize("t", T32)
def test_f32_alpha_beta(t, tile):
    tile(F32, t)
    M, N, K = 300, 280, 100
    A, B, C = rand((M, K), 3), rand((K, N), 4), rand((M, N), 5)
    R, T = oracle.gemm(np32(A), np32(B), 1.5, 0.5, np32(C))
    assert_close(run_gemm_f32(A, B, 1.5, 0.5, C), R, T, f"f32 alpha/beta tile {t}")
    R, T = oracle.gemm(np32(A), np32(B), -0.75, 0.0)
    assert_close(run_gemm_f32(A, B, -0.75, 0.0), R, T, f"f32 alpha only tile {t}")


@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("M,N,K", [(301, 517, 203), (70, 33, 5), (5, 9, 1)])
def test_f32_scalar_path(t, M, N, K, tile):
    # K or N not a multiple of 4: the scalar-load kernels
    tile(F32, t)
    A, B = rand((M, K), 6), rand((K, N), 7)
    R, T = oracle.gemm(np32(A), np32(B))
    assert_close(run_gemm_f32(A, B), R, T, f"f32 scalar tile {t}")


@pytest.mark.parametrize("t", T32)
def test_f32_unaligned_views(t, tile):
    # operands starting one element into a buffer, with padded leading dims
    tile(F32, t)
    M, N, K = 150, 140, 72
    Abuf, Bbuf = rand((M, K + 5), 8), rand((K, N + 3), 9)
    A, B = Abuf[:, 1:K + 1], Bbuf[:, 1:N + 1]
    Cbuf = torch.full((M, N + 6), 7.0, device=DEV)
    C = Cbuf[:, 2:N + 2]
    ll.gemm_f32(Abuf.to(DEV)[:, 1:K + 1], Bbuf.to(DEV)[:, 1:N + 1], C, 1.0, 0.0)
    torch.cuda.synchronize()
    R, T = oracle.gemm(np32(A), np32(B))
    assert_close(np32(C), R, T, "unaligned")
    guard = np32(Cbuf)
    assert np.all(guard[:, :2] == 7.0) and np.all(guard[:, N + 2:] == 7.0)


@pytest.mark.parametrize("t", T16)
@pytest.mark.parametrize("M,N,K", [(600, 520, 192), (257, 264, 64), (33, 72, 40), (1, 8, 8)])
def test_f16_small(t, M, N, K, tile):
    tile(F16, t)
    A, B = wl.to_half(rand((M, K), 10)), wl.to_half(rand((K, N), 11))
    R, T = oracle.gemm(bits16(A), bits16(B))
    assert_close(run_gemm_f16(A, B), R, T, f"f16 tile {t} {M}x{N}x{K}")


@pytest.mark.parametrize("t", T16)
@pytest.mark.parametrize("M,N,K", [(301, 517, 203), (40, 30, 10), (3, 5, 1)])
def test_f16_scalar_path(t, M, N, K, tile):
    tile(F16, t)
    A, B = wl.to_half(rand((M, K), 12)), wl.to_half(rand((K, N), 13))
    C = rand((M, N), 14)
    R, T = oracle.gemm(bits16(A), bits16(B), 1.5, 0.5, np32(C))
    assert_close(run_gemm_f16(A, B, 1.5, 0.5, C), R, T, f"f16 scalar tile {t}")


@pytest.mark.parametrize("t", T16)
@pytest.mark.parametrize("M,N,K", [(600, 520, 192), (257, 264, 64), (33, 72, 40), (301, 517, 203)])
def test_bf16_small(t, M, N, K, tile):
    tile(F16, t)
    A, B, C = wl.to_bf16(rand((M, K), 60)), wl.to_bf16(rand((K, N), 61)), rand((M, N), 62)
    R, T = oracle.gemm(bits16(A), bits16(B), 1.5, 0.5, np32(C), bf16=True)
    assert_close(run_gemm_bf16(A, B, 1.5, 0.5, C), R, T, f"bf16 tile {t} {M}x{N}x{K}")


@pytest.mark.parametrize("t", T16)
def test_bf16_integer_exact(t, tile):
    tile(F16, t)
    M, N, K = 300, 280, 256
    A = wl.to_bf16(wl.integers((M, K), 63, -8, 8))
    B = wl.to_bf16(wl.integers((K, N), 64, -8, 8))
    R, _ = oracle.gemm(bits16(A), bits16(B), bf16=True)
    assert_exact(run_gemm_bf16(A, B), R, f"bf16 int tile {t}")


def test_bf16_is_not_read_as_fp16():
    # the same bits through both entry points give different products
    M, N, K = 64, 64, 64
    A, B = wl.to_bf16(rand((M, K), 65)), wl.to_bf16(rand((K, N), 66))
    got = run_gemm_bf16(A, B)
    R, T = oracle.gemm(bits16(A), bits16(B), bf16=True)
    assert_close(got, R, T, "bf16")
    R16, _ = oracle.gemm(bits16(A), bits16(B))
    assert not np.allclose(got, R16)


@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("with_bias", [True, False])
def test_linear_small(t, act, with_bias, tile):
    tile(F32, t)
    M, N, K = 513, 260, 96
    X, W = rand((M, K), 15, 1 / 8), rand((K, N), 16, 1 / 8)
    b = wl.bias_uniform(N, 17) if with_bias else None
    R, T = oracle.linear(np32(X), np32(W), None if b is None else np32(b), act)
    Y = run_linear(X, W, b, act)
    assert_close(Y, R, T, f"linear tile {t} act {act} bias {with_bias}")
    if act == 1:
        assert not np.any(np.signbit(Y))  # +0.0 for y <= 0


@pytest.mark.parametrize("t", T32)
def test_linear_scalar_path(t, tile):
    tile(F32, t)
    M, N, K = 97, 131, 45
    X, W, b = rand((M, K), 18), rand((K, N), 19), wl.bias_uniform(N, 20)
    R, T = oracle.linear(np32(X), np32(W), np32(b), 1)
    assert_close(run_linear(X, W, b, 1), R, T, "linear scalar")


# ---- integer-valued inputs: bit-exact --------------------------------------

@pytest.mark.parametrize("t", T32)
def test_f32_integer_exact(t, tile):
    tile(F32, t)
    M, N, K = 333, 290, 260
    A = wl.integers((M, K), 21, -2, 2)
    B = wl.integers((K, N), 22, -2, 2)
    C = wl.integers((M, N), 23, -4, 4)
    R, _ = oracle.gemm(np32(A), np32(B), 1.5, 0.5, np32(C))
    assert_exact(run_gemm_f32(A, B, 1.5, 0.5, C), R, f"f32 int tile {t}")


@pytest.mark.parametrize("t", T16)
def test_f16_integer_exact(t, tile):
    tile(F16, t)
    M, N, K = 300, 280, 256
    A = wl.to_half(wl.integers((M, K), 24, -8, 8))
    B = wl.to_half(wl.integers((K, N), 25, -8, 8))
    R, _ = oracle.gemm(bits16(A), bits16(B))
    assert_exact(run_gemm_f16(A, B), R, f"f16 int tile {t}")


@pytest.mark.parametrize("t", T32)
def test_linear_integer_exact(t, tile):
    tile(F32, t)
    M, N, K = 300, 264, 128
    X, W, b = wl.integers((M, K), 26, -2, 2), wl.integers((K, N), 27, -2, 2), wl.integers((N,), 28, -4, 4)
    R, _ = oracle.linear(np32(X), np32(W), np32(b), 1)
    assert_exact(run_linear(X, W, b, 1), R, f"linear int tile {t}")


# ---- split-K: partial products added atomically -----------------------------

@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("S", [2, 3, 5])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (1.5, 0.5), (-0.5, 1.0)])
def test_f32_split_k(t, S, alpha, beta, tile, split):
    tile(F32, t)
    split(S)
    M, N, K = 300, 260, 1000          # ragged in every dimension, K not a multiple of the split
    A, B, C = rand((M, K), 40), rand((K, N), 41), rand((M, N), 42)
    R, T = oracle.gemm(np32(A), np32(B), alpha, beta, np32(C))
    got = run_gemm_f32(A, B, alpha, beta, C if beta != 0.0 else None)
    assert_close(got, R, T, f"f32 split {S} tile {t}")


@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("S", [2, 4])
def test_f32_split_k_scalar_path(t, S, tile, split):
    tile(F32, t)
    split(S)
    M, N, K = 97, 131, 517
    A, B = rand((M, K), 43), rand((K, N), 44)
    R, T = oracle.gemm(np32(A), np32(B))
    assert_close(run_gemm_f32(A, B), R, T, f"f32 split scalar {S} tile {t}")


@pytest.mark.parametrize("t", T16)
@pytest.mark.parametrize("S", [2, 3])
def test_f16_split_k(t, S, tile, split):
    tile(F16, t)
    split(S)
    for (M, N, K), seed in (((257, 264, 520), 45), ((130, 70, 301), 46)):
        A, B, C = wl.to_half(rand((M, K), seed)), wl.to_half(rand((K, N), seed + 1)), rand((M, N), seed + 2)
        R, T = oracle.gemm(bits16(A), bits16(B), 1.5, 0.5, np32(C))
        assert_close(run_gemm_f16(A, B, 1.5, 0.5, C), R, T, f"f16 split {S} tile {t} {M}x{N}x{K}")
        Ab, Bb = wl.to_bf16(rand((M, K), seed)), wl.to_bf16(rand((K, N), seed + 1))
        R, T = oracle.gemm(bits16(Ab), bits16(Bb), 1.5, 0.5, np32(C), bf16=True)
        assert_close(run_gemm_bf16(Ab, Bb, 1.5, 0.5, C), R, T, f"bf16 split {S} tile {t} {M}x{N}x{K}")


@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("with_bias", [True, False])
def test_linear_split_k(t, act, with_bias, tile, split):
    tile(F32, t)
    split(3)
    M, N, K = 200, 300, 700
    X, W = rand((M, K), 47, 1 / 16), rand((K, N), 48, 1 / 16)
    b = wl.bias_uniform(N, 49) if with_bias else None
    R, T = oracle.linear(np32(X), np32(W), None if b is None else np32(b), act)
    Y = run_linear(X, W, b, act)
    assert_close(Y, R, T, f"linear split tile {t} act {act} bias {with_bias}")
    if act == 1:
        assert not np.any(np.signbit(Y))


@pytest.mark.parametrize("S", [2, 7, 16])
def test_split_k_integer_exact(S, split):
    split(S)
    M, N, K = 190, 210, 1500
    A, B, C = wl.integers((M, K), 50, -2, 2), wl.integers((K, N), 51, -2, 2), wl.integers((M, N), 52, -4, 4)
    R, _ = oracle.gemm(np32(A), np32(B), 1.5, 0.5, np32(C))
    assert_exact(run_gemm_f32(A, B, 1.5, 0.5, C), R, f"f32 int split {S}")
    Ah, Bh = wl.to_half(wl.integers((M, K), 53, -8, 8)), wl.to_half(wl.integers((K, N), 54, -8, 8))
    R, _ = oracle.gemm(bits16(Ah), bits16(Bh))
    assert_exact(run_gemm_f16(Ah, Bh), R, f"f16 int split {S}")
    X, W, b = wl.integers((M, K), 55, -2, 2), wl.integers((K, N), 56, -2, 2), wl.integers((N,), 57, -4, 4)
    R, _ = oracle.linear(np32(X), np32(W), np32(b), 1)
    assert_exact(run_linear(X, W, b, 1), R, f"linear int split {S}")


@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("M,N", [(512, 512), (500, 512), (512, 516)])
@pytest.mark.parametrize("S", [1, 2])
def test_interior_and_edge_tiles_exact(t, M, N, S, tile, split):
    """512 x 512: every tile whole, so the launch takes the kernel whose copies
    need no bounds selects (also with K split in two); M = 500: only A's rows
    checked (B given K-by-N); N = 516: a ragged last tile column, every bound
    checked. Integer inputs, exact."""
    tile(F32, t)
    split(S)
    K = 512
    A, B, C = wl.integers((M, K), 170, -2, 2), wl.integers((K, N), 171, -2, 2), wl.integers((M, N), 172, -4, 4)
    R, _ = oracle.gemm(np32(A), np32(B), 1.5, 0.5, np32(C))
    assert_exact(run_gemm_f32(A, B, 1.5, 0.5, C), R, f"tile {t} {M}x{N} split {S}")
    assert_exact(run_nt(ll.gemm_f32_nt, A, B.t().contiguous(), 1.5, 0.5, C), R, f"tile {t} {M}x{N} nt")
    b = wl.integers((N,), 173, -4, 4)
    R, _ = oracle.linear(np32(A), np32(B), np32(b), 1)
    assert_exact(run_linear(A, B, b, 1), R, f"linear tile {t} {M}x{N} split {S}")


@pytest.mark.parametrize("N", [512, 520])
def test_16bit_interior_and_edge_tiles_exact(N):
    """16-bit direct kernel: whole 256x256 tiles (no bounds selects) or a ragged
    last column; both B layouts; integer inputs, exact."""
    M, K = 512, 256
    for bf in (False, True):
        dt = torch.bfloat16 if bf else torch.float16
        A8, B8 = wl.integers((M, K), 174, -8, 8), wl.integers((K, N), 175, -8, 8)
        R, _ = oracle.gemm(np32(A8), np32(B8))
        fn, fn_nt = (ll.gemm_bf16f32, ll.gemm_bf16f32_nt) if bf else (ll.gemm_f16f32, ll.gemm_f16f32_nt)
        Cd = torch.full((M, N), float("nan"), device=DEV)
        fn(A8.to(dt).to(DEV), B8.to(dt).to(DEV), Cd)
        torch.cuda.synchronize()
        assert_exact(np32(Cd), R, f"16-bit bf16={bf} N={N}")
        assert_exact(run_nt(fn_nt, A8.to(dt), B8.t().contiguous().to(dt)), R, f"16-bit nt bf16={bf} N={N}")


@pytest.mark.parametrize("M,N", [(384, 384), (385, 392), (3072, 3072)])
def test_16bit_192_tile_exact(M, N, tile):
    """The 192x192 tile: whole tiles (the interior path, no bounds selects;
    3072^2 is one tile per CU), or a ragged last row and column; both B
    layouts, fp16 and bf16; integer inputs, exact."""
    tile(F16, [ll.tile_name(F16, t) for t in T16].index("f16_192x192_direct"))
    K = 256
    A8, B8 = wl.integers((M, K), 176, -8, 8), wl.integers((K, N), 177, -8, 8)
    R, _ = oracle.gemm(np32(A8), np32(B8))
    for bf in (False, True):
        dt = torch.bfloat16 if bf else torch.float16
        fn, fn_nt = (ll.gemm_bf16f32, ll.gemm_bf16f32_nt) if bf else (ll.gemm_f16f32, ll.gemm_f16f32_nt)
        Cd = torch.full((M, N), float("nan"), device=DEV)
        fn(A8.to(dt).to(DEV), B8.to(dt).to(DEV), Cd)
        torch.cuda.synchronize()
        assert_exact(np32(Cd), R, f"192 tile bf16={bf} {M}x{N}")
        assert_exact(run_nt(fn_nt, A8.to(dt), B8.t().contiguous().to(dt)), R,
                     f"192 tile nt bf16={bf} {M}x{N}")


@pytest.mark.parametrize("t", [4, 5])
@pytest.mark.parametrize("K", [1, 40, 96, 97, 1000])
@pytest.mark.parametrize("S", [1, 3])
def test_k_slices_integer_exact(t, K, S, tile, split):
    """K-sliced tiles: slices past the end of K (K = 1, 40), ragged last stages, a
    workgroup-level K-split on top; integer inputs, so every order is exact."""
    tile(F32, t)
    split(S)
    M, N = 150, 136   # N % 4 == 0: K-by-N B takes the direct kernel when K % 4 == 0
    A, B, C = wl.integers((M, K), 160, -2, 2), wl.integers((K, N), 161, -2, 2), wl.integers((M, N), 162, -4, 4)
    R, _ = oracle.gemm(np32(A), np32(B), 1.5, 0.5, np32(C))
    assert_exact(run_gemm_f32(A, B, 1.5, 0.5, C), R, f"k-sliced tile {t} K={K} split {S}")
    got = run_nt(ll.gemm_f32_nt, A, B.t().contiguous(), 1.5, 0.5, C)
    assert_exact(got, R, f"k-sliced tile {t} K={K} split {S}, B given N-by-K")
    b = wl.integers((N,), 163, -4, 4)
    R, _ = oracle.linear(np32(A), np32(B), np32(b), 1)
    assert_exact(run_linear(A, B, b, 1), R, f"k-sliced linear tile {t} K={K} split {S}")


def test_split_k_beta_zero_ignores_nan(split):
    split(4)
    M, N, K = 100, 120, 640
    A, B = rand((M, K), 58), rand((K, N), 59)
    R, T = oracle.gemm(np32(A), np32(B), 2.0, 0.0)
    got = run_gemm_f32(A, B, 2.0, 0.0)   # C prefilled with NaN
    assert_close(got, R, T, "split NaN prefill")


# ---- degenerate cases and the write-back contract ---------------------------

def test_k_zero_and_alpha_zero():
    M, N = 70, 90
    C = rand((M, N), 30)
    A0, B0 = torch.zeros((M, 0)), torch.zeros((0, N))
    got = run_gemm_f32(A0, B0, 2.0, 0.5, C)
    assert np.array_equal(got, (np32(C) * np.float32(0.5)))
    A, B = rand((M, 8), 31), rand((8, N), 32)
    got = run_gemm_f32(A, B, 0.0, -1.0, C)
    assert np.array_equal(got, -np32(C))
    got = run_gemm_f32(A, B, 0.0, 0.0, C)
    assert np.all(got == 0)
    got = run_gemm_f16(wl.to_half(A0), wl.to_half(B0), 1.0, 0.0, C)
    assert np.all(got == 0)
    b = wl.bias_uniform(N, 33)
    Y = run_linear(torch.zeros((M, 0)), torch.zeros((0, N)), b, 1)
    assert np.array_equal(Y, np.broadcast_to(np.maximum(np32(b), 0), (M, N)))
    Y = run_linear(torch.zeros((M, 0)), torch.zeros((0, N)), None, 0)
    assert np.all(Y == 0)


def test_empty_outputs_are_no_ops():
    C = torch.zeros((0, 5), device=DEV)
    ll.gemm_f32(torch.zeros((0, 3), device=DEV), torch.zeros((3, 5), device=DEV), C)
    C = torch.zeros((4, 0), device=DEV)
    ll.gemm_f16f32(torch.zeros((4, 3), device=DEV, dtype=torch.float16),
                   torch.zeros((3, 0), device=DEV, dtype=torch.float16), C)
    torch.cuda.synchronize()


@pytest.mark.parametrize("t", T32)
def test_beta_zero_ignores_nan_and_guards_stay(t, tile):
    tile(F32, t)
    M, N, K = 131, 100, 48
    A, B = rand((M, K), 34), rand((K, N), 35)
    Cbuf = torch.full((M + 3, N + 8), float("nan"), device=DEV)
    C = Cbuf[:M, :N]
    ll.gemm_f32(A.to(DEV), B.to(DEV), C, 1.0, 0.0)
    torch.cuda.synchronize()
    R, T = oracle.gemm(np32(A), np32(B))
    assert_close(np32(C), R, T, "nan prefill")
    g = np32(Cbuf)
    assert np.all(np.isnan(g[:, N:])) and np.all(np.isnan(g[M:, :]))


def test_non_default_stream():
    M, N, K = 512, 384, 256
    A, B = rand((M, K), 36), rand((K, N), 37)
    s = torch.cuda.Stream()
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((M, N), device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ll.gemm_f32(Ad, Bd, C)
    s.synchronize()
    R, T = oracle.gemm(np32(A), np32(B))
    assert_close(np32(C), R, T, "stream")


def test_concurrent_streams_and_threads():
    """Products of every kind running at the same time on two streams, issued
    from two host threads: the library keeps no state between calls (beyond
    the device-property cache), so each result matches the oracle. The shapes
    include one row against a 4096 x 11008 B (the skinny kernels, K split
    over the CUs) and 16 rows against an 8192 x 4096 one (the 32x128 tile)."""
    import threading
    cases = []
    shapes = [(600, 520, 200), (257, 300, 1000), (1024, 768, 512), (300, 264, 72), (1, 11008, 4096),
              (16, 4096, 8192)]
    for i, (M, N, K) in enumerate(shapes):
        A, B = rand((M, K), 171 + 2 * i), rand((K, N), 172 + 2 * i)
        cases.append(("f32", A, B, oracle.gemm(np32(A), np32(B))))
        Ah, Bh = A.half(), B.half()
        cases.append(("f16", Ah, Bh, oracle.gemm(bits16(Ah), bits16(Bh))))
        Ab, Bb = A.bfloat16(), B.t().contiguous().bfloat16()
        cases.append(("bf16_nt", Ab, Bb, oracle.gemm(bits16(Ab), bits16(Bb), bf16=True, b_trans=True)))
        b = wl.bias_uniform(N, 180 + i)
        cases.append(("linear", A, (B, b), oracle.linear(np32(A), np32(B), np32(b), 1)))
    dev_in = [(kind, a.to(DEV), tuple(x.to(DEV) for x in bb) if isinstance(bb, tuple) else bb.to(DEV))
              for kind, a, bb, _ in cases]
    outs = [torch.full((a.shape[0], (bb[0] if isinstance(bb, tuple) else bb).shape[0 if kind.endswith("_nt") else 1]),
                       float("nan"), device=DEV) for kind, a, bb in dev_in]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def worker(w):
        try:
            with torch.cuda.stream(streams[w]):
                for rep in range(3):
                    for i in range(w, len(dev_in), 2):
                        kind, a, bb = dev_in[i]
                        if kind == "f32":
                            ll.gemm_f32(a, bb, outs[i])
                        elif kind == "f16":
                            ll.gemm_f16f32(a, bb, outs[i])
                        elif kind == "bf16_nt":
                            ll.gemm_bf16f32_nt(a, bb, outs[i])
                        else:
                            ll.linear_bias_act(a, bb[0], bb[1], 1, outs[i])
            streams[w].synchronize()
        except Exception as e:   # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(w,)) for w in (0, 1)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for (kind, _, _, (R, T)), out in zip(cases, outs):
        assert_close(np32(out), R, T, f"concurrent {kind} {tuple(out.shape)}")


def test_16bit_non_default_stream():
    M, N, K = 512, 384, 256
    A, B = rand((M, K), 38).half(), rand((K, N), 39).half()
    s = torch.cuda.Stream()
    C = torch.empty((M, N), device=DEV)
    Ad, Bd = A.to(DEV), B.to(DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ll.gemm_f16f32(Ad, Bd, C)
    s.synchronize()
    R, T = oracle.gemm(bits16(A), bits16(B))
    assert_close(np32(C), R, T, "16-bit stream")


def test_errors_raise():
    A = torch.zeros((4, 4), device=DEV)
    with pytest.raises(ll.LinearLayerError):
        ll.linear_bias_act(A, A, None, 7, torch.zeros((4, 4), device=DEV))
    with pytest.raises(ll.LinearLayerError):
        ll.gemm_f32(A, A, A)  # C overlaps A


# ---- transposed B (B given N-by-K): every tile, ragged tails -----------------

NT16 = {"f16": (ll.gemm_f16f32_nt, torch.float16, False),
        "bf16": (ll.gemm_bf16f32_nt, torch.bfloat16, True)}


@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("M,N,K", SMALL + [(301, 517, 203), (70, 33, 5)])
def test_f32_nt_small(t, M, N, K, tile):
    tile(F32, t)
    A, B = rand((M, K), 71), rand((N, K), 72)
    C = rand((M, N), 73)
    for alpha, beta in ((1.0, 0.0), (1.5, 0.5)):
        got = run_nt(ll.gemm_f32_nt, A, B, alpha, beta, C if beta else None)
        R, T = oracle.gemm(np32(A), np32(B), alpha, beta, np32(C), b_trans=True)
        assert_close(got, R, T, f"f32_nt tile {t} {M}x{N}x{K} a={alpha} b={beta}")


@pytest.mark.parametrize("t", T32)
def test_f32_nt_strided_b(t, tile):
    """B as a column slice of a wider matrix: ldb = K + 12 (vector path), K + 3 (scalar)."""
    tile(F32, t)
    M, N, K = 300, 270, 132
    A = rand((M, K), 74)
    for pad in (12, 3):
        Bw = rand((N, K + pad), 75)
        B = Bw[:, :K]
        Bd = Bw.to(DEV)[:, :K]
        Cd = torch.full((M, N), float("nan"), device=DEV)
        ll.gemm_f32_nt(A.to(DEV), Bd, Cd)
        torch.cuda.synchronize()
        R, T = oracle.gemm(np32(A), np32(B).copy(), b_trans=True)
        assert_close(np32(Cd), R, T, f"f32_nt tile {t} ldb={K + pad}")


@pytest.mark.parametrize("t", [t for t in T32 if not ll.tile_name(F32, t).endswith("_skinny")])
def test_f32_nt_matches_explicit_transpose(t, tile, split):
    """A*B^T through the _nt entry point equals gemm_f32 on B^T made contiguous, bit for bit:
    both feed the matrix units the same operands in the same k order. (One K-split:
    split-K adds its partial sums atomically, in no fixed order. The skinny
    kernel is left out: its two layouts add a column's k-values in different
    orders, by design, and its own tests compare each with the oracle.)"""
    tile(F32, t)
    split(1)
    M, N, K = 520, 392, 200
    A, B = rand((M, K), 76), rand((N, K), 77)
    got = run_nt(ll.gemm_f32_nt, A, B)
    ref = run_gemm_f32(A, B.t().contiguous())
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("t", T16)
@pytest.mark.parametrize("which", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(600, 520, 192), (257, 264, 64), (33, 70, 40), (301, 517, 203), (1, 8, 8)])
def test_16bit_nt_small(t, which, M, N, K, tile):
    tile(F16, t)
    fn, dt, bf = NT16[which]
    A, B = rand((M, K), 81).to(dt), rand((N, K), 82).to(dt)
    C = rand((M, N), 83)
    for alpha, beta in ((1.0, 0.0), (-0.75, 0.5)):
        got = run_nt(fn, A, B, alpha, beta, C if beta else None)
        R, T = oracle.gemm(bits16(A), bits16(B), alpha, beta, np32(C), bf16=bf, b_trans=True)
        assert_close(got, R, T, f"{which}_nt tile {t} {M}x{N}x{K} a={alpha} b={beta}")


@pytest.mark.parametrize("t", [t for t in T16 if "_skinny" not in ll.tile_name(F16, t)])
@pytest.mark.parametrize("which", ["f16", "bf16"])
def test_16bit_nt_matches_explicit_transpose(t, which, tile, split):
    """As for FP32; the skinny kernel (B given N-by-K only: forced with B given
    K-by-N, the 128x128 tile runs) has its own tests against the oracle."""
    tile(F16, t)
    split(1)
    fn, dt, _ = NT16[which]
    nn = ll.gemm_bf16f32 if which == "bf16" else ll.gemm_f16f32
    M, N, K = 520, 392, 192
    A, B = rand((M, K), 84).to(dt), rand((N, K), 85).to(dt)
    got = run_nt(fn, A, B)
    ref = run_nt(lambda a, b, c, al, be: nn(a, b.t().contiguous(), c, al, be), A, B)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("with_bias", [True, False])
def test_linear_nt_small(t, act, with_bias, tile):
    tile(F32, t)
    for M, N, K in ((300, 520, 136), (257, 70, 33)):
        X, W = rand((M, K), 91, 0.125), rand((N, K), 92, 0.125)
        b = wl.bias_uniform(N, 93) if with_bias else None
        got = run_linear_nt(X, W, b, act)
        R, T = oracle.linear(np32(X), np32(W), None if b is None else np32(b), act, w_trans=True)
        assert_close(got, R, T, f"linear_nt tile {t} {M}x{N}x{K} act={act} bias={with_bias}")


@pytest.mark.parametrize("t", T32)
def test_nt_integer_exact(t, tile):
    tile(F32, t)
    tile(F16, min(t, len(T16) - 1))
    M, N, K = 333, 301, 260
    A, B = wl.integers((M, K), 94, -2, 2), wl.integers((N, K), 95, -2, 2)
    R, _ = oracle.gemm(np32(A), np32(B), b_trans=True)
    assert_exact(run_nt(ll.gemm_f32_nt, A, B), R, f"f32_nt tile {t}")
    A8, B8 = wl.integers((M, K), 96, -8, 8), wl.integers((N, K), 97, -8, 8)
    for fn, dt, bf in NT16.values():
        R, _ = oracle.gemm(bits16(A8.to(dt)), bits16(B8.to(dt)), bf16=bf, b_trans=True)
        assert_exact(run_nt(fn, A8.to(dt), B8.to(dt)), R, f"16-bit nt bf16={bf}")
    b = wl.integers((N,), 98, -4, 4)
    R, _ = oracle.linear(np32(A), np32(B), np32(b), 1, w_trans=True)
    assert_exact(run_linear_nt(A, B, b, 1), R, f"linear_nt tile {t}")


@pytest.mark.parametrize("S", [2, 5])
def test_nt_split_k(S, split):
    split(S)
    M, N, K = 200, 264, 1000
    A, B, C = rand((M, K), 101), rand((N, K), 102), rand((M, N), 103)
    got = run_nt(ll.gemm_f32_nt, A, B, 1.5, 0.5, C)
    R, T = oracle.gemm(np32(A), np32(B), 1.5, 0.5, np32(C), b_trans=True)
    assert_close(got, R, T, f"f32_nt split {S}")
    for which, (fn, dt, bf) in NT16.items():
        A16, B16 = A.to(dt), B.to(dt)
        got = run_nt(fn, A16, B16)
        R, T = oracle.gemm(bits16(A16), bits16(B16), bf16=bf, b_trans=True)
        assert_close(got, R, T, f"{which}_nt split {S}")
    b = wl.bias_uniform(N, 104)
    got = run_linear_nt(A, B, b, 1)
    R, T = oracle.linear(np32(A), np32(B), np32(b), 1, w_trans=True)
    assert_close(got, R, T, f"linear_nt split {S}")


def test_nt_shape_errors():
    A = torch.zeros((8, 16), device=DEV)
    B = torch.zeros((12, 16), device=DEV)
    C = torch.zeros((8, 12), device=DEV)
    ll.gemm_f32_nt(A, B, C)
    with pytest.raises((ValueError, ll.LinearLayerError)):
        ll.gemm_f32_nt(A, B.t(), C)          # B given K-by-N
    with pytest.raises((ValueError, ll.LinearLayerError)):
        ll.linear_bias_act_nt(A, B, torch.zeros(16, device=DEV), 1, C)   # bias of length K



# ---- strided batches ------------------------------------------------------------

BATCHED = {"f32": (ll.gemm_f32_batched, torch.float32, False),
           "f16": (ll.gemm_f16f32_batched, torch.float16, False),
           "bf16": (ll.gemm_bf16f32_batched, torch.bfloat16, True)}


def host_bits(t, which):
    return np32(t) if which == "f32" else bits16(t)


def run_batched(fn, A, B, alpha=1.0, beta=0.0, C=None, trans_b=False, N=None):
    """Device copies of 3-D host tensors (expanded ones keep batch stride 0)."""
    def dev(t):
        if t.shape[0] > 1 and t.stride(0) == 0:
            return t[:1].to(DEV).expand(t.shape)
        return t.to(DEV)
    Ad, Bd = dev(A), dev(B)
    nb, M = A.shape[0], A.shape[1]
    N = (B.shape[1] if trans_b else B.shape[2]) if N is None else N
    Cd = (C.clone() if C is not None else torch.full((nb, M, N), float("nan"))).to(DEV)
    fn(Ad, Bd, Cd, alpha, beta, trans_b=trans_b)
    torch.cuda.synchronize()
    return np32(Cd)


def oracle_batched(A, B, which, alpha=1.0, beta=0.0, C=None, trans_b=False):
    Ah = host_bits(A.contiguous(), which)
    Bh = host_bits(B.contiguous(), which)
    return oracle.gemm_batched(Ah, Bh, alpha, beta, None if C is None else np32(C),
                               bf16=which == "bf16", b_trans=trans_b)


@pytest.mark.parametrize("which", list(BATCHED))
@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("nb,M,N,K", [(7, 130, 70, 72), (3, 257, 300, 64), (16, 33, 40, 24)])
def test_batched_small(which, trans_b, nb, M, N, K):
    fn, dt, _ = BATCHED[which]
    A = rand((nb, M, K), 111).to(dt)
    B = rand((nb, N, K) if trans_b else (nb, K, N), 112).to(dt)
    C = rand((nb, M, N), 113)
    for alpha, beta in ((1.0, 0.0), (1.5, -0.5)):
        got = run_batched(fn, A, B, alpha, beta, C if beta else None, trans_b)
        R, T = oracle_batched(A, B, which, alpha, beta, C if beta else None, trans_b)
        assert_close(got, R, T, f"{which} batched tb={trans_b} {nb}x{M}x{N}x{K} a={alpha} b={beta}")


@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("M,N,K", [(300, 264, 136), (256, 256, 256)])
def test_batched_f32_every_tile(t, M, N, K, tile):
    """(256, 256, 256): whole tiles, the kernels without bounds selects, on
    every item of the batch (integer inputs, exact)."""
    tile(F32, t)
    nb = 5
    if M % 256 == 0:
        A, B = wl.integers((nb, M, K), 116, -2, 2), wl.integers((nb, K, N), 117, -2, 2)
        R, _ = oracle_batched(A, B, "f32")
        assert_exact(run_batched(ll.gemm_f32_batched, A, B), R, f"f32 batched tile {t} whole tiles")
        return
    A, B = rand((nb, M, K), 114), rand((nb, K, N), 115)
    got = run_batched(ll.gemm_f32_batched, A, B)
    R, T = oracle_batched(A, B, "f32")
    assert_close(got, R, T, f"f32 batched tile {t}")


@pytest.mark.parametrize("t", T16)
def test_batched_16bit_every_tile(t, tile):
    tile(F16, t)
    nb, M, N, K = 5, 300, 264, 136
    for which in ("f16", "bf16"):
        fn, dt, _ = BATCHED[which]
        A, B = rand((nb, M, K), 116).to(dt), rand((nb, N, K), 117).to(dt)
        got = run_batched(fn, A, B, trans_b=True)
        R, T = oracle_batched(A, B, which, trans_b=True)
        assert_close(got, R, T, f"{which} batched tile {t}")


@pytest.mark.parametrize("which", ["f32", "f16"])
def test_batched_shared_operands(which):
    """Batch stride 0: one A (or B) for every item."""
    fn, dt, _ = BATCHED[which]
    nb, M, N, K = 6, 140, 96, 80
    A1, B = rand((1, M, K), 118).to(dt), rand((nb, K, N), 119).to(dt)
    A = A1.expand(nb, M, K)
    got = run_batched(fn, A, B)
    R, T = oracle_batched(A, B, which)
    assert_close(got, R, T, f"{which} shared A")
    B1 = rand((1, K, N), 120).to(dt)
    got = run_batched(fn, rand((nb, M, K), 121).to(dt), B1.expand(nb, K, N))
    R, T = oracle_batched(rand((nb, M, K), 121).to(dt), B1.expand(nb, K, N), which)
    assert_close(got, R, T, f"{which} shared B")


def test_batched_padded_strides_and_guards():
    """Items further apart than one matrix (stride > span) and C row padding:
    the gaps between items and the padding columns keep their contents."""
    nb, M, N, K = 4, 70, 50, 44
    Aw, Bw = rand((nb, M + 3, K + 4), 122), rand((nb, K + 2, N + 8), 123)
    A, B = Aw[:, :M, :K], Bw[:, :K, :N]
    Cw = torch.full((nb, M + 2, N + 4), 7.0, device=DEV)
    Cd = Cw[:, :M, :N]
    ll.gemm_f32_batched(Aw.to(DEV)[:, :M, :K], Bw.to(DEV)[:, :K, :N], Cd)
    torch.cuda.synchronize()
    R, T = oracle_batched(A, B, "f32")
    assert_close(np32(Cd), R, T, "padded strides")
    guard = np32(Cw).copy()
    guard[:, :M, :N] = 7.0
    assert np.all(guard == 7.0)


@pytest.mark.parametrize("S", [2, 3])
@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
def test_batched_split_k(S, beta, split):
    """Split-K on a batch: C_i = beta*C_i for every item first, then atomics."""
    split(S)
    nb, M, N, K = 3, 100, 72, 400
    A, B, C = rand((nb, M, K), 124), rand((nb, K, N), 125), rand((nb, M, N), 126)
    got = run_batched(ll.gemm_f32_batched, A, B, 1.25, beta, C if beta else None)
    R, T = oracle_batched(A, B, "f32", 1.25, beta, C if beta else None)
    assert_close(got, R, T, f"batched split {S} beta {beta}")
    for which in ("f16", "bf16"):
        fn, dt, _ = BATCHED[which]
        A16, B16 = A.to(dt), B.to(dt)
        got = run_batched(fn, A16, B16, 1.0, beta, C if beta else None)
        R, T = oracle_batched(A16, B16, which, 1.0, beta, C if beta else None)
        assert_close(got, R, T, f"{which} batched split {S} beta {beta}")


def test_batched_degenerate():
    nb, M, N = 5, 20, 12
    C = rand((nb, M, N), 127)
    # K == 0 and alpha == 0: C_i = beta*C_i for every item
    for K, alpha in ((0, 1.0), (8, 0.0)):
        A, B = rand((nb, M, K), 128), rand((nb, K, N), 129)
        got = run_batched(ll.gemm_f32_batched, A, B, alpha, 0.5, C)
        R, T = oracle_batched(A, B, "f32", alpha, 0.5, C)
        assert_close(got, R, T, f"K={K} alpha={alpha}")
    # an empty batch is a no-op
    Ce = torch.zeros((0, M, N), device=DEV)
    ll.gemm_f32_batched(torch.zeros((0, M, 8), device=DEV), torch.zeros((0, 8, N), device=DEV), Ce)
    # one item equals the single-product entry point bit for bit
    A, B = rand((1, M, 8), 130), rand((1, 8, N), 131)
    assert np.array_equal(run_batched(ll.gemm_f32_batched, A, B), run_gemm_f32(A[0], B[0])[None])


def test_batched_more_items_than_one_launch():
    """70000 items exceed the 65535 items of one launch's grid z."""
    nb, M, N, K = 70000, 8, 8, 8
    A, B = wl.integers((nb, M, K), 132, -2, 2), wl.integers((nb, K, N), 133, -2, 2)
    got = run_batched(ll.gemm_f32_batched, A, B)
    R, _ = oracle_batched(A, B, "f32")
    assert_exact(got, R, "70000 items")


def test_batched_integer_exact():
    nb, M, N, K = 9, 150, 130, 260
    A, B = wl.integers((nb, M, K), 134, -2, 2), wl.integers((nb, N, K), 135, -2, 2)
    for trans_b in (False, True):
        Bx = B if trans_b else B.transpose(1, 2).contiguous()
        R, _ = oracle_batched(A, Bx, "f32", trans_b=trans_b)
        assert_exact(run_batched(ll.gemm_f32_batched, A, Bx, trans_b=trans_b), R, f"f32 tb={trans_b}")
    A8, B8 = wl.integers((nb, M, K), 136, -8, 8), wl.integers((nb, N, K), 137, -8, 8)
    for which in ("f16", "bf16"):
        fn, dt, _ = BATCHED[which]
        R, _ = oracle_batched(A8.to(dt), B8.to(dt), which, trans_b=True)
        assert_exact(run_batched(fn, A8.to(dt), B8.to(dt), trans_b=True), R, which)


# ---- stream-K: leftover tiles shared out over one round of workgroups -------

@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("M,N,K", [(300, 264, 200), (257, 70, 1000), (600, 520, 72)])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (1.5, 0.5), (-0.5, 1.0)])
def test_f32_stream_k(t, M, N, K, alpha, beta, tile, stream_k):
    """Every tile shared out (fewer tiles than CUs): several atomic segments per tile."""
    tile(F32, t)
    stream_k(1)
    A, B, C = rand((M, K), 141), rand((K, N), 142), rand((M, N), 143)
    got = run_gemm_f32(A, B, alpha, beta, C if beta else None)
    R, T = oracle.gemm(np32(A), np32(B), alpha, beta, np32(C))
    assert_close(got, R, T, f"stream-K tile {t} {M}x{N}x{K} a={alpha} b={beta}")
    got = run_nt(ll.gemm_f32_nt, A, B.t().contiguous(), alpha, beta, C if beta else None)
    assert_close(got, R, T, f"stream-K A*B^T tile {t} {M}x{N}x{K}")


@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("with_bias", [True, False])
def test_linear_stream_k(t, act, with_bias, tile, stream_k):
    tile(F32, t)
    stream_k(1)
    M, N, K = 330, 270, 520
    X, W = rand((M, K), 144, 0.125), rand((K, N), 145, 0.125)
    b = wl.bias_uniform(N, 146) if with_bias else None
    got = run_linear(X, W, b, act)
    R, T = oracle.linear(np32(X), np32(W), None if b is None else np32(b), act)
    assert_close(got, R, T, f"stream-K linear tile {t} act={act} bias={with_bias}")
    got = run_linear_nt(X, W.t().contiguous(), b, act)
    assert_close(got, R, T, f"stream-K linear_nt tile {t}")


def test_stream_k_hybrid_rounds(tile, stream_k):
    """576 tiles of 64x64 on 512 slots: one data-parallel round, 64 tiles shared out."""
    tile(F32, 3)
    stream_k(1)
    M = N = 1536
    K = 256
    props = torch.cuda.get_device_properties(0)
    assert ll.chosen_stream_k(F32, M, N, K, props.multi_processor_count) > 0
    A, B, C = wl.integers((M, K), 147, -2, 2), wl.integers((K, N), 148, -2, 2), wl.integers((M, N), 149, -4, 4)
    R, _ = oracle.gemm(np32(A), np32(B), 1.5, 0.5, np32(C))
    assert_exact(run_gemm_f32(A, B, 1.5, 0.5, C), R, "hybrid integer")
    Af, Bf = rand((M, K), 150), rand((K, N), 151)
    R, T = oracle.gemm(np32(Af), np32(Bf))
    assert_close(run_gemm_f32(Af, Bf), R, T, "hybrid")
    b = wl.integers((N,), 152, -4, 4)
    R, _ = oracle.linear(np32(A), np32(B), np32(b), 1)
    assert_exact(run_linear(A, B, b, 1), R, "hybrid linear integer")


def test_stream_k_guards_untouched(tile, stream_k):
    """Shared-out tiles' passes stay inside the output: the padding columns of C keep their values."""
    tile(F32, 1)
    stream_k(1)
    M, N, K = 300, 264, 192
    A, B = rand((M, K), 153), rand((K, N), 154)
    Cw = torch.full((M, N + 8), 7.0, device=DEV)
    Cd = Cw[:, :N]
    ll.gemm_f32(A.to(DEV), B.to(DEV), Cd, 1.0, 0.0)
    b = wl.bias_uniform(N, 155).to(DEV)
    Yw = torch.full((M, N + 8), 7.0, device=DEV)
    ll.linear_bias_act(A.to(DEV), B.to(DEV), b, 1, Yw[:, :N])
    torch.cuda.synchronize()
    assert torch.all(Cw[:, N:] == 7.0) and torch.all(Yw[:, N:] == 7.0)
    R, T = oracle.gemm(np32(A), np32(B))
    assert_close(np32(Cd), R, T, "stream-K strided C")


SK16 = {("f16", False): ll.gemm_f16f32, ("f16", True): ll.gemm_f16f32_nt,
        ("bf16", False): ll.gemm_bf16f32, ("bf16", True): ll.gemm_bf16f32_nt}


def run_16(which, trans_b, A, B, alpha=1.0, beta=0.0, C=None):
    """One of the 16-bit products on device copies; B is N-by-K when trans_b."""
    Ad, Bd = A.to(DEV), B.to(DEV)
    N = B.shape[0] if trans_b else B.shape[1]
    Cd = (C.clone() if C is not None else torch.full((A.shape[0], N), float("nan"))).to(DEV)
    SK16[(which, trans_b)](Ad, Bd, Cd, alpha, beta)
    torch.cuda.synchronize()
    return np32(Cd)


@pytest.mark.parametrize("which,trans_b", list(SK16))
@pytest.mark.parametrize("M,N,K", [(300, 264, 200), (257, 70, 1000), (600, 520, 72), (512, 512, 256)])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (1.5, 0.5), (-0.5, 1.0)])
def test_16bit_stream_k(which, trans_b, M, N, K, alpha, beta, tile, stream_k):
    """The 256x256 16-bit direct kernel with every tile shared out (fewer tiles
    than CUs): several atomic segments per tile, ragged and whole (512^3-like)
    shapes."""
    t = 0
    tile(F16, t)
    stream_k(1)
    dt = torch.float16 if which == "f16" else torch.bfloat16
    A = rand((M, K), 161).to(dt)
    B = rand((N, K) if trans_b else (K, N), 162).to(dt)
    C = rand((M, N), 163)
    got = run_16(which, trans_b, A, B, alpha, beta, C if beta else None)
    R, T = oracle.gemm(bits16(A), bits16(B), alpha, beta, np32(C), bf16=which == "bf16",
                       b_trans=trans_b)
    assert_close(got, R, T, f"{which} tb={trans_b} tile {t} stream-K {M}x{N}x{K} a={alpha} b={beta}")


@pytest.mark.parametrize("which,trans_b", [("f16", False), ("bf16", True)])
def test_16bit_stream_k_hybrid_rounds(which, trans_b, tile, stream_k):
    """289 tiles of 256x256 on 256 CUs: one data-parallel round, 33 tiles shared
    out; integer inputs, so every order of the atomic additions gives the
    oracle's result exactly."""
    tile(F16, 0)
    stream_k(1)
    M = N = 17 * 256
    K = 192
    props = torch.cuda.get_device_properties(0)
    assert ll.chosen_stream_k(F16, M, N, K, props.multi_processor_count) > 0
    dt = torch.float16 if which == "f16" else torch.bfloat16
    A = wl.integers((M, K), 164, -2, 2).to(dt)
    B = wl.integers((N, K) if trans_b else (K, N), 165, -2, 2).to(dt)
    C = wl.integers((M, N), 166, -4, 4)
    R, _ = oracle.gemm(bits16(A), bits16(B), 1.5, 0.5, np32(C), bf16=which == "bf16", b_trans=trans_b)
    assert_exact(run_16(which, trans_b, A, B, 1.5, 0.5, C), R, f"{which} hybrid integer")
    Af, Bf = rand((M, K), 167).to(dt), rand(tuple(B.shape), 168).to(dt)
    R, T = oracle.gemm(bits16(Af), bits16(Bf), bf16=which == "bf16", b_trans=trans_b)
    assert_close(run_16(which, trans_b, Af, Bf), R, T, f"{which} hybrid")


def test_16bit_stream_k_guards_untouched(tile, stream_k):
    """The shared-out tiles' passes and atomics stay inside C."""
    tile(F16, 0)
    stream_k(1)
    M, N, K = 300, 264, 192
    A, B = rand((M, K), 169).half(), rand((K, N), 170).half()
    Cw = torch.full((M, N + 8), 7.0, device=DEV)
    Cd = Cw[:, :N]
    Cd.copy_(torch.ones((M, N)))
    ll.gemm_f16f32(A.to(DEV), B.to(DEV), Cd, 1.0, 0.5)
    torch.cuda.synchronize()
    assert torch.all(Cw[:, N:] == 7.0)
    R, T = oracle.gemm(bits16(A), bits16(B), 1.0, 0.5, np.ones((M, N), np.float32))
    assert_close(np32(Cd), R, T, "16-bit stream-K strided C")


# ---- full-size workloads, as the bench launches them ------------------------
#
# Every output element of every full-size workload is compared with the full
# float64 oracle (the bench's workloads, in its launch configuration: the
# automatic plan). Integer-valued variants must match it bit for bit on every
# element.

def full_inputs(w, integer=False):
    """Host inputs of workload w and the oracle's operands for them."""
    x = wl.make_inputs(w, integer=integer)
    half = w.kind in wl.HALF_KINDS
    ops = {
        "A": bits16(x["A"]) if half else np32(x["A"]),
        "B": bits16(x["B"]) if half else np32(x["B"]),
        "C": np32(x["C"]) if "C" in x else None,
        "bias": np32(x["bias"]) if "bias" in x else None,
    }
    return x, ops


def full_run(w, x):
    """The GPU result of workload w on inputs x, through the C ABI."""
    A, B = x["A"], x["B"]
    if w.kind == "gemm_f32":
        return run_gemm_f32(A, B, w.alpha, w.beta, x.get("C"))
    if w.kind == "gemm_f16f32":
        return run_gemm_f16(A, B, w.alpha, w.beta, x.get("C"))
    if w.kind == "gemm_bf16f32":
        return run_gemm_bf16(A, B, w.alpha, w.beta, x.get("C"))
    if w.kind == "gemm_f16f32_nt":
        return run_nt(ll.gemm_f16f32_nt, A, B, w.alpha, w.beta, x.get("C"))
    if w.kind == "linear":
        return run_linear(A, B, x["bias"], w.act)
    if w.kind == "linear_nt":
        return run_linear_nt(A, B, x["bias"], w.act)
    if w.kind == "gemm_f32_batched":
        return run_batched(ll.gemm_f32_batched, A, B, w.alpha, w.beta)
    raise ValueError(w.kind)


def full_oracle(w, ops):
    """The oracle's (R, T) for the whole output of workload w."""
    A, B, C = ops["A"], ops["B"], ops["C"]
    bt = w.kind in wl.B_TRANSPOSED_KINDS
    if w.kind in ("linear", "linear_nt"):
        return oracle.linear(A, B, ops["bias"], w.act, w_trans=bt)
    if w.kind in wl.BATCHED_KINDS:
        return oracle.gemm_batched(A, B, w.alpha, w.beta, C)
    return oracle.gemm(A, B, w.alpha, w.beta, C, bf16=w.kind == "gemm_bf16f32", b_trans=bt)


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_full_workload(name):
    """Every element of the full-size workload within 1e-4*t (+ half an ulp) of
    the float64 oracle."""
    import time
    w = wl.WORKLOADS[name]
    x, ops = full_inputs(w)
    t0 = time.perf_counter()
    got = full_run(w, x)
    t1 = time.perf_counter()
    R, T = full_oracle(w, ops)
    t2 = time.perf_counter()
    ratio = assert_close(got, R, T, name)
    if w.kind in ("linear", "linear_nt") and w.act == 1:
        assert not np.any(np.signbit(got)), f"{name}: ReLU output holds -0 or a negative value"
    print(f"{name}: all {got.size} elements within bound, max err/t = {ratio:.3g} "
          f"(GPU {t1 - t0:.1f} s, oracle {t2 - t1:.1f} s on {oracle.max_threads()} threads)")


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_full_integer_exact(name):
    """Integer-valued inputs of the full-size shape: every element equals the
    oracle's bit for bit (every partial sum is an exact fp32 integer, so every
    summation order, split or atomic, reaches it)."""
    w = wl.WORKLOADS[name]
    x, ops = full_inputs(w, integer=True)
    got = full_run(w, x)
    R, _ = full_oracle(w, ops)
    assert_exact(got, R, name)
