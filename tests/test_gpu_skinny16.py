"""GPU parity of the skinny 16-bit kernel (dot2 instructions for a few rows of
A with B given N-by-K, memory-bound; chosen by itself for one row of A with a
large B, and forced here for the rest): binary16 and bfloat16, every row
count from 1 to 16 and a few past it, all five row-pass widths (1, 2, 4, 8, 16),
both epilogues and the K-split atomics, K ranges longer than the staged A
block, ragged and unaligned N and K, a strided batch, the forced tile with B
given K-by-N (the 128x128 tile runs in its place), and the decode-sized
products at full size; against the float64 oracle element by element, and
bit-exact on integer inputs."""
import numpy as np
import pytest

import linear_layer_amd as ll
import oracle
from linear_layer_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F16 = ll.DTYPE_F16
SKINNY = "f16_16x256_skinny_nt"
TYPES = {"f16": (torch.float16, False, ll.gemm_f16f32_nt, ll.gemm_f16f32),
         "bf16": (torch.bfloat16, True, ll.gemm_bf16f32_nt, ll.gemm_bf16f32)}


@pytest.fixture(autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    ll.set_tile(F16, -1)
    ll.set_split_k(-1)
    ll.set_stream_k(-1)
    yield
    ll.set_tile(F16, -1)
    ll.set_split_k(-1)


def np32(t):
    return t.detach().cpu().numpy()


def bits(t):
    return wl.half_bits(t.cpu())


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def assert_close(got, R, T, what):
    bound = 1e-4 * T + np.spacing(np.abs(R).astype(np.float32)).astype(np.float64) / 2
    bad = ~(np.abs(np.asarray(got, np.float64) - R) <= bound)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside the bound"


def skinny_index():
    return [ll.tile_name(F16, t) for t in range(ll.num_tiles(F16))].index(SKINNY)


def plan(flags, M, N, K):
    return (ll.tile_name(F16, ll.chosen_tile(flags, M, N, K, cus())),
            ll.chosen_split_k(flags, M, N, K, cus()))


def force_skinny():
    ll.set_tile(F16, skinny_index())


def run_nt(fn, A, Bnk, alpha, beta, C0):
    Cd = C0.to(DEV) if C0 is not None else torch.full((A.shape[0], Bnk.shape[0]), float("nan"), device=DEV)
    fn(A.to(DEV), Bnk.to(DEV), Cd, alpha, beta)
    torch.cuda.synchronize()
    return np32(Cd)


@pytest.mark.parametrize("M", list(range(1, 17)))
@pytest.mark.parametrize("which", ["f16", "bf16"])
def test_every_row_count(M, which):
    """Forced (this B is too small for the automatic choice); N and K ragged."""
    dt, bf, fn, _ = TYPES[which]
    N, K = 1000, 777
    assert plan(F16 | ll.PLAN_B_NK, M, N, K)[0] != SKINNY
    force_skinny()
    assert plan(F16 | ll.PLAN_B_NK, M, N, K)[0] == SKINNY
    A, B, C0 = wl.uniform((M, K), 800 + M).to(dt), wl.uniform((N, K), 801).to(dt), wl.uniform((M, N), 802)
    got = run_nt(fn, A, B, 1.5, 0.5, C0)
    R, T = oracle.gemm(bits(A), bits(B), 1.5, 0.5, np32(C0), bf16=bf, b_trans=True)
    assert_close(got, R, T, f"{which} M={M}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (16, 256, 256), (5, 257, 255),
                                   (16, 4099, 1030), (7, 300, 4), (2, 64, 40000)])
@pytest.mark.parametrize("splits", [1, 2, 5, 16])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (1.5, 0.5), (-0.5, 1.0)])
@pytest.mark.parametrize("which", ["f16", "bf16"])
def test_forced_splits_integer_exact(M, N, K, splits, alpha, beta, which):
    """Integer inputs: every order of additions, atomics included, gives the
    oracle's result exactly; beta = 0 ignores NaN in C. (2 x 64 x 40000 walks
    a K range longer than the staged A block when unsplit.)"""
    dt, bf, fn, _ = TYPES[which]
    force_skinny()
    ll.set_split_k(splits)
    assert plan(F16 | ll.PLAN_B_NK, M, N, K)[0] == SKINNY
    A, B = wl.integers((M, K), 810, -2, 2).to(dt), wl.integers((N, K), 811, -2, 2).to(dt)
    C0 = wl.integers((M, N), 812, -4, 4) if beta else None
    got = run_nt(fn, A, B, alpha, beta, C0)
    R, _ = oracle.gemm(bits(A), bits(B), alpha, beta, np32(C0) if beta else None, bf16=bf, b_trans=True)
    bad = got != R.astype(np.float32)
    assert not bad.any(), f"{which} {M}x{N}x{K} splits {splits} a={alpha} b={beta}: {bad.sum()} differ"


@pytest.mark.parametrize("pad,shift", [(1, 0), (3, 1), (2, 3), (5, 7)])
@pytest.mark.parametrize("which", ["f16", "bf16"])
def test_unaligned(pad, shift, which):
    """Leading dimensions and base pointers off 16 bytes (2-byte steps): chunk
    loads at any alignment; guard columns of C untouched."""
    dt, bf, fn, _ = TYPES[which]
    force_skinny()
    M, N, K = 9, 1031, 517
    A, B, C0 = wl.uniform((M, K), 820).to(dt), wl.uniform((N, K), 821).to(dt), wl.uniform((M, N), 822)
    abuf = torch.zeros((M, K + pad + shift), dtype=dt, device=DEV)
    Ad = abuf[:, shift:shift + K]; Ad.copy_(A.to(DEV))
    bbuf = torch.zeros((N, K + pad + shift), dtype=dt, device=DEV)
    Bd = bbuf[:, shift:shift + K]; Bd.copy_(B.to(DEV))
    cbuf = torch.full((M, N + pad + shift), 7.0, device=DEV)
    Cd = cbuf[:, shift:shift + N]; Cd.copy_(C0.to(DEV))
    fn(Ad, Bd, Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    R, T = oracle.gemm(bits(A), bits(B), 1.5, 0.5, np32(C0), bf16=bf, b_trans=True)
    assert_close(np32(Cd), R, T, f"{which} unaligned pad {pad} shift {shift}")
    assert bool(torch.all(cbuf[:, :shift] == 7.0)) and bool(torch.all(cbuf[:, shift + N:] == 7.0))


@pytest.mark.parametrize("M", [17, 40])
@pytest.mark.parametrize("which", ["f16", "bf16"])
def test_forced_past_sixteen_rows(M, which):
    """Forced on more than 16 rows, the kernel walks the rows 16 at a time."""
    dt, bf, fn, _ = TYPES[which]
    force_skinny()
    N, K = 700, 900
    A, B, C0 = wl.uniform((M, K), 830).to(dt), wl.uniform((N, K), 831).to(dt), wl.uniform((M, N), 832)
    got = run_nt(fn, A, B, -0.5, 1.0, C0)
    R, T = oracle.gemm(bits(A), bits(B), -0.5, 1.0, np32(C0), bf16=bf, b_trans=True)
    assert_close(got, R, T, f"{which} forced M={M}")


@pytest.mark.parametrize("which", ["f16", "bf16"])
def test_forced_with_b_given_k_by_n(which):
    """Forced with B given K-by-N, the 128x128 tile runs in its place."""
    dt, bf, _, fn = TYPES[which]
    force_skinny()
    M, N, K = 6, 300, 260
    A, B, C0 = wl.uniform((M, K), 840).to(dt), wl.uniform((K, N), 841).to(dt), wl.uniform((M, N), 842)
    Cd = C0.to(DEV)
    fn(A.to(DEV), B.to(DEV), Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    R, T = oracle.gemm(bits(A), bits(B), 1.5, 0.5, np32(C0), bf16=bf)
    assert_close(np32(Cd), R, T, f"{which} K-by-N forced")


@pytest.mark.parametrize("which", ["f16", "bf16"])
def test_batched_forced(which):
    """A strided batch runs the skinny kernel only when forced; each item's
    rows and columns stay its own."""
    dt, bf, _, _ = TYPES[which]
    force_skinny()
    nb, M, N, K = 6, 5, 300, 260
    A, B, C0 = wl.uniform((nb, M, K), 850).to(dt), wl.uniform((nb, N, K), 851).to(dt), wl.uniform((nb, M, N), 852)
    Cd = C0.to(DEV)
    (ll.gemm_bf16f32_batched if bf else ll.gemm_f16f32_batched)(A.to(DEV), B.to(DEV), Cd, 1.5, 0.5, trans_b=True)
    torch.cuda.synchronize()
    R, T = oracle.gemm_batched(bits(A), bits(B), 1.5, 0.5, np32(C0), bf16=bf, b_trans=True)
    assert_close(np32(Cd), R, T, f"{which} batched")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("which", ["f16", "bf16"])
def test_decode_sized_full_size(M, which):
    """A 11008 x 4096 weight given [out][in] with a handful of rows: the
    automatic plan for one row (skinny, K split over the CUs), forced for more;
    checked on every element against the oracle."""
    dt, bf, fn, _ = TYPES[which]
    N, K = 11008, 4096
    if M > 1:
        assert plan(F16 | ll.PLAN_B_NK, M, N, K)[0] != SKINNY
        force_skinny()
    name, s = plan(F16 | ll.PLAN_B_NK, M, N, K)
    assert name == SKINNY and s > 1
    A, B = wl.uniform((M, K), 860).to(dt), wl.uniform((N, K), 861).to(dt)
    got = run_nt(fn, A, B, 1.0, 0.0, None)
    R, T = oracle.gemm(bits(A), bits(B), bf16=bf, b_trans=True)
    assert_close(got, R, T, f"{which} decode M={M}")
