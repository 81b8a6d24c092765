"""GPU parity of the skinny FP32 kernel (vector FMAs for a few rows of A,
memory-bound; chosen by itself for up to 4 rows, or 8 with a large B, and
forced here for more): every row count from 1 to 16 and a few past it, all
five row-pass widths (1, 2, 4, 8, 16), both B layouts, every epilogue (beta = 0,
general beta, K-split atomics, the fused layer with and without bias and
ReLU), K ranges longer than the staged A block, ragged and unaligned N and
K, and the layer's decode-sized shapes at full size; against the float64
oracle element by element, and bit-exact on integer inputs."""
import numpy as np
import pytest

import linear_layer_amd as ll
import oracle
from linear_layer_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32 = ll.DTYPE_F32
SKINNY = "f32_16x256_skinny"


@pytest.fixture(autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    ll.set_tile(F32, -1)
    ll.set_split_k(-1)
    ll.set_stream_k(-1)
    yield
    ll.set_tile(F32, -1)
    ll.set_split_k(-1)


def np32(t):
    return t.detach().cpu().numpy()


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def assert_close(got, R, T, what):
    bound = 1e-4 * T + np.spacing(np.abs(R).astype(np.float32)).astype(np.float64) / 2
    bad = ~(np.abs(np.asarray(got, np.float64) - R) <= bound)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside the bound"


def skinny_index():
    names = [ll.tile_name(F32, t) for t in range(ll.num_tiles(F32))]
    return names.index(SKINNY)


def plan(flags, M, N, K):
    return (ll.tile_name(F32, ll.chosen_tile(flags, M, N, K, cus())),
            ll.chosen_split_k(flags, M, N, K, cus()))


def padded(host, pad, shift=0, fill=0.0):
    rows, cols = host.shape
    buf = torch.full((rows, cols + pad + shift), fill, dtype=host.dtype, device=DEV)
    v = buf[:, shift:shift + cols]
    v.copy_(host.to(DEV))
    return buf, v


def force_skinny():
    ll.set_tile(F32, skinny_index())


@pytest.mark.parametrize("M", list(range(1, 17)))
@pytest.mark.parametrize("nt", [False, True])
def test_every_row_count(M, nt):
    """M = 1 .. 4 take the skinny kernel by themselves here (5 .. 8 do only
    with a larger B), 5 .. 16 when forced; N and K ragged."""
    N, K = 1000, 777
    flags = F32 | (ll.PLAN_B_NK if nt else 0)
    if M <= 4:
        assert plan(flags, M, N, K)[0] == SKINNY
    else:
        assert plan(flags, M, N, K)[0] != SKINNY
        force_skinny()
        assert plan(flags, M, N, K)[0] == SKINNY
    A, Bkn, C0 = wl.uniform((M, K), 600 + M), wl.uniform((K, N), 601), wl.uniform((M, N), 602)
    Bd = (Bkn.t().contiguous() if nt else Bkn).to(DEV)
    Cd = C0.to(DEV)
    (ll.gemm_f32_nt if nt else ll.gemm_f32)(A.to(DEV), Bd, Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    R, T = oracle.gemm(np32(A), np32(Bkn), 1.5, 0.5, np32(C0))
    assert_close(np32(Cd), R, T, f"M={M} nt={nt}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (16, 256, 256), (5, 257, 255),
                                   (16, 4099, 1030), (7, 300, 4), (2, 64, 20000)])
@pytest.mark.parametrize("splits", [1, 2, 5, 16])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (1.5, 0.5), (-0.5, 1.0)])
@pytest.mark.parametrize("nt", [False, True])
def test_forced_splits_integer_exact(M, N, K, splits, alpha, beta, nt):
    """Integer inputs: every order of additions, atomics included, gives the
    oracle's result exactly; beta = 0 ignores NaN in C."""
    force_skinny()
    ll.set_split_k(splits)
    assert plan(F32 | (ll.PLAN_B_NK if nt else 0), M, N, K)[0] == SKINNY
    A, Bkn = wl.integers((M, K), 610, -2, 2), wl.integers((K, N), 611, -2, 2)
    C0 = wl.integers((M, N), 612, -4, 4) if beta else torch.full((M, N), float("nan"))
    Bd = (Bkn.t().contiguous() if nt else Bkn).to(DEV)
    Cd = C0.to(DEV)
    (ll.gemm_f32_nt if nt else ll.gemm_f32)(A.to(DEV), Bd, Cd, alpha, beta)
    torch.cuda.synchronize()
    R, _ = oracle.gemm(np32(A), np32(Bkn), alpha, beta, None if not beta else np32(C0))
    got = np32(Cd)
    bad = got != R.astype(np.float32)
    assert not bad.any(), f"{M}x{N}x{K} splits {splits} a={alpha} b={beta} nt={nt}: {bad.sum()} differ"


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("with_bias", [True, False])
@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("splits", [-1, 1, 3])
def test_linear(M, act, with_bias, nt, splits):
    """The fused layer: bias and ReLU in the kernel's own store (one split) or
    in the bias fill and ReLU passes around the K-split atomics."""
    force_skinny()
    ll.set_split_k(splits)
    N, K = 1100, 1300
    X, Wkn = wl.uniform((M, K), 620, 0.125), wl.uniform((K, N), 621, 0.125)
    b = wl.bias_uniform(N, 622) if with_bias else None
    Wd = (Wkn.t().contiguous() if nt else Wkn).to(DEV)
    Yd = torch.full((M, N), float("nan"), device=DEV)
    (ll.linear_bias_act_nt if nt else ll.linear_bias_act)(X.to(DEV), Wd, None if b is None else b.to(DEV),
                                                          act, Yd)
    torch.cuda.synchronize()
    R, T = oracle.linear(np32(X), np32(Wkn), None if b is None else np32(b), act)
    got = np32(Yd)
    assert_close(got, R, T, f"linear M={M} act={act} bias={with_bias} nt={nt} splits={splits}")
    if act:
        assert not np.any(np.signbit(got))


@pytest.mark.parametrize("pad,shift", [(1, 0), (3, 1), (2, 3)])
@pytest.mark.parametrize("nt", [False, True])
def test_unaligned(pad, shift, nt):
    """Leading dimensions and base pointers off 16 bytes: chunk loads at 4-byte
    alignment; guard columns of C untouched."""
    force_skinny()
    M, N, K = 9, 1031, 517
    A, Bkn, C0 = wl.uniform((M, K), 630), wl.uniform((K, N), 631), wl.uniform((M, N), 632)
    _, Ad = padded(A, pad, shift)
    _, Bd = padded(Bkn.t().contiguous() if nt else Bkn, pad, shift)
    cbuf, Cd = padded(C0, pad, shift, fill=7.0)
    (ll.gemm_f32_nt if nt else ll.gemm_f32)(Ad, Bd, Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    R, T = oracle.gemm(np32(A), np32(Bkn), 1.5, 0.5, np32(C0))
    assert_close(np32(Cd), R, T, f"unaligned pad {pad} shift {shift} nt {nt}")
    assert bool(torch.all(cbuf[:, :shift] == 7.0)) and bool(torch.all(cbuf[:, shift + N:] == 7.0))


@pytest.mark.parametrize("M", [17, 40])
def test_forced_past_sixteen_rows(M):
    """Forced on more than 16 rows, the kernel walks the rows 16 at a time."""
    ll.set_tile(F32, skinny_index())
    N, K = 700, 900
    A, Bkn, C0 = wl.uniform((M, K), 640), wl.uniform((K, N), 641), wl.uniform((M, N), 642)
    for nt in (False, True):
        Bd = (Bkn.t().contiguous() if nt else Bkn).to(DEV)
        Cd = C0.to(DEV)
        (ll.gemm_f32_nt if nt else ll.gemm_f32)(A.to(DEV), Bd, Cd, -0.5, 1.0)
        torch.cuda.synchronize()
        R, T = oracle.gemm(np32(A), np32(Bkn), -0.5, 1.0, np32(C0))
        assert_close(np32(Cd), R, T, f"forced M={M} nt={nt}")


def test_batched_forced():
    """A strided batch runs the skinny kernel only when forced; each item's
    rows and columns stay its own."""
    ll.set_tile(F32, skinny_index())
    nb, M, N, K = 6, 5, 300, 260
    A, Bkn, C0 = wl.uniform((nb, M, K), 650), wl.uniform((nb, K, N), 651), wl.uniform((nb, M, N), 652)
    for tb in (False, True):
        Bd = (Bkn.transpose(1, 2).contiguous() if tb else Bkn).to(DEV)
        Cd = C0.to(DEV)
        ll.gemm_f32_batched(A.to(DEV), Bd, Cd, 1.5, 0.5, trans_b=tb)
        torch.cuda.synchronize()
        R, T = oracle.gemm_batched(np32(A), np32(Bkn), 1.5, 0.5, np32(C0))
        assert_close(np32(Cd), R, T, f"batched tb={tb}")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("nt", [False, True])
def test_decode_sized_layer_full_size(M, nt):
    """The layer's weight at full size (K 4096, N 11008) with a handful of
    rows: the automatic plan (skinny, K split over the CUs; 16 rows forced),
    checked on every element against the oracle."""
    N, K = 11008, 4096
    flags = F32 | ll.PLAN_RELU | (ll.PLAN_B_NK if nt else 0)
    if M > 8:
        force_skinny()
    name, s = plan(flags, M, N, K)
    assert name == SKINNY and s > 1
    X, Wkn, b = wl.uniform((M, K), 660, 0.125), wl.uniform((K, N), 661, 0.125), wl.bias_uniform(N, 662)
    Wd = (Wkn.t().contiguous() if nt else Wkn).to(DEV)
    Yd = torch.full((M, N), float("nan"), device=DEV)
    (ll.linear_bias_act_nt if nt else ll.linear_bias_act)(X.to(DEV), Wd, b.to(DEV), 1, Yd)
    torch.cuda.synchronize()
    R, T = oracle.linear(np32(X), np32(Wkn), np32(b), 1)
    assert_close(np32(Yd), R, T, f"decode M={M} nt={nt}")
