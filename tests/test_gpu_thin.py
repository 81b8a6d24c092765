"""GPU parity of the 32x128 FP32 tile (two-wave workgroups for products of 9
to 32 rows): shapes the automatic plan gives it, with and without K-splits,
both B layouts, every epilogue, ragged M, N and K, the staged fallback for
unaligned operands, and a full-size layer; against the float64 oracle element
by element, and bit-exact on integer inputs."""
import numpy as np
import pytest

import linear_layer_amd as ll
import oracle
from linear_layer_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32 = ll.DTYPE_F32
THIN = "f32_32x128"


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


def plan(flags, M, N, K):
    return (ll.tile_name(F32, ll.chosen_tile(flags, M, N, K, cus())),
            ll.chosen_split_k(flags, M, N, K, cus()))


def thin_index():
    return [ll.tile_name(F32, t) for t in range(ll.num_tiles(F32))].index(THIN)


def assert_close(got, R, T, what):
    bound = 1e-4 * T + np.spacing(np.abs(R).astype(np.float32)).astype(np.float64) / 2
    bad = ~(np.abs(np.asarray(got, np.float64) - R) <= bound)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside the bound"


@pytest.mark.parametrize("M,N,K", [(9, 11008, 4096), (16, 11008, 4096), (32, 4096, 11008),
                                   (12, 8192, 8192)])
def test_automatic_plan_takes_it(M, N, K):
    """These shapes (the planner's own choice) run the 32x128 tile."""
    for flags in (F32, F32 | ll.PLAN_B_NK, F32 | ll.PLAN_RELU):
        assert plan(flags, M, N, K)[0] == THIN
    assert plan(F32 | ll.PLAN_UNALIGNED, M, N, K)[0] != THIN   # direct kernel only
    assert plan(F32, 33, N, K)[0] != THIN                       # two rows of tiles


@pytest.mark.parametrize("M", [9, 17, 31, 32, 33, 70])
@pytest.mark.parametrize("N,K", [(1000, 777), (384, 2048), (129, 64)])
@pytest.mark.parametrize("nt", [False, True])
def test_forced_ragged(M, N, K, nt):
    """Forced on ragged shapes (rows past one tile row included), alpha and beta."""
    ll.set_tile(F32, thin_index())
    A, Bkn, C0 = wl.uniform((M, K), 700 + M), wl.uniform((K, N), 701), wl.uniform((M, N), 702)
    Bd = (Bkn.t().contiguous() if nt else Bkn).to(DEV)
    Cd = C0.to(DEV)
    (ll.gemm_f32_nt if nt else ll.gemm_f32)(A.to(DEV), Bd, Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    R, T = oracle.gemm(np32(A), np32(Bkn), 1.5, 0.5, np32(C0))
    assert_close(np32(Cd), R, T, f"{M}x{N}x{K} nt={nt}")


@pytest.mark.parametrize("splits", [1, 3, 16])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (-0.5, 1.0)])
@pytest.mark.parametrize("nt", [False, True])
def test_forced_splits_integer_exact(splits, alpha, beta, nt):
    """Integer inputs through the K-split atomics: the oracle's result bit for
    bit; beta = 0 ignores NaN in C."""
    ll.set_tile(F32, thin_index())
    ll.set_split_k(splits)
    M, N, K = 24, 520, 3000
    A, Bkn = wl.integers((M, K), 710, -2, 2), wl.integers((K, N), 711, -2, 2)
    C0 = wl.integers((M, N), 712, -4, 4) if beta else torch.full((M, N), float("nan"))
    Bd = (Bkn.t().contiguous() if nt else Bkn).to(DEV)
    Cd = C0.to(DEV)
    (ll.gemm_f32_nt if nt else ll.gemm_f32)(A.to(DEV), Bd, Cd, alpha, beta)
    torch.cuda.synchronize()
    R, _ = oracle.gemm(np32(A), np32(Bkn), alpha, beta, np32(C0) if beta else None)
    bad = np32(Cd) != R.astype(np.float32)
    assert not bad.any(), f"splits {splits} a={alpha} b={beta} nt={nt}: {bad.sum()} differ"


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("splits", [1, 4])
def test_linear(act, nt, splits):
    ll.set_tile(F32, thin_index())
    ll.set_split_k(splits)
    M, N, K = 20, 1100, 1300
    X, Wkn = wl.uniform((M, K), 720, 0.125), wl.uniform((K, N), 721, 0.125)
    b = wl.bias_uniform(N, 722)
    Wd = (Wkn.t().contiguous() if nt else Wkn).to(DEV)
    Yd = torch.full((M, N), float("nan"), device=DEV)
    (ll.linear_bias_act_nt if nt else ll.linear_bias_act)(X.to(DEV), Wd, b.to(DEV), act, Yd)
    torch.cuda.synchronize()
    R, T = oracle.linear(np32(X), np32(Wkn), np32(b), act)
    got = np32(Yd)
    assert_close(got, R, T, f"linear act={act} nt={nt} splits={splits}")
    if act:
        assert not np.any(np.signbit(got))


def test_unaligned_operands_run_the_staged_fallback():
    """Forced with a leading dimension off 16 bytes: the staged 64x64 kernel
    runs instead, and the result is the oracle's; guard columns untouched."""
    ll.set_tile(F32, thin_index())
    M, N, K = 20, 300, 260
    A, Bkn, C0 = wl.uniform((M, K), 730), wl.uniform((K, N), 731), wl.uniform((M, N), 732)
    abuf = torch.zeros((M, K + 1), device=DEV); Ad = abuf[:, :K]; Ad.copy_(A.to(DEV))
    cbuf = torch.full((M, N + 3), 7.0, device=DEV); Cd = cbuf[:, :N]; Cd.copy_(C0.to(DEV))
    ll.gemm_f32(Ad, Bkn.to(DEV), Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    R, T = oracle.gemm(np32(A), np32(Bkn), 1.5, 0.5, np32(C0))
    assert_close(np32(Cd), R, T, "unaligned")
    assert bool(torch.all(cbuf[:, N:] == 7.0))


@pytest.mark.parametrize("nt", [False, True])
def test_full_size_layer(nt):
    """Sixteen rows of X against the 4096 x 11008 weight (11 K-splits, the
    automatic plan), every element against the oracle."""
    M, N, K = 16, 11008, 4096
    flags = F32 | ll.PLAN_RELU | (ll.PLAN_B_NK if nt else 0)
    assert plan(flags, M, N, K)[0] == THIN
    X, Wkn, b = wl.uniform((M, K), 740, 0.125), wl.uniform((K, N), 741, 0.125), wl.bias_uniform(N, 742)
    Wd = (Wkn.t().contiguous() if nt else Wkn).to(DEV)
    Yd = torch.full((M, N), float("nan"), device=DEV)
    (ll.linear_bias_act_nt if nt else ll.linear_bias_act)(X.to(DEV), Wd, b.to(DEV), 1, Yd)
    torch.cuda.synchronize()
    R, T = oracle.linear(np32(X), np32(Wkn), np32(b), 1)
    assert_close(np32(Yd), R, T, f"full nt={nt}")
