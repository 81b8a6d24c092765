"""GPU parity on seeded random shapes under the automatic plan (no overrides):
every product family and the fused layer, both B layouts, ragged sizes from 1
to a few thousand, padded and unaligned leading dimensions, against the
float64 oracle element by element. The forced-tile tests cover each kernel;
these cover what the planner picks (tile, K-split, K-slices, stream-K) on
shapes nobody chose by hand."""
import numpy as np
import pytest

import linear_layer_amd as ll
import oracle
from linear_layer_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KINDS = ["gemm_f32", "gemm_f32_nt", "gemm_f16f32", "gemm_bf16f32", "gemm_f16f32_nt",
         "gemm_bf16f32_nt", "linear", "linear_nt"]
AB = [(1.0, 0.0), (1.5, 0.5), (-0.5, 1.0)]


def draw_cases(n=80, seed=20261202, max_macs=1.2e10):
    """(kind, M, N, K, pad, alpha, beta, act, bias): half the cases with
    log-uniform sizes in [1, 3000], half with uniform sizes in [512, 3000]
    (so that the larger tiles, stream-K and K-slices come up too); pad = extra
    leading-dimension elements (3 breaks the 16-byte alignment and sends the
    call down the scalar-load path)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        kind = KINDS[len(out) % len(KINDS)]
        if len(out) % 2 == 0:
            M, N, K = (int(round(np.exp(rng.uniform(0.0, np.log(3000.0))))) for _ in range(3))
        else:
            M, N, K = (int(rng.integers(512, 3001)) for _ in range(3))
        if float(M) * N * K > max_macs:
            continue
        pad = int(rng.choice([0, 0, 0, 8, 3]))
        alpha, beta = AB[int(rng.integers(len(AB)))]
        act = int(rng.integers(2))
        bias = bool(rng.integers(4) != 0)
        out.append((kind, M, N, K, pad, alpha, beta, act, bias))
    return out


CASES = draw_cases()


@pytest.fixture(autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    ll.set_tile(ll.DTYPE_F32, -1)
    ll.set_tile(ll.DTYPE_F16, -1)
    ll.set_split_k(-1)
    ll.set_stream_k(-1)


def padded(host, pad, dtype=None):
    """A device view of `host` whose leading dimension is pad elements longer."""
    rows, cols = host.shape
    base = torch.zeros((rows, cols + pad), dtype=dtype or host.dtype, device=DEV)
    view = base[:, :cols]
    view.copy_(host.to(DEV))
    return base, view


def np32(t):
    return t.detach().cpu().numpy()


def plan_of(kind, M, N, K, act):
    f16 = "16" in kind
    flags = (ll.DTYPE_F16 if f16 else ll.DTYPE_F32) | (ll.PLAN_B_NK if kind.endswith("_nt") else 0)
    if kind.startswith("linear") and act:
        flags |= ll.PLAN_RELU
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return (ll.tile_name(ll.DTYPE_F16 if f16 else ll.DTYPE_F32, ll.chosen_tile(flags, M, N, K, cus)),
            ll.chosen_split_k(flags, M, N, K, cus), ll.chosen_stream_k(flags, M, N, K, cus))


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-pad{c[4]}" for c in CASES])
def test_random_shape_automatic_plan(case):
    kind, M, N, K, pad, alpha, beta, act, with_bias = case
    seed = 7000 + CASES.index(case) * 4
    nt = kind.endswith("_nt")
    A = wl.uniform((M, K), seed)
    Bkn = wl.uniform((K, N), seed + 1)        # B (or W) as K-by-N
    plan = plan_of(kind, M, N, K, act)
    what = f"{kind} {M}x{N}x{K} pad {pad} plan {plan}"
    if kind.startswith("linear"):
        b = wl.bias_uniform(N, seed + 2) if with_bias else None
        _, Xd = padded(A, pad)
        _, Wd = padded(Bkn.t().contiguous() if nt else Bkn, pad)
        out, Yd = padded(torch.full((M, N), float("nan")), pad)
        fn = ll.linear_bias_act_nt if nt else ll.linear_bias_act
        fn(Xd, Wd, None if b is None else b.to(DEV), act, Yd)
        torch.cuda.synchronize()
        R, T = oracle.linear(np32(A), np32(Bkn), None if b is None else np32(b), act)
        got = np32(Yd)
    else:
        C0 = wl.uniform((M, N), seed + 3)
        if "16" in kind:
            conv = wl.to_bf16 if "bf16" in kind else wl.to_half
            Ah, Bh = conv(A), conv(Bkn)
            _, Ad = padded(Ah, pad)
            _, Bd = padded(Bh.t().contiguous() if nt else Bh, pad)
            R, T = oracle.gemm(wl.half_bits(Ah), wl.half_bits(Bh), alpha, beta, np32(C0),
                               bf16="bf16" in kind)
        else:
            _, Ad = padded(A, pad)
            _, Bd = padded(Bkn.t().contiguous() if nt else Bkn, pad)
            R, T = oracle.gemm(np32(A), np32(Bkn), alpha, beta, np32(C0))
        out, Cd = padded(C0, pad)
        getattr(ll, kind)(Ad, Bd, Cd, alpha, beta)
        torch.cuda.synchronize()
        got = np32(Cd)
    assert not torch.any(out[:, N:] != 0), f"{what}: guard columns written"
    bound = 1e-4 * T + np.spacing(np.abs(R).astype(np.float32)).astype(np.float64) / 2
    bad = ~(np.abs(got.astype(np.float64) - R) <= bound)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside the bound"


def draw_batched(n=24, seed=20261203, max_macs=2.0e9):
    """(dtype, trans_b, batch, M, N, K, alpha, beta) for the strided-batch
    entry points: batch in [1, 48], log-uniform sizes in [1, 700]."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dt = ["f32", "f16", "bf16"][len(out) % 3]
        nb = int(rng.integers(1, 49))
        M, N, K = (int(round(np.exp(rng.uniform(0.0, np.log(700.0))))) for _ in range(3))
        if float(nb) * M * N * K > max_macs:
            continue
        alpha, beta = AB[int(rng.integers(len(AB)))]
        out.append((dt, bool(rng.integers(2)), nb, M, N, K, alpha, beta))
    return out


BATCHED = draw_batched()


@pytest.mark.parametrize("case", BATCHED,
                         ids=[f"{c[0]}-{'nt' if c[1] else 'nn'}-b{c[2]}-{c[3]}x{c[4]}x{c[5]}" for c in BATCHED])
def test_random_batched_automatic_plan(case):
    dt, tb, nb, M, N, K, alpha, beta = case
    seed = 9000 + BATCHED.index(case) * 4
    A = wl.uniform((nb, M, K), seed)
    Bkn = wl.uniform((nb, K, N), seed + 1)
    C0 = wl.uniform((nb, M, N), seed + 2)
    Bg = Bkn.transpose(1, 2).contiguous() if tb else Bkn
    if dt == "f32":
        R, T = oracle.gemm_batched(np32(A), np32(Bkn), alpha, beta, np32(C0))
        Ad, Bd = A.to(DEV), Bg.to(DEV)
        fn = ll.gemm_f32_batched
    else:
        conv = wl.to_bf16 if dt == "bf16" else wl.to_half
        Ah, Bh = conv(A), conv(Bkn)
        R, T = oracle.gemm_batched(wl.half_bits(Ah), wl.half_bits(Bh), alpha, beta, np32(C0),
                                   bf16=dt == "bf16")
        Ad = Ah.to(DEV)
        Bd = (Bh.transpose(1, 2).contiguous() if tb else Bh).to(DEV)
        fn = ll.gemm_bf16f32_batched if dt == "bf16" else ll.gemm_f16f32_batched
    Cd = C0.to(DEV)
    fn(Ad, Bd, Cd, alpha, beta, trans_b=tb)
    torch.cuda.synchronize()
    got = np32(Cd).astype(np.float64)
    bound = 1e-4 * T + np.spacing(np.abs(R).astype(np.float32)).astype(np.float64) / 2
    bad = ~(np.abs(got - R) <= bound)
    assert not bad.any(), f"{case}: {bad.sum()} of {bad.size} outside the bound"
