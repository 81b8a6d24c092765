"""The no-allocation fused layer (linear_bias_act_noalloc), called through the
C ABI: its output against linear_bias_act_ws on the same inputs and against
the float64 oracle, on two calls in a row (the second smaller) that share the
library's static workspace; shapes whose plan needs more workspace than the
static array are refused and leave Y untouched; decode-sized plans (a few rows,
K split, no workspace); a call on a stream of its own; and the call captured
in a HIP graph, a stream-K plan and a K-split one, replayed with new inputs."""
import ctypes

import numpy as np
import pytest

import linear_layer_amd as ll
import oracle
from linear_layer_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32 = ll.DTYPE_F32


@pytest.fixture(autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.fixture
def auto_plan():
    """Every test here starts and ends with the automatic plan."""
    ll.set_tile(F32, -1)
    ll.set_stream_k(-1)
    ll.set_split_k(-1)
    ll.set_noalloc_limit(-1)
    yield
    ll.set_tile(F32, -1)
    ll.set_stream_k(-1)
    ll.set_noalloc_limit(-1)


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def np32(t):
    return t.detach().cpu().numpy()


def bound(R, T):
    return 1e-4 * T + np.spacing(np.abs(R).astype(np.float32)).astype(np.float64) / 2


def call(lib_fn, X, W, b, act, Y, w_trans, *ws):
    """One call of a fused-layer entry point through the C ABI on torch's
    current stream; returns the status."""
    s = torch.cuda.current_stream().cuda_stream
    ldw = W.stride(0)
    return lib_fn(X.shape[0], Y.shape[1], X.shape[1], X.data_ptr(), X.stride(0), W.data_ptr(), ldw,
                  int(w_trans), None if b is None else b.data_ptr(), act, Y.data_ptr(), Y.stride(0),
                  *ws, s)


def both(X, W, b, act, w_trans):
    """(Y from linear_bias_act_noalloc, Y from linear_bias_act_ws) on device
    copies of the host inputs (W given K-by-N, handed over N-by-K when
    w_trans), each Y NaN-filled first."""
    lib = ll.load()
    M, K = X.shape
    N = W.shape[1]
    Xd, Wd = X.to(DEV), (W.t().contiguous() if w_trans else W).to(DEV)
    bd = None if b is None else b.to(DEV)
    need = ll.linear_workspace_size(M, N, K, w_trans, act, cus())
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=DEV)
    Yn = torch.full((M, N), float("nan"), device=DEV)
    Yw = torch.full((M, N), float("nan"), device=DEV)
    assert call(lib.linear_bias_act_noalloc, Xd, Wd, bd, act, Yn, w_trans) == ll.OK
    assert call(lib.linear_bias_act_ws, Xd, Wd, bd, act, Yw, w_trans, ws.data_ptr(),
                ctypes.c_int64(ws.numel())) == ll.OK
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws)) == 0
    return np32(Yn), np32(Yw), need


def check(case, X, W, b, act, w_trans, integer):
    got, ref, need = both(X, W, b, act, w_trans)
    R, T = oracle.linear(np32(X), np32(W), None if b is None else np32(b), act)
    if integer:
        assert np.array_equal(got, ref), f"{case}: noalloc and ws differ"
        assert np.array_equal(got, R.astype(np.float32)), f"{case}: noalloc differs from the oracle"
    else:
        B = bound(R, T)
        bad = ~(np.abs(got.astype(np.float64) - R) <= B)
        assert not bad.any(), f"{case}: {bad.sum()} of {bad.size} outside the oracle bound"
        bad = ~(np.abs(got.astype(np.float64) - ref.astype(np.float64)) <= 2 * B)
        assert not bad.any(), f"{case}: {bad.sum()} of {bad.size} away from linear_bias_act_ws"
    if act:
        assert not np.any(np.signbit(got))
    return need


@pytest.mark.parametrize("integer", [True, False])
@pytest.mark.parametrize("w_trans", [False, True])
def test_two_calls_second_smaller(integer, w_trans, auto_plan):
    """The fused-layer workload 2047x4096x11008 (a stream-K hybrid using the
    static workspace), then a smaller stream-K layer on the same workspace:
    the second call reads only counters and partials the first left zeroed."""
    w = wl.WORKLOADS["linear_relu_2047x4096x11008"]
    x = wl.make_inputs(w, integer=integer)
    need1 = check("first call", x["A"], x["B"], x["bias"], 1, w_trans, integer)
    assert 0 < need1 <= ll.NOALLOC_SCRATCH_BYTES
    M, N, K = 1536, 1536, 256
    ll.set_tile(F32, 3)
    ll.set_stream_k(1)
    flags = F32 | ll.PLAN_RELU | (ll.PLAN_B_NK if w_trans else 0)
    assert ll.chosen_stream_k(flags, M, N, K, cus()) > 0
    if integer:
        X, W, b = (wl.integers((M, K), 301, -2, 2), wl.integers((K, N), 302, -2, 2),
                   wl.integers((N,), 303, -4, 4))
    else:
        X, W, b = wl.uniform((M, K), 301, 0.125), wl.uniform((K, N), 302, 0.125), wl.bias_uniform(N, 303)
    need2 = check("second call", X, W, b, 1, w_trans, integer)
    assert 0 < need2 < need1


@pytest.mark.parametrize("shape,act,with_bias", [((330, 270, 520), 0, False),
                                                 ((257, 300, 200), 1, True),
                                                 ((4096, 4096, 512), 1, True)])
def test_small_and_whole_tile_plans(shape, act, with_bias, auto_plan):
    """Plans with and without shared tiles, with and without bias and ReLU."""
    M, N, K = shape
    X, W = wl.uniform((M, K), 311, 0.125), wl.uniform((K, N), 312, 0.125)
    b = wl.bias_uniform(N, 313) if with_bias else None
    check(f"{M}x{N}x{K}", X, W, b, act, False, False)


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("w_trans", [False, True])
def test_decode_sized_plans(M, w_trans, auto_plan):
    """A few rows against the 4096 x 11008 weight: the skinny kernel (1 and 4
    rows) or the 32x128 tile (16 rows) with K split over the CUs, so bias
    fill, atomic partial sums and ReLU pass, and no workspace."""
    N, K = 11008, 4096
    flags = F32 | ll.PLAN_RELU | (ll.PLAN_B_NK if w_trans else 0)
    assert ll.tile_name(F32, ll.chosen_tile(flags, M, N, K, cus())) == (
        "f32_16x256_skinny" if M <= 4 else "f32_32x128")
    assert ll.chosen_split_k(flags, M, N, K, cus()) > 1
    X, W, b = wl.uniform((M, K), 321, 0.125), wl.uniform((K, N), 322, 0.125), wl.bias_uniform(N, 323)
    assert check(f"decode {M} rows w_trans={w_trans}", X, W, b, 1, w_trans, False) == 0


def test_too_large_is_refused(auto_plan):
    """A shape whose plan needs more than the usable static workspace is
    refused with LL_ERR_INVALID_VALUE before anything runs: Y keeps its NaNs.
    (No plan on 256 CUs needs the whole array, so the usable part is lowered
    to 16 MiB for the fused-layer workload's 22 MiB.)"""
    M, N, K = 2047, 11008, 4096
    need = ll.linear_workspace_size(M, N, K, False, 1, cus())
    assert 16 << 20 < need <= ll.NOALLOC_SCRATCH_BYTES
    ll.set_noalloc_limit(16 << 20)
    lib = ll.load()
    X = torch.zeros((M, K), device=DEV)
    W = torch.zeros((K, N), device=DEV)
    Y = torch.full((M, N), float("nan"), device=DEV)
    assert call(lib.linear_bias_act_noalloc, X, W, None, 1, Y, False) == ll.ERR_INVALID_VALUE
    torch.cuda.synchronize()
    assert bool(torch.isnan(Y).all())
    with pytest.raises(ll.LinearLayerError):
        ll.linear_bias_act_noalloc(X, W, None, 1, Y)
    ll.set_noalloc_limit(need)   # exactly enough: runs
    assert call(lib.linear_bias_act_noalloc, X, W, None, 1, Y, False) == ll.OK
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(Y)) == 0


def test_largest_plans_fit(auto_plan):
    """Plans that share out most of a round of tiles fit the static array:
    4096 x 11008 x 4096 (44 MiB of workspace) and 3000 x 5000 x 11008 (60 MiB),
    integer inputs, bit for bit against linear_bias_act_ws."""
    for (M, N, K), seed in (((4096, 11008, 4096), 361), ((3000, 5000, 11008), 365)):
        need = ll.linear_workspace_size(M, N, K, False, 1, cus())
        assert 40 << 20 < need <= ll.NOALLOC_SCRATCH_BYTES
        X, W = wl.integers((M, K), seed, -2, 2), wl.integers((K, N), seed + 1, -1, 1)
        b = wl.integers((N,), seed + 2, -4, 4)
        got, ref, _ = both(X, W, b, 1, False)
        assert np.array_equal(got, ref), f"{M}x{N}x{K}: noalloc and ws differ"
        assert not np.isnan(got).any()


def test_argument_errors(auto_plan):
    lib = ll.load()
    X = torch.zeros((8, 8), device=DEV)
    W = torch.zeros((8, 8), device=DEV)
    Y = torch.zeros((8, 8), device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    args = (8, 8, 8, X.data_ptr(), 8, W.data_ptr(), 8)
    E = ll.ERR_INVALID_VALUE
    assert lib.linear_bias_act_noalloc(*args, 2, None, 1, Y.data_ptr(), 8, s) == E
    assert lib.linear_bias_act_noalloc(*args, 0, None, 5, Y.data_ptr(), 8, s) == E
    assert lib.linear_bias_act_noalloc(*args, 0, None, 1, Y.data_ptr(), 4, s) == E
    assert lib.linear_bias_act_noalloc(*args, 0, None, 1, Y.data_ptr(), 8, s) == ll.OK
    torch.cuda.synchronize()


def test_non_default_stream(auto_plan):
    """On a stream of its own (same device): the same result as
    linear_bias_act_ws on the default stream, and the stream check passes."""
    M, N, K = 330, 270, 520
    X, W = wl.uniform((M, K), 321, 0.125), wl.uniform((K, N), 322, 0.125)
    b = wl.bias_uniform(N, 323)
    Xd, Wd, bd = X.to(DEV), W.to(DEV), b.to(DEV)
    side = torch.cuda.Stream()
    Yn = torch.full((M, N), float("nan"), device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ll.linear_bias_act_noalloc(Xd, Wd, bd, 1, Yn)
    side.synchronize()
    torch.cuda.current_stream().wait_stream(side)
    R, T = oracle.linear(np32(X), np32(W), np32(b), 1)
    bad = ~(np.abs(np32(Yn).astype(np.float64) - R) <= bound(R, T))
    assert not bad.any(), f"{bad.sum()} of {bad.size} outside the oracle bound"


def test_graph_capture_replays(auto_plan):
    """The use the entry point exists for: captured once in a HIP graph (no
    allocation, no memset inside), then replayed three times with new inputs
    written eagerly between the replays; every replay against the oracle and
    against an eager linear_bias_act_ws call on the same inputs."""
    w = wl.WORKLOADS["linear_relu_2047x4096x11008"]
    M, N, K = w.M, w.N, w.K
    need = ll.linear_workspace_size(M, N, K, False, 1, cus())
    assert 0 < need <= ll.NOALLOC_SCRATCH_BYTES   # a stream-K plan that uses the static array
    Xd = torch.empty((M, K), device=DEV)
    Wd = torch.empty((K, N), device=DEV)
    bd = torch.empty((N,), device=DEV)
    Y = torch.empty((M, N), device=DEV)
    x = wl.make_inputs(w, integer=True)
    Xd.copy_(x["A"]); Wd.copy_(x["B"]); bd.copy_(x["bias"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # first call outside the capture: device set-up
        ll.linear_bias_act_noalloc(Xd, Wd, bd, 1, Y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ll.linear_bias_act_noalloc(Xd, Wd, bd, 1, Y)
    torch.cuda.synchronize()
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for rep in range(3):
        X = wl.integers((M, K), 330 + rep, -2, 2)
        Wh = wl.integers((K, N), 340 + rep, -2, 2)
        b = wl.integers((N,), 350 + rep, -4, 4)
        Xd.copy_(X); Wd.copy_(Wh); bd.copy_(b)
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = np32(Y)
        Ye = torch.full((M, N), float("nan"), device=DEV)
        ll.linear_bias_act_ws(Xd, Wd, bd, 1, Ye, ws)
        torch.cuda.synchronize()
        assert np.array_equal(got, np32(Ye)), f"replay {rep}: graph and eager call differ"
        R, _ = oracle.linear(np32(X), np32(Wh), np32(b), 1)
        assert np.array_equal(got, R.astype(np.float32)), f"replay {rep}: differs from the oracle"
        assert int(torch.count_nonzero(ws)) == 0
    del g


@pytest.mark.parametrize("M", [1, 16])
def test_graph_capture_replays_split_plan(M, auto_plan):
    """A decode-sized call (a few rows against the 4096 x 11008 weight: bias
    fill, K-split atomics and ReLU pass, three launches) captured in a graph
    and replayed three times with new integer inputs; every replay bit-exact
    against the oracle."""
    N, K = 11008, 4096
    assert ll.chosen_split_k(F32 | ll.PLAN_RELU, M, N, K, cus()) > 1
    Xd = torch.empty((M, K), device=DEV)
    Wd = torch.empty((K, N), device=DEV)
    bd = torch.empty((N,), device=DEV)
    Y = torch.empty((M, N), device=DEV)
    Xd.zero_(); Wd.zero_(); bd.zero_()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # first call outside the capture: device set-up
        ll.linear_bias_act_noalloc(Xd, Wd, bd, 1, Y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ll.linear_bias_act_noalloc(Xd, Wd, bd, 1, Y)
    torch.cuda.synchronize()
    for rep in range(3):
        X = wl.integers((M, K), 360 + rep, -2, 2)
        Wh = wl.integers((K, N), 370 + rep, -2, 2)
        b = wl.integers((N,), 380 + rep, -4, 4)
        Xd.copy_(X); Wd.copy_(Wh); bd.copy_(b)
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        R, _ = oracle.linear(np32(X), np32(Wh), np32(b), 1)
        assert np.array_equal(np32(Y), R.astype(np.float32)), f"replay {rep}: differs from the oracle"
    del g
