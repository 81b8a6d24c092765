"""GPU parity with unaligned operands, which run the register-staged kernels:
16-byte chunk loads at 4- or 2-byte alignment, and the chunk that crosses K
or N element by element. Leading dimensions 1-9 elements past a multiple,
base pointers shifted by 1-3 elements, K and N that are and are not chunk
multiples; against the float64 oracle element by element, guard columns
untouched."""
import numpy as np
import pytest

import linear_layer_amd as ll
import oracle
from linear_layer_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SHAPES = [(300, 264, 200), (1000, 1032, 512), (2047, 1376, 4096)]


@pytest.fixture(autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    ll.set_tile(ll.DTYPE_F32, -1)
    ll.set_tile(ll.DTYPE_F16, -1)
    ll.set_split_k(-1)
    ll.set_stream_k(-1)


def np32(t):
    return t.detach().cpu().numpy()


def view(host, pad, shift, fill=0.0):
    """A device view of `host` inside a buffer whose rows are pad elements
    longer, starting `shift` elements into the buffer; returns (buffer, view)."""
    rows, cols = host.shape
    buf = torch.full((rows, cols + pad + shift), fill, dtype=host.dtype, device=DEV)
    v = buf[:, shift:shift + cols]
    v.copy_(host.to(DEV))
    return buf, v


def check(got, R, T, what):
    bound = 1e-4 * T + np.spacing(np.abs(R).astype(np.float32)).astype(np.float64) / 2
    bad = ~(np.abs(np.asarray(got, np.float64) - R) <= bound)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside the bound"


def guards_ok(buf, shift, cols, fill):
    left = buf[:, :shift]
    right = buf[:, shift + cols:]
    return bool(torch.all(left == fill)) and bool(torch.all(right == fill))


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("pad,shift", [(1, 0), (2, 1), (3, 1)])
@pytest.mark.parametrize("nt", [False, True])
def test_f32_unaligned(M, N, K, pad, shift, nt):
    A, Bkn, C0 = wl.uniform((M, K), 501), wl.uniform((K, N), 502), wl.uniform((M, N), 503)
    _, Ad = view(A, pad, shift)
    _, Bd = view(Bkn.t().contiguous() if nt else Bkn, pad, shift)
    cbuf, Cd = view(C0, pad, shift, fill=7.0)
    (ll.gemm_f32_nt if nt else ll.gemm_f32)(Ad, Bd, Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    R, T = oracle.gemm(np32(A), np32(Bkn), 1.5, 0.5, np32(C0))
    check(np32(Cd), R, T, f"f32 {M}x{N}x{K} pad {pad} shift {shift} nt {nt}")
    assert guards_ok(cbuf, shift, N, 7.0)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("pad,shift", [(1, 1), (3, 0)])
@pytest.mark.parametrize("nt", [False, True])
def test_linear_unaligned(M, N, K, pad, shift, nt):
    X, Wkn, b = wl.uniform((M, K), 511, 0.125), wl.uniform((K, N), 512, 0.125), wl.bias_uniform(N, 513)
    _, Xd = view(X, pad, shift)
    _, Wd = view(Wkn.t().contiguous() if nt else Wkn, pad, shift)
    ybuf, Yd = view(torch.full((M, N), float("nan")), pad, shift, fill=7.0)
    (ll.linear_bias_act_nt if nt else ll.linear_bias_act)(Xd, Wd, b.to(DEV), 1, Yd)
    torch.cuda.synchronize()
    R, T = oracle.linear(np32(X), np32(Wkn), np32(b), 1)
    check(np32(Yd), R, T, f"linear {M}x{N}x{K} pad {pad} shift {shift} nt {nt}")
    assert guards_ok(ybuf, shift, N, 7.0)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("pad,shift", [(1, 1), (2, 0), (6, 3)])
@pytest.mark.parametrize("which,nt", [("f16", False), ("bf16", False), ("f16", True), ("bf16", True)])
def test_16bit_unaligned(M, N, K, pad, shift, which, nt):
    conv = wl.to_bf16 if which == "bf16" else wl.to_half
    A, Bkn = conv(wl.uniform((M, K), 521)), conv(wl.uniform((K, N), 522))
    C0 = wl.uniform((M, N), 523)
    _, Ad = view(A, pad, shift)
    _, Bd = view(Bkn.t().contiguous() if nt else Bkn, pad, shift)
    cbuf, Cd = view(C0, pad, shift, fill=7.0)
    fn = {("f16", False): ll.gemm_f16f32, ("bf16", False): ll.gemm_bf16f32,
          ("f16", True): ll.gemm_f16f32_nt, ("bf16", True): ll.gemm_bf16f32_nt}[(which, nt)]
    fn(Ad, Bd, Cd, -0.5, 1.0)
    torch.cuda.synchronize()
    R, T = oracle.gemm(wl.half_bits(A), wl.half_bits(Bkn), -0.5, 1.0, np32(C0), bf16=which == "bf16")
    check(np32(Cd), R, T, f"{which} {M}x{N}x{K} pad {pad} shift {shift} nt {nt}")
    assert guards_ok(cbuf, shift, N, 7.0)


def test_batched_unaligned_items():
    """Strided batch whose items start 1 element apart from 16-byte multiples."""
    nb, M, N, K = 5, 130, 72, 96
    A = wl.uniform((nb, M, K), 531)
    Bkn = wl.uniform((nb, K, N), 532)
    C0 = wl.uniform((nb, M, N), 533)
    flat_a = torch.zeros(nb * (M * K + 1) + 1, device=DEV)
    flat_b = torch.zeros(nb * (K * N + 1) + 1, device=DEV)
    flat_c = torch.zeros(nb * (M * N + 1) + 1, device=DEV)
    Ad = flat_a[1:1 + nb * (M * K + 1)].view(nb, M * K + 1)[:, :M * K].view(nb, M, K)
    Bd = flat_b[1:1 + nb * (K * N + 1)].view(nb, K * N + 1)[:, :K * N].view(nb, K, N)
    Cd = flat_c[1:1 + nb * (M * N + 1)].view(nb, M * N + 1)[:, :M * N].view(nb, M, N)
    Ad.copy_(A.to(DEV)); Bd.copy_(Bkn.to(DEV)); Cd.copy_(C0.to(DEV))
    ll.gemm_f32_batched(Ad, Bd, Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    R, T = oracle.gemm_batched(np32(A), np32(Bkn), 1.5, 0.5, np32(C0))
    check(np32(Cd), R, T, "batched unaligned items")


@pytest.mark.parametrize("M,N,K", [(301, 517, 203), (257, 263, 1001), (1000, 999, 997)])
@pytest.mark.parametrize("which", ["f32", "f16", "bf16", "linear"])
def test_ragged_k_and_n(M, N, K, which):
    """K and N that are not chunk multiples: whole chunks, then the crossing
    chunk element by element."""
    A, Bkn, C0 = wl.uniform((M, K), 541), wl.uniform((K, N), 542), wl.uniform((M, N), 543)
    if which == "linear":
        b = wl.bias_uniform(N, 544)
        _, Xd = view(A, 1, 0)
        _, Wd = view(Bkn, 1, 0)
        ybuf, Yd = view(torch.full((M, N), float("nan")), 1, 0, fill=7.0)
        ll.linear_bias_act(Xd, Wd, b.to(DEV), 1, Yd)
        torch.cuda.synchronize()
        R, T = oracle.linear(np32(A), np32(Bkn), np32(b), 1)
        check(np32(Yd), R, T, f"linear {M}x{N}x{K}")
        assert guards_ok(ybuf, 0, N, 7.0)
        return
    if which == "f32":
        Ad, Bd = A.to(DEV), Bkn.to(DEV)
        R, T = oracle.gemm(np32(A), np32(Bkn), 1.5, 0.5, np32(C0))
        fn = ll.gemm_f32
    else:
        conv = wl.to_bf16 if which == "bf16" else wl.to_half
        Ah, Bh = conv(A), conv(Bkn)
        Ad, Bd = Ah.to(DEV), Bh.to(DEV)
        R, T = oracle.gemm(wl.half_bits(Ah), wl.half_bits(Bh), 1.5, 0.5, np32(C0), bf16=which == "bf16")
        fn = ll.gemm_bf16f32 if which == "bf16" else ll.gemm_f16f32
    cbuf, Cd = view(C0, 0, 0)
    fn(Ad, Bd, Cd, 1.5, 0.5)
    torch.cuda.synchronize()
    check(np32(Cd), R, T, f"{which} {M}x{N}x{K}")
