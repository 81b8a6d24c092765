"""GPU parity at the far end of the address range.

The kernels form every operand address in 64 bits. These cases place the last
rows of A, B and C (and the last items of a batch) more than 2^31 elements and
2^32 bytes from their base pointers, with leading dimensions that are still
valid ints, and compare every output element with the float64 oracle under the
same tolerance as the other parity tests (bit-exact is not asked: the operands
are uniform, not integer-valued).

Each case carves its operands out of three device buffers of about 11 GiB,
filled beforehand with a pattern that is NaN as fp32, fp16 and bf16, so a read
outside an operand's rows or columns turns its output into NaN, and a write
outside C is seen in the guard columns checked after each call.
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
T32 = list(range(ll.num_tiles(F32)))
T16 = list(range(ll.num_tiles(F16)))

M, N, K = 600, 300, 168          # ragged against every tile and stage depth
LDA = 2 ** 22 + 64               # row M-1 of A starts 2.51e9 elements in
LDB_NN = 2 ** 24 + 64            # row K-1 of a K-by-N B: 2.80e9
LDB_NT = 2 ** 23 + 64            # row N-1 of an N-by-K B: 2.51e9
LDC = 2 ** 22 + 128              # row M-1 of C: 2.51e9
BUF_BYTES = (K * LDB_NN + 64) * 4
NAN16 = 0x7FC0                   # NaN as fp16 and bf16; 0x7FC07FC0 is NaN as fp32


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    out = {k: torch.empty(BUF_BYTES // 2, dtype=torch.int16, device=DEV) for k in ("A", "B", "C")}
    yield out
    out.clear()
    torch.cuda.empty_cache()


@pytest.fixture
def bufs(big):
    """The three buffers, refilled with the NaN pattern for each case."""
    for b in big.values():
        b.fill_(NAN16)
    return big


@pytest.fixture
def tile():
    forced = []

    def force(dtype, t):
        ll.set_tile(dtype, t)
        forced.append(dtype)

    yield force
    for d in forced:
        ll.set_tile(d, -1)


def view(buf, dtype, rows, cols, ld):
    """A rows-by-cols row-major matrix with leading dimension ld at the buffer's base."""
    flat = buf.view(dtype)
    assert (rows - 1) * ld + cols <= flat.numel()
    return flat.as_strided((rows, cols), (ld, 1))


def place(buf, host, ld):
    """Copy a host matrix into the buffer with leading dimension ld; return the view."""
    v = view(buf, host.dtype, host.shape[0], host.shape[1], ld)
    v.copy_(host.to(DEV))
    return v


def out_view(bufs, ld=LDC, rows=M, cols=N):
    return view(bufs["C"], torch.float32, rows, cols, ld)


def guards_untouched(bufs, ld=LDC, rows=M, cols=N):
    """The 64 floats after each row of C (and after the last row) are still the fill."""
    flat = bufs["C"].view(torch.float32)
    g = flat.as_strided((rows, 64), (ld, 1), cols).cpu().view(torch.int32)
    assert torch.all(g == (NAN16 << 16 | NAN16)), "a write outside C"


def assert_close(gpu, R, T, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    half_ulp = np.spacing(np.abs(R).astype(np.float32)).astype(np.float64) / 2
    err = np.abs(gpu - R)
    bad = ~(err <= 1e-4 * T + half_ulp)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside bound; first at flat {i}: "
                             f"gpu={gpu.ravel()[i]!r} oracle={R.ravel()[i]!r}")


def test_layout_reaches_past_32_bits():
    """The leading dimensions above do put the last rows beyond 2^31 elements and
    2^32 bytes (fp32) while fitting a C int."""
    for ld, rows in ((LDA, M), (LDB_NN, K), (LDB_NT, N), (LDC, M)):
        assert ld < 2 ** 31 and (rows - 1) * ld > 2 ** 31 and (rows - 1) * ld * 4 > 2 ** 32
    assert (K - 1) * LDB_NN + N <= BUF_BYTES // 4


@pytest.mark.parametrize("t", T32)
@pytest.mark.parametrize("trans_b", [False, True])
def test_f32_far_rows(bufs, t, trans_b, tile):
    tile(F32, t)
    A = wl.uniform((M, K), 301)
    B = wl.uniform((N, K) if trans_b else (K, N), 302)
    C0 = wl.uniform((M, N), 303)
    Av = place(bufs["A"], A, LDA)
    Bv = place(bufs["B"], B, LDB_NT if trans_b else LDB_NN)
    Cv = out_view(bufs)
    Cv.copy_(C0.to(DEV))
    (ll.gemm_f32_nt if trans_b else ll.gemm_f32)(Av, Bv, Cv, 1.5, 0.5)
    torch.cuda.synchronize()
    R, T = oracle.gemm(A.numpy(), B.numpy(), 1.5, 0.5, C0.numpy(), b_trans=trans_b)
    assert_close(Cv.cpu().numpy(), R, T, f"f32 tile {t} tb={trans_b}")
    guards_untouched(bufs)


def test_f32_far_rows_unaligned(bufs):
    """Leading dimensions that are not multiples of four take the kernel that reads
    scalars; its addresses are 64-bit too."""
    A = wl.uniform((M, K), 311)
    B = wl.uniform((K, N), 312)
    Av = place(bufs["A"], A, LDA + 1)
    Bv = place(bufs["B"], B, LDB_NN - 3)
    Cv = out_view(bufs, LDC + 1)
    ll.gemm_f32(Av, Bv, Cv)
    torch.cuda.synchronize()
    R, T = oracle.gemm(A.numpy(), B.numpy())
    assert_close(Cv.cpu().numpy(), R, T, "f32 unaligned")
    guards_untouched(bufs, LDC + 1)


@pytest.mark.parametrize("t", T16)
@pytest.mark.parametrize("which,trans_b", [("f16", False), ("bf16", True), ("bf16", False),
                                           ("f16", True)])
def test_16bit_far_rows(bufs, t, which, trans_b, tile):
    """16-bit operands at twice the leading dimension: the far rows lie beyond 2^32
    elements."""
    tile(F16, t)
    dt = torch.float16 if which == "f16" else torch.bfloat16
    A = wl.uniform((M, K), 321).to(dt)
    B = wl.uniform((N, K) if trans_b else (K, N), 322).to(dt)
    Av = place(bufs["A"], A, 2 * LDA)
    Bv = place(bufs["B"], B, 2 * (LDB_NT if trans_b else LDB_NN))
    Cv = out_view(bufs)
    fn = {("f16", False): ll.gemm_f16f32, ("f16", True): ll.gemm_f16f32_nt,
          ("bf16", False): ll.gemm_bf16f32, ("bf16", True): ll.gemm_bf16f32_nt}[(which, trans_b)]
    fn(Av, Bv, Cv)
    torch.cuda.synchronize()
    R, T = oracle.gemm(wl.half_bits(A), wl.half_bits(B), bf16=which == "bf16", b_trans=trans_b)
    assert_close(Cv.cpu().numpy(), R, T, f"{which} tile {t} tb={trans_b}")
    guards_untouched(bufs)


@pytest.mark.parametrize("trans_w", [False, True])
def test_linear_far_rows(bufs, trans_w):
    X = wl.uniform((M, K), 331)
    W = wl.uniform((N, K) if trans_w else (K, N), 332)
    b = wl.bias_uniform(N, 333)
    Xv = place(bufs["A"], X, LDA)
    Wv = place(bufs["B"], W, LDB_NT if trans_w else LDB_NN)
    Yv = out_view(bufs)
    (ll.linear_bias_act_nt if trans_w else ll.linear_bias_act)(Xv, Wv, b.to(DEV), 1, Yv)
    torch.cuda.synchronize()
    R, T = oracle.linear(X.numpy(), W.numpy(), b.numpy(), 1, w_trans=trans_w)
    assert_close(Yv.cpu().numpy(), R, T, f"linear tw={trans_w}")
    guards_untouched(bufs)


@pytest.mark.parametrize("which", ["f32", "bf16"])
def test_batched_far_items(bufs, which):
    """Three items 1.2e9 elements apart: the last one starts past 2^31 elements."""
    nb, m, n, k = 3, 130, 70, 72
    stride = 1_200_000_000
    dt = torch.float32 if which == "f32" else torch.bfloat16
    scale = 1 if which == "f32" else 2        # same byte stride for the 16-bit items
    A = wl.uniform((nb, m, k), 341).to(dt)
    B = wl.uniform((nb, k, n), 342).to(dt)
    C0 = wl.uniform((nb, m, n), 343)

    def place3(buf, host, st):
        flat = buf.view(host.dtype)
        assert (host.shape[0] - 1) * st + host[0].numel() <= flat.numel()
        v = flat.as_strided(host.shape, (st, host.shape[2], 1))
        v.copy_(host.to(DEV))
        return v

    Av = place3(bufs["A"], A, scale * stride)
    Bv = place3(bufs["B"], B, scale * stride)
    Cv = place3(bufs["C"], C0, stride)
    fn = ll.gemm_f32_batched if which == "f32" else ll.gemm_bf16f32_batched
    fn(Av, Bv, Cv, 1.5, -0.5)
    torch.cuda.synchronize()
    Ah = A.numpy() if which == "f32" else wl.half_bits(A)
    Bh = B.numpy() if which == "f32" else wl.half_bits(B)
    R, T = oracle.gemm_batched(Ah, Bh, 1.5, -0.5, C0.numpy(), bf16=which == "bf16")
    assert_close(Cv.cpu().numpy(), R, T, f"{which} batched far items")
    # the floats after each item's last row are untouched
    flat = bufs["C"].view(torch.float32)
    g = flat.as_strided((nb, 64), (stride, 1), m * n).cpu().view(torch.int32)
    assert torch.all(g == (NAN16 << 16 | NAN16)), "a write outside C"


def test_rows_near_int_max():
    """M = 2^31 - 1 (FP32, N = K = 4, 32 GB per operand): the last tile's row
    indices, the tile count and the launch grid sit at the 32-bit limits. A
    repeats a seeded 5-row integer pattern down its rows, so every output row
    equals the pattern row m % 5: the oracle computes those five rows (and a
    sample of rows at the end is compared with them), and the whole of C is
    checked for that period."""
    M, N, K = 2 ** 31 - 1, 4, 4
    assert ll.chosen_tile(F32, M, N, K, torch.cuda.get_device_properties(0).multi_processor_count) >= 0
    pat = wl.integers((5, K), 351, -2, 2)
    Bh = wl.integers((K, N), 352, -2, 2)
    q = -(-M // 5)
    Ad = pat.to(DEV).repeat(q, 1)[:M]          # row m is pat[m % 5]
    Cd = torch.full((M, N), float("nan"), device=DEV)
    ll.gemm_f32(Ad, Bh.to(DEV), Cd)
    torch.cuda.synchronize()
    R, _ = oracle.gemm(pat.numpy(), Bh.numpy())
    want = torch.from_numpy(R.astype(np.float32)).to(DEV)
    rows = np.concatenate([np.arange(5), np.arange(M - 300, M), np.random.default_rng(353).integers(0, M, 300)])
    got = Cd[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert np.array_equal(got, R.astype(np.float32)[rows % 5]), "sampled rows"
    chunk = 5 * (1 << 24)
    for s0 in range(0, M, chunk):
        c = Cd[s0:s0 + chunk]
        full = (c.shape[0] // 5) * 5
        assert torch.equal(c[:full].view(-1, 5, N), want.expand(full // 5, 5, N)), f"rows from {s0}"
        if full < c.shape[0]:
            assert torch.equal(c[full:], want[:c.shape[0] - full]), "tail rows"
    del Ad, Cd
    torch.cuda.empty_cache()
