"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects bad arguments before touching the device, reports a
missing device as a status (never an abort), and picks tiles as documented."""
import ctypes
import os
import re

import pytest

import linear_layer_amd as ll

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("linear_layer.h", "linear_layer_tuning.h")]

# Fake, well-aligned, non-overlapping "device" addresses: these calls must
# fail validation (or find no device) before anything is dereferenced.
PA, PB, PC = 0x10000000, 0x20000000, 0x30000000


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        text = re.sub(r"^\s*#.*$", "", text, flags=re.M)   # preprocessor lines
        names |= set(re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{]*\)\s*;", text))
    return names


def test_library_exports_every_declared_symbol():
    lib = ll.load()
    declared = header_functions()
    assert declared == set(ll.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {ll.library_path()}").read()
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    assert declared <= exported


def test_status_strings():
    for s in range(5):
        assert ll.status_string(s).startswith(("LL_OK", "LL_ERR"))
    assert "unknown" in ll.status_string(99)


def call_gemm(M, N, K, alpha=1.0, A=PA, lda=None, B=PB, ldb=None, beta=0.0, C=PC, ldc=None, f16=False):
    lib = ll.load()
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    fn = lib.gemm_f16f32 if f16 else lib.gemm_f32
    return fn(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None)


@pytest.mark.parametrize("f16", [False, True])
def test_invalid_arguments(f16):
    E = ll.ERR_INVALID_VALUE
    assert call_gemm(-1, 4, 4, f16=f16) == E
    assert call_gemm(4, -1, 4, f16=f16) == E
    assert call_gemm(4, 4, -1, f16=f16) == E
    assert call_gemm(4, 4, 8, lda=7, f16=f16) == E          # lda < K
    assert call_gemm(4, 8, 4, ldb=7, f16=f16) == E          # ldb < N
    assert call_gemm(4, 8, 4, ldc=7, f16=f16) == E          # ldc < N
    assert call_gemm(4, 4, 4, A=None, f16=f16) == E
    assert call_gemm(4, 4, 4, B=None, f16=f16) == E
    assert call_gemm(4, 4, 4, C=None, f16=f16) == E
    assert call_gemm(4, 4, 4, C=PC + 2, f16=f16) == E       # C not 4-byte aligned
    assert call_gemm(4, 4, 4, A=PA + 1, f16=f16) == E       # A not element aligned
    # C overlapping A or B
    assert call_gemm(4, 4, 4, C=PA + 8, f16=f16) == E
    assert call_gemm(4, 4, 4, C=PB - 16, f16=f16) == E


@pytest.mark.parametrize("name", ["gemm_f32_nt", "gemm_f16f32_nt", "gemm_bf16f32_nt"])
def test_nt_leading_dimension_rule(name):
    """With B given N-by-K, ldb is bounded by K, not N."""
    fn = getattr(ll.load(), name)
    E = ll.ERR_INVALID_VALUE
    # M=4, N=16, K=8: ldb = 8 is fine for B^T (would be too small for a K-by-N B)
    ok = fn(4, 16, 8, 1.0, PA, 8, PB, 8, 0.0, PC, 16, None)
    assert ok in (ll.ERR_NO_DEVICE, ll.OK, ll.ERR_UNSUPPORTED_ARCH)
    assert fn(4, 16, 8, 1.0, PA, 8, PB, 7, 0.0, PC, 16, None) == E          # ldb < K
    assert fn(4, 16, 8, 1.0, PA, 8, PB, 8, 0.0, PC, 15, None) == E          # ldc < N
    assert fn(4, 16, 8, 1.0, PA, 8, PB, 8, 0.0, PB + 64, 16, None) == E   # C inside B
    assert fn(0, 16, 8, 1.0, None, 8, None, 8, 0.0, None, 16, None) == ll.OK


def test_linear_nt_leading_dimension_rule():
    lib = ll.load()
    E = ll.ERR_INVALID_VALUE
    ok = lib.linear_bias_act_nt(4, 16, 8, PA, 8, PB, 8, None, 1, PC, 16, None)
    assert ok in (ll.ERR_NO_DEVICE, ll.OK, ll.ERR_UNSUPPORTED_ARCH)
    assert lib.linear_bias_act_nt(4, 16, 8, PA, 8, PB, 7, None, 1, PC, 16, None) == E   # ldw < K
    assert lib.linear_bias_act_nt(4, 16, 8, PA, 8, PB, 8, None, 3, PC, 16, None) == E   # unknown act


def call_batched(M, N, K, sa, sb, sc, batch, trans_b=0, A=PA, B=PB, C=PC, lda=None, ldb=None,
                 ldc=None, name="gemm_f32_batched", alpha=1.0):
    lda = max(K, 1) if lda is None else lda
    ldb = max(K if trans_b else N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    fn = getattr(ll.load(), name)
    return fn(trans_b, M, N, K, alpha, A, lda, sa, B, ldb, sb, 0.0, C, ldc, sc, batch, None)


@pytest.mark.parametrize("name", ["gemm_f32_batched", "gemm_f16f32_batched", "gemm_bf16f32_batched"])
def test_batched_invalid_arguments(name):
    E = ll.ERR_INVALID_VALUE
    fine = (ll.ERR_NO_DEVICE, ll.OK, ll.ERR_UNSUPPORTED_ARCH)
    one = 8 * 8
    assert call_batched(8, 8, 8, one, one, one, 3, name=name) in fine
    assert call_batched(8, 8, 8, 0, 0, one, 3, name=name) in fine             # shared A and B
    assert call_batched(8, 8, 8, one, one, one, 3, trans_b=1, name=name) in fine
    assert call_batched(8, 8, 8, one, one, one, -1, name=name) == E           # negative batch
    assert call_batched(8, 8, 8, -one, one, one, 3, name=name) == E           # negative stride
    assert call_batched(8, 8, 8, one, one, one - 1, 3, name=name) == E        # C items overlap
    assert call_batched(8, 8, 8, one, one, 0, 2, name=name) == E              # one C for two items
    assert call_batched(8, 8, 8, one, one, one, 3, trans_b=2, name=name) == E
    # the last C item reaches B: C + 2*stride_c*4 bytes spans into [B, ...)
    assert call_batched(8, 8, 8, one, one, one, 3, C=PB - 2 * one * 4, name=name) == E
    # ... while the same C with one item stays clear of B
    assert call_batched(8, 8, 8, one, one, one, 1, C=PB - one * 4, name=name) in fine
    # strides whose span overflows 64 bits are rejected, not wrapped
    assert call_batched(8, 8, 8, 1 << 62, one, one, 3, name=name) == E
    # batch 0, like M = 0, is a no-op that touches nothing
    assert call_batched(8, 8, 8, one, one, one, 0, A=None, B=None, C=None, name=name) == ll.OK


def test_quick_returns_touch_nothing():
    # M == 0 or N == 0: OK with no device and even with NULL pointers
    assert call_gemm(0, 5, 5, A=None, B=None, C=None) == ll.OK
    assert call_gemm(5, 0, 5, A=None, B=None, C=None, f16=True) == ll.OK
    lib = ll.load()
    assert lib.linear_bias_act(0, 3, 3, None, 3, None, 3, None, 1, None, 3, None) == ll.OK


def test_linear_invalid_arguments():
    lib = ll.load()
    E = ll.ERR_INVALID_VALUE
    assert lib.linear_bias_act(4, 4, 4, PA, 4, PB, 4, None, 2, PC, 4, None) == E   # unknown act
    assert lib.linear_bias_act(4, 4, 4, PA, 4, PB, 4, None, -1, PC, 4, None) == E
    assert lib.linear_bias_act(4, 4, 4, PA, 3, PB, 4, None, 1, PC, 4, None) == E   # ldx < K
    assert lib.linear_bias_act(4, 4, 4, PA, 4, PB, 4, PC + 4, 1, PC, 4, None) == E  # bias inside Y
    assert lib.linear_bias_act(4, 4, 4, PA, 4, PB, 4, PB + 2, 1, PC, 4, None) == E  # bias misaligned
    assert lib.linear_bias_act(4, 4, 4, PA, 4, PB, 4, None, 1, PA, 4, None) == E    # Y overlaps X


def test_alpha_zero_does_not_need_a_or_b():
    # A, B are not read when alpha == 0 or K == 0, so NULL is accepted; with no
    # device present the call then reports the missing device.
    st = call_gemm(4, 4, 4, alpha=0.0, A=None, B=None, beta=1.0)
    assert st in (ll.ERR_NO_DEVICE, ll.OK, ll.ERR_UNSUPPORTED_ARCH)


def _has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device status on a host without a GPU")
def test_no_device_is_a_status_not_an_abort():
    assert call_gemm(64, 64, 64) == ll.ERR_NO_DEVICE
    assert call_gemm(64, 64, 64, f16=True) == ll.ERR_NO_DEVICE
    lib = ll.load()
    assert lib.linear_bias_act(4, 4, 4, PA, 4, PB, 4, None, 1, PC, 4, None) == ll.ERR_NO_DEVICE


def test_plans_at_int32_limits():
    """Tile counts are computed without overflow near 2^31, and a plan never has
    more workgroups than one launch can hold: an output whose tiles cannot fit
    gets no plan (-1), and the product call then returns LL_ERR_INVALID_VALUE."""
    f32, f16 = ll.DTYPE_F32, ll.DTYPE_F16
    big = 2 ** 31 - 1
    t = ll.chosen_tile(f32, big, 4, 4, 256)
    assert ll.tile_name(f32, t) == "f32_256x128"          # 8.4M tiles of 256 threads
    assert ll.chosen_tile(f16, big - 512, 1, 1, 256) == 1   # 128x128: 16.8M tiles
    # a single row of 2^31 - 1 columns: 8.4M skinny workgroups fit one launch;
    # 17 rows: 16.8M workgroups of the two-wave 32x128 tile; 33 rows are past
    # both, and no 64-row tile's grid fits
    assert ll.tile_name(f32, ll.chosen_tile(f32, 1, big, 1, 256)) == "f32_16x256_skinny"
    assert ll.tile_name(f32, ll.chosen_tile(f32, 17, big, 1, 256)) == "f32_32x128"
    for dt, shape in ((f32, (33, big, 1)), (f16, (big, 64, 64)), (f16, (1, big, 1))):
        assert ll.chosen_tile(dt, *shape, 256) == -1
        assert ll.chosen_split_k(dt, *shape, 256) == -1
        assert ll.chosen_stream_k(dt, *shape, 256) == -1
    # a deep K splits or streams without overflow
    assert ll.chosen_tile(f32, 1, 1, big, 256) >= 0 and ll.chosen_tile(f16, 1, 1, big, 256) >= 0


def test_tile_choice():
    f32, f16 = ll.DTYPE_F32, ll.DTYPE_F16
    names32 = [ll.tile_name(f32, t) for t in range(ll.num_tiles(f32))]
    names16 = [ll.tile_name(f16, t) for t in range(ll.num_tiles(f16))]
    assert names32[0] == "f32_256x256" and names16[0] == "f16_256x256_direct"
    assert ll.tile_name(f32, 99) == "" and ll.num_tiles(7) == 0

    def choice(dt, M, N, K, cus=256):
        names = names32 if dt == f32 else names16
        return names[ll.chosen_tile(dt, M, N, K, cus)], ll.chosen_split_k(dt, M, N, K, cus)

    # 4096^2 on 256 CUs: exactly one 256x256 tile per CU; no K-split
    assert choice(f32, 4096, 4096, 4096) == ("f32_256x256", 1)
    # 2047 x 11008: 344 tiles of 256x256 are 1.34 rounds; the full round runs
    # tile by tile and the 88 leftover tiles are shared out with stream-K
    assert choice(f32, 2047, 11008, 4096) == ("f32_256x256", 1)
    assert ll.chosen_stream_k(f32, 2047, 11008, 4096, 256) == 88
    assert ll.chosen_stream_k(f32, 4096, 4096, 4096, 256) == 0     # one whole round
    assert ll.chosen_stream_k(f16, 8192, 8192, 8192, 256) == 0     # four whole rounds
    ll.set_stream_k(0)
    try:
        assert choice(f32, 2047, 11008, 4096) == ("f32_256x128", 1)
        assert ll.chosen_stream_k(f32, 2047, 11008, 4096, 256) == 0
    finally:
        ll.set_stream_k(-1)
    with pytest.raises(ll.LinearLayerError):
        ll.set_stream_k(2)
    # the K-sliced tiles' rates depend on the K each slice walks: 64x64 in
    # four slices over the whole of K = 2048 or 4096 (its slices long enough),
    # but not split 16 ways over K = 1024 or 2048 (64 or 32 k-values per
    # slice), where the plain 64x64 tile runs the splits
    assert choice(f32, 512, 2048, 2048) == ("f32_64x64_k4", 1)
    assert choice(f32, 256, 4096, 4096) == ("f32_64x64_k4", 1)
    assert choice(f32, 1024, 64, 1024) == ("f32_64x64", 16)
    assert choice(f32, 512, 128, 2048) == ("f32_64x64", 16)
    assert choice(f32, 2048, 2048, 2048) == ("f32_128x128_k2", 1)
    assert choice(f32, 1024, 1024, 1024) == ("f32_64x64_k4", 1)
    assert choice(f16, 8192, 8192, 8192) == ("f16_256x256_direct", 1)
    # 16-bit: 6144^2 is 576 tiles of 256x256, 2.25 rounds: two run whole, 64
    # tiles are shared out; 3072^2 is 256 tiles of 192x192, one full round
    # (144 of 256x256 would leave 112 CUs idle), at any K; 5120^3 (400 tiles)
    # runs whole on 256x256 (729 tiles of 192x192 are three rounds); a K-split
    # is not worth its passes at the 16-bit rate; 2048^3 and the thin
    # 512x4096x4096 take 128x128 in two K-slices (one lone workgroup per CU
    # otherwise), 1024x8192x8192 plain 128x128 (two per CU), tiny products
    # plain 128x128 (too few stages per slice)
    assert choice(f16, 6144, 6144, 6144) == ("f16_256x256_direct", 1)
    assert ll.chosen_stream_k(f16, 6144, 6144, 6144, 256) == 64
    for K in (1024, 3072, 8192):
        assert choice(f16, 3072, 3072, K) == ("f16_192x192_direct", 1)
        assert ll.chosen_stream_k(f16, 3072, 3072, K, 256) == 0
    assert choice(f16, 5120, 5120, 5120) == ("f16_256x256_direct", 1)
    assert choice(f16, 4096, 4096, 4096) == ("f16_256x256_direct", 1)
    assert ll.chosen_stream_k(f16, 5120, 5120, 5120, 256) == 0
    assert choice(f16, 2048, 2048, 2048) == ("f16_128x128_k2", 1)
    assert choice(f16, 512, 4096, 4096) == ("f16_128x128_k2", 1)
    assert choice(f16, 1024, 8192, 8192) == ("f16_128x128x64", 1)
    assert choice(f16, 512, 512, 512) == ("f16_128x128x64", 1)
    # only the 256x256 16-bit tile takes a stream-K share, even when forced
    ll.set_stream_k(1)
    try:
        for t in (1, 2, 3):
            ll.set_tile(f16, t)
            assert ll.chosen_stream_k(f16, 2047, 11008, 4096, 256) == 0
        ll.set_tile(f16, 0)
        assert ll.chosen_stream_k(f16, 300, 264, 200, 256) > 0
    finally:
        ll.set_stream_k(-1)
        ll.set_tile(f16, -1)
    # problems too small to fill 256 CUs use small tiles split along K: in
    # the workgroup (K-slices), across workgroups, or both
    assert choice(f32, 1024, 1024, 1024) == ("f32_64x64_k4", 1)
    assert choice(f32, 2048, 2048, 2048) == ("f32_128x128_k2", 1)
    # below 8 stages per slice the slices cost more than they save
    assert choice(f32, 256, 256, 256) == ("f32_64x64", 1)   # one launch: launch-bound size
    assert choice(f32, 512, 512, 512) == ("f32_64x64", 4)
    # K-sliced tiles take no stream-K share
    ll.set_tile(f32, 4)
    ll.set_stream_k(1)
    try:
        assert ll.chosen_stream_k(f32, 2047, 11008, 4096, 256) == 0
    finally:
        ll.set_stream_k(-1)
        ll.set_tile(f32, -1)
    # short K is never split below 64 per split
    assert choice(f32, 512, 512, 64)[1] == 1
    assert choice(f32, 64, 64, 100)[1] <= 2
    # a device with fewer CUs moves the balance towards bigger tiles
    assert choice(f32, 4096, 4096, 4096, 64)[0] in names32
    ll.set_tile(f32, 2)
    try:
        assert ll.chosen_tile(f32, 4096, 4096, 4096, 256) == 2
    finally:
        ll.set_tile(f32, -1)
    ll.set_split_k(5)
    try:
        assert ll.chosen_split_k(f32, 4096, 4096, 4096, 256) == 5
        assert ll.chosen_split_k(f32, 64, 64, 100, 256) == 2   # 100 = 64 + 36
    finally:
        ll.set_split_k(-1)
    assert ll.chosen_tile(f32, 4096, 4096, 4096, 256) == 0
    # a batch counts all its items' tiles: 256 items of 256^3 fill the CUs
    # with 256x256 tiles, one item alone takes small tiles
    assert ll.chosen_tile(f32, 256, 256, 256, 256, batch=256) == 0
    assert ll.chosen_split_k(f32, 256, 256, 256, 256, batch=256) == 1
    assert ll.tile_name(f32, ll.chosen_tile(f32, 256, 256, 256, 256, batch=1)) == "f32_64x64"
    assert ll.chosen_tile(f32, 256, 256, 256, 256, batch=0) == -1
    with pytest.raises(ll.LinearLayerError):
        ll.set_tile(f32, 17)
    with pytest.raises(ll.LinearLayerError):
        ll.set_tile(5, 0)
    with pytest.raises(ll.LinearLayerError):
        ll.set_split_k(0)
    with pytest.raises(ll.LinearLayerError):
        ll.set_split_k(17)


def test_plan_query_flags():
    f32, f16 = ll.DTYPE_F32, ll.DTYPE_F16
    relu, nk = ll.PLAN_RELU, ll.PLAN_B_NK
    shape = (2047, 11008, 4096, 256)
    # the fused layer with ReLU still shares out the 88 leftover tiles
    assert ll.chosen_stream_k(f32 | relu, *shape) == 88
    # B given N-by-K plans alike
    assert ll.tile_name(f32, ll.chosen_tile(f32 | relu | nk, *shape)) == "f32_256x256"
    assert ll.chosen_stream_k(f32 | nk, *shape) == 88
    assert ll.chosen_stream_k(f32 | relu | nk, *shape) == 88
    ll.set_stream_k(0)
    try:
        assert ll.chosen_stream_k(f32 | nk, *shape) == 0
        assert ll.tile_name(f32, ll.chosen_tile(f32 | nk, *shape)) == "f32_256x128"
    finally:
        ll.set_stream_k(-1)
    # 256x128 tiles: 688 tiles on 512 slots, 176 shared out
    ll.set_tile(f32, 1)
    try:
        assert ll.chosen_stream_k(f32 | relu | nk, *shape) == 176
    finally:
        ll.set_tile(f32, -1)
    # 16-bit: the layout flag is accepted, the ReLU flag (no 16-bit layer) is not
    assert ll.chosen_tile(f16 | nk, 8192, 8192, 8192, 256) == 0
    assert ll.chosen_tile(f16 | relu, 8192, 8192, 8192, 256) == -1
    # an unknown flag is rejected (0x400 is LL_PLAN_UNALIGNED)
    assert ll.chosen_tile(f32 | 0x800, 8192, 8192, 8192, 256) == -1
    assert ll.chosen_split_k(f32 | 0x800, 64, 64, 64, 256) == -1
    assert ll.chosen_tile(f32 | ll.PLAN_UNALIGNED, 8192, 8192, 8192, 256) == 0


def test_binding_rejects_host_tensors():
    import torch
    A = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        ll.gemm_f32(A, A, A)
    with pytest.raises(TypeError):
        ll.gemm_f32(A.double(), A, A)


def test_extreme_sizes_stay_in_range():
    """Sizes at the 32-bit limits go through the argument checks and the plan
    queries without overflow (the sanitizer build runs this under UBSan)."""
    big = 2**31 - 1
    lib = ll.load()
    for f16 in (False, True):
        fn = lib.gemm_f16f32 if f16 else lib.gemm_f32
        elem = 2 if f16 else 4
        # K at the limit, one output element
        st = fn(1, 1, big, 1.0, PA, big, PA + big * elem + 64, 1, 0.0, PC + 2 * big * elem, 1, None)
        assert st in (ll.OK, ll.ERR_NO_DEVICE, ll.ERR_UNSUPPORTED_ARCH, ll.ERR_INVALID_VALUE)
        # leading dimensions at the limit
        st = fn(2, 2, 2, 1.0, PA, big, PB, big, 0.0, PC, big, None)
        assert st in (ll.ERR_NO_DEVICE, ll.ERR_UNSUPPORTED_ARCH, ll.ERR_INVALID_VALUE)
    for dt in (ll.DTYPE_F32, ll.DTYPE_F16):
        for M, N, K in [(1, 1, big), (big, 1, 1), (1, big, 1), (big, big, big), (big, 256, big)]:
            for flags in (0, ll.PLAN_UNALIGNED):
                t = ll.chosen_tile(dt | flags, M, N, K, 256)
                s = ll.chosen_split_k(dt | flags, M, N, K, 256)
                sk = ll.chosen_stream_k(dt | flags, M, N, K, 256)
                smax = 64 if t >= 0 and "_skinny" in ll.tile_name(dt, t) else 16
                assert t == -1 or (0 <= t < ll.num_tiles(dt) and 1 <= s <= smax and sk >= 0)


def test_linear_workspace_query():
    """Workspace of the fused layer's stream-K plan: 88 shared 256x256 tiles at
    2047 x 11008 x 4096 (one int counter each, rounded up to 256 bytes, then one
    FP32 tile each); none for plans without stream-K; -1 for bad arguments."""
    need = ll.linear_workspace_size(2047, 11008, 4096, False, 1, 256)
    assert need == 512 + 88 * 256 * 256 * 4
    assert ll.linear_workspace_size(2047, 11008, 4096, True, 1, 256) == need
    assert ll.linear_workspace_size(4096, 4096, 4096, False, 1, 256) == 0
    assert ll.linear_workspace_size(0, 11008, 4096) == 0
    lib = ll.load()
    assert lib.ll_linear_workspace_size(-1, 8, 8, 0, 1, 256) == -1
    assert lib.ll_linear_workspace_size(8, 8, 8, 2, 1, 256) == -1
    assert lib.ll_linear_workspace_size(8, 8, 8, 0, 5, 256) == -1


def test_linear_ws_argument_checks():
    lib = ll.load()
    E = ll.ERR_INVALID_VALUE
    args = (8, 8, 8, PA, 8, PB, 8)
    assert lib.linear_bias_act_ws(*args, 2, None, 1, PC, 8, 0x40000000, 4096, None) == E   # layout
    assert lib.linear_bias_act_ws(*args, 0, None, 1, PC, 8, 0x40000010, 4096, None) == E   # alignment
    assert lib.linear_bias_act_ws(*args, 0, None, 1, PC, 8, None, 64, None) == E           # NULL, bytes
    assert lib.linear_bias_act_ws(*args, 0, None, 1, PC, 8, PC, 4096, None) == E           # overlaps Y
    assert lib.linear_bias_act_ws(*args, 0, None, 1, PC, 8, PA, 4096, None) == E           # overlaps X
    st = lib.linear_bias_act_ws(*args, 0, None, 1, PC, 8, 0x40000000, 4096, None)
    assert st in (ll.ERR_NO_DEVICE, ll.ERR_UNSUPPORTED_ARCH, ll.OK)


def test_linear_noalloc_argument_checks():
    lib = ll.load()
    args = (8, 8, 8, PA, 8, PB, 8)
    assert lib.linear_bias_act_noalloc(*args, 2, None, 1, PC, 8, None) == ll.ERR_INVALID_VALUE
    st = lib.linear_bias_act_noalloc(*args, 0, None, 1, PC, 8, None)
    assert st in (ll.ERR_NO_DEVICE, ll.ERR_UNSUPPORTED_ARCH, ll.OK)


def test_noalloc_limit_matches_header():
    text = open(HEADERS[0]).read()
    m = re.search(r"#define\s+LL_NOALLOC_SCRATCH_BYTES\s+\((\d+)ll\s*<<\s*(\d+)\)", text)
    assert m, "LL_NOALLOC_SCRATCH_BYTES not found"
    assert ll.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
    # every fused-layer plan on 256 CUs fits the static workspace: a stream-K
    # plan shares out less than a round of tiles (at most 64 MiB of them)
    for M, N, K in ((2047, 11008, 4096), (4096, 11008, 4096), (4096, 14336, 4096),
                    (3000, 5000, 11008), (11008, 6000, 4096)):
        for wt in (False, True):
            assert ll.linear_workspace_size(M, N, K, wt, 1, 256) <= ll.NOALLOC_SCRATCH_BYTES
    lib = ll.load()
    E = ll.ERR_INVALID_VALUE
    assert lib.ll_set_noalloc_limit(-2) == E
    assert lib.ll_set_noalloc_limit(ll.NOALLOC_SCRATCH_BYTES + 1) == E
    assert lib.ll_set_noalloc_limit(0) == ll.OK
    assert lib.ll_set_noalloc_limit(-1) == ll.OK


def test_every_forced_stream_k_plan_fits_the_static_workspace():
    """Even with a tile and stream-K forced, no fused-layer plan on 256 CUs
    needs more than the no-allocation entry point's static array."""
    sizes = [64, 300, 1024, 2047, 3000, 4096, 5000, 8192, 11008, 16384]
    worst = 0
    try:
        for t in range(ll.num_tiles(ll.DTYPE_F32)):
            ll.set_tile(ll.DTYPE_F32, t)
            ll.set_stream_k(1)
            for M in sizes:
                for N in sizes:
                    for K in (512, 4096):
                        worst = max(worst, ll.linear_workspace_size(M, N, K, False, 1, 256))
    finally:
        ll.set_tile(ll.DTYPE_F32, -1)
        ll.set_stream_k(-1)
    assert 40 << 20 < worst <= ll.NOALLOC_SCRATCH_BYTES
