"""Properties every plan of the tile / K-split / stream-K planner must have,
over random shapes (host logic only: the plan queries run without a GPU).

For any product the planner either returns a usable plan or none (-1, for
shapes whose tiles cannot fit one launch's grid); a usable plan names a tile
of the data type's table whose grid fits, splits K into at most 16 parts (64
for the skinny kernels) of at least one 64-deep stage (unless forced), shares out stream-K tiles only
for single products without a K-split, never shares out more tiles than the
product has, and honours forced settings.
"""
import pytest
from hypothesis import given, settings, strategies as st

import linear_layer_amd as ll

F32, F16 = ll.DTYPE_F32, ll.DTYPE_F16
TILE_SHAPES = {
    F32: [(256, 256), (256, 128), (128, 128), (64, 64), (64, 64), (128, 128), (16, 256), (32, 128)],
    F16: [(256, 256), (128, 128), (64, 64), (128, 128), (192, 192), (16, 256)],
}
dims = st.one_of(st.integers(1, 300), st.integers(1, 20000), st.sampled_from([255, 256, 257, 2047, 4096, 11008]))


def tiles_of(dt, t, M, N):
    bm, bn = TILE_SHAPES[dt][t]
    return -(-M // bm) * -(-N // bn)


@pytest.fixture(autouse=True)
def _automatic():
    yield
    for dt in (F32, F16):
        ll.set_tile(dt, -1)
    ll.set_split_k(-1)
    ll.set_stream_k(-1)


def test_table_shapes_match_names():
    for dt, shapes in TILE_SHAPES.items():
        assert ll.num_tiles(dt) == len(shapes)
        for t, (bm, bn) in enumerate(shapes):
            assert f"{bm}x{bn}" in ll.tile_name(dt, t)


@settings(max_examples=400, deadline=None)
@given(dt=st.sampled_from([F32, F16]), M=dims, N=dims, K=dims, batch=st.sampled_from([1, 1, 2, 7]),
       cus=st.sampled_from([0, 256, 304, 64]), relu=st.booleans(), nk=st.booleans())
def test_automatic_plans_are_well_formed(dt, M, N, K, batch, cus, relu, nk):
    q = dt | (ll.PLAN_RELU if relu and dt == F32 else 0) | (ll.PLAN_B_NK if nk else 0)
    t = ll.chosen_tile(q, M, N, K, cus, batch)
    s = ll.chosen_split_k(q, M, N, K, cus, batch)
    sk = ll.chosen_stream_k(q, M, N, K, cus, batch)
    assert 0 <= t < ll.num_tiles(dt)                 # these shapes always fit
    # the skinny kernels (a few rows of A) split K up to 64 ways, the others 16
    assert 1 <= s <= (64 if "_skinny" in ll.tile_name(dt, t) else 16)
    if s > 1:
        assert K >= 64 * (s - 1), "a split is at least one stage deep"
    assert sk >= 0
    if sk > 0:
        assert batch == 1 and s == 1
        assert sk <= tiles_of(dt, t, M, N)


@settings(max_examples=200, deadline=None)
@given(dt=st.sampled_from([F32, F16]), M=dims, N=dims, K=dims, data=st.data())
def test_forced_settings_are_honoured(dt, M, N, K, data):
    t = data.draw(st.integers(0, ll.num_tiles(dt) - 1))
    ll.set_tile(dt, t)
    assert ll.chosen_tile(dt, M, N, K, 256) == t
    s = data.draw(st.integers(1, 16))
    ll.set_split_k(s)
    got = ll.chosen_split_k(dt, M, N, K, 256)
    # the split length is ceil(K / s) rounded up to whole 64-deep stages, or
    # for a K-sliced tile to whole stages of every slice (KS x 32 FP32 or
    # KS x 64 16-bit values, if more), or for the 16-bit skinny tile to whole
    # 128-value loads, so the count may come out smaller
    name = ll.tile_name(dt, t)
    ks = 4 if name.endswith("_k4") else 2 if name.endswith("_k2") else 1
    align = max(64, ks * (64 if dt == F16 else 32))
    if dt == F16 and "_skinny" in name:
        align = 128
    k_split = -(-(-(-K // s)) // align) * align
    assert got == -(-K // k_split) and 1 <= got <= s
    assert ll.chosen_stream_k(dt, M, N, K, 256) == 0   # a forced split excludes stream-K
    ll.set_split_k(-1)
    ll.set_stream_k(0)
    assert ll.chosen_stream_k(dt, M, N, K, 256) == 0


@settings(max_examples=100, deadline=None)
@given(dt=st.sampled_from([F32, F16]), M=dims, N=dims, K=st.integers(128, 20000))
def test_forced_stream_k_shares_only_leftover_tiles(dt, M, N, K):
    ll.set_stream_k(1)
    t = ll.chosen_tile(dt, M, N, K, 256)
    sk = ll.chosen_stream_k(dt, M, N, K, 256)
    assert ll.chosen_split_k(dt, M, N, K, 256) == 1 or sk == 0
    if sk > 0:
        tiles = tiles_of(dt, t, M, N)
        slots = 256 * (1 if TILE_SHAPES[dt][t] == (256, 256) or (dt == F32 and t in (4, 5)) or
                       (dt == F16 and t == 3) else 2)
        assert sk == tiles % slots if tiles >= slots else sk == tiles


@settings(max_examples=300, deadline=None)
@given(dt=st.sampled_from([F32, F16]), M=dims, N=dims, K=dims, batch=st.sampled_from([1, 1, 3]),
       relu=st.booleans())
def test_unaligned_plans_cost_what_runs(dt, M, N, K, batch, relu):
    """Operands that rule out the 128-bit-load kernels: the planner picks
    neither stream-K nor a tile that exists only as a direct kernel (whose
    call would then run another shape's staged kernel)."""
    q = dt | ll.PLAN_UNALIGNED | (ll.PLAN_RELU if relu and dt == F32 else 0)
    t = ll.chosen_tile(q, M, N, K, 256, batch)
    assert 0 <= t < ll.num_tiles(dt)
    name = ll.tile_name(dt, t)
    assert not name.endswith(("_k2", "_k4")) and "192x192" not in name and name != "f32_32x128", name
    assert ll.chosen_stream_k(q, M, N, K, 256, batch) == 0


def test_unaligned_flag_changes_only_direct_only_choices():
    # 3072^2 16-bit takes the 192x192 direct tile when aligned, a staged one when not
    assert ll.tile_name(F16, ll.chosen_tile(F16, 3072, 3072, 3072, 256)) == "f16_192x192_direct"
    assert ll.tile_name(F16, ll.chosen_tile(F16 | ll.PLAN_UNALIGNED, 3072, 3072, 3072, 256)) != \
        "f16_192x192_direct"
    # 1024^3 FP32 takes four K-slices when aligned
    assert ll.tile_name(F32, ll.chosen_tile(F32, 1024, 1024, 1024, 256)) == "f32_64x64_k4"
    assert not ll.tile_name(F32, ll.chosen_tile(F32 | ll.PLAN_UNALIGNED, 1024, 1024, 1024,
                                                 256)).endswith("_k4")
    # 4096^3 is unaffected
    assert ll.chosen_tile(F32 | ll.PLAN_UNALIGNED, 4096, 4096, 4096, 256) == \
        ll.chosen_tile(F32, 4096, 4096, 4096, 256)


def test_skinny_kernel_choice():
    """Single FP32 products of at most 4 rows of A, or at most 8 with a large
    B, take the skinny kernel; its K-splits give about two workgroups per CU with B given
    K-by-N, three with B given N-by-K, keep each split within the A block the
    kernel stages whole (8192 / rows-per-pass k-values), and stay at most 64."""
    name = lambda q, M, N, K, batch=1: ll.tile_name(F32, ll.chosen_tile(q, M, N, K, 256, batch))
    split = lambda q, M, N, K: ll.chosen_split_k(q, M, N, K, 256)
    for M in (1, 2, 3, 4):
        for q in (F32, F32 | ll.PLAN_B_NK, F32 | ll.PLAN_RELU, F32 | ll.PLAN_UNALIGNED):
            assert name(q, M, 11008, 4096).endswith("_skinny")
    # 5 to 8 rows only with a B of at least 2^25 values
    for M in (5, 8):
        assert name(F32, M, 11008, 4096).endswith("_skinny")
        assert name(F32 | ll.PLAN_B_NK, M, 4096, 8192).endswith("_skinny")
        assert not name(F32, M, 4096, 4096).endswith("_skinny")
    assert not name(F32, 9, 11008, 4096).endswith("_skinny")
    assert not name(F32, 4, 11008, 4096, batch=2).endswith("_skinny")
    assert "_skinny" not in ll.tile_name(F16, ll.chosen_tile(F16, 1, 11008, 4096, 256))
    # 43 column blocks of 256: ceil(512 / 43) = 12 splits of 384 -> 11 splits;
    # N-by-K: ceil(768 / 43) = 18 splits of 256 -> 16 splits
    assert split(F32, 1, 11008, 4096) == 11
    assert split(F32 | ll.PLAN_B_NK, 1, 11008, 4096) == 16
    # 4 rows stage 2048 k-values: K = 20000 needs at least 10 splits even with
    # many column blocks
    assert split(F32, 4, 65536, 20000) >= 10
    # the split count never passes 64; a K no split can keep within the
    # staged block still gets 64 splits (the kernel then walks its range in
    # chunks)
    assert split(F32, 4, 256, 2 ** 20) == 64
    # short K: no split shorter than 64
    assert split(F32, 1, 256, 100) == 2 and split(F32, 1, 256, 64) == 1


def test_skinny16_kernel_choice():
    """Single 16-bit products of one row of A with B given N-by-K and at least
    2^25 values take the 16-bit skinny kernel, split K in ranges the kernel
    stages whole; B given K-by-N, more rows, smaller B or a batch do not."""
    nt = F16 | ll.PLAN_B_NK
    name = lambda q, M, N, K, batch=1: ll.tile_name(F16, ll.chosen_tile(q, M, N, K, 256, batch))
    for N, K in ((11008, 4096), (4096, 11008), (14336, 4096)):
        assert name(nt, 1, N, K) == "f16_16x256_skinny_nt"
        assert "_skinny" not in name(F16, 1, N, K)
        assert "_skinny" not in name(nt, 2, N, K)
        assert "_skinny" not in name(nt, 1, N, K, batch=2)
    assert "_skinny" not in name(nt, 1, 4096, 4096)
    # 43 column blocks of 256: ceil(768 / 43) = 18 splits of 228 -> 256 -> 16 splits
    assert ll.chosen_split_k(nt, 1, 11008, 4096, 256) == 16
    assert ll.chosen_stream_k(nt, 1, 11008, 4096, 256) == 0
