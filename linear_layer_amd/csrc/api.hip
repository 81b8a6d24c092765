// The C ABI: argument checks, quick returns, tile choice and one launch on the
// caller's stream. Nothing here allocates, synchronises or keeps per-call
// state; the only global data are a per-device property cache, the plan
// overrides of linear_layer_tuning.h, and the no-allocation entry point's
// static device workspace with its per-device address cache.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdint.h>
#include <string.h>

#include "linear_layer.h"
#include "linear_layer_tuning.h"
#include "launch.hpp"

using namespace ll;

namespace {

// ---- argument checks (host only, before any HIP call) ----

int64_t span_bytes(int rows, int cols, int64_t ld, int64_t elem)
{
    if (rows <= 0 || cols <= 0)
        return 0;
    return ((int64_t)(rows - 1) * ld + cols) * elem;
}

bool overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes)
{
    if (abytes <= 0 || bbytes <= 0)
        return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

int imax1(int v) { return v > 1 ? v : 1; }

// A strided batch: `count` products whose operands lie stride_{a,b,c}
// elements apart (a single product is {1, 0, 0, 0}).
struct Batch {
    int count;
    int64_t sa, sb, sc;
};
constexpr Batch kSingle{1, 0, 0, 0};

// Bytes from the first item's first element to the last item's last one;
// -1 on overflow.
int64_t batch_span(int count, int64_t stride, int64_t one, int64_t elem)
{
    int64_t step, reach, total;
    if (__builtin_mul_overflow(stride, elem, &step) ||
        __builtin_mul_overflow((int64_t)(count - 1), step, &reach) ||
        __builtin_add_overflow(reach, one, &total))
        return -1;
    return total;
}

// Returns LL_OK and sets *noop when nothing is to be done. b_trans: B is
// given N-by-K (ldb >= K) instead of K-by-N (ldb >= N). For a batch, the
// items of C must not overlap one another (stride_c covers one item), and the
// whole address range of C must not meet that of A or of B.
int check_gemm(int M, int N, int K, float alpha, const void *A, int lda, const void *B, int ldb,
               const float *C, int ldc, int64_t elem_ab, bool *noop, bool b_trans = false,
               const Batch &bt = kSingle)
{
    *noop = false;
    if (M < 0 || N < 0 || K < 0 || bt.count < 0 || bt.sa < 0 || bt.sb < 0 || bt.sc < 0)
        return LL_ERR_INVALID_VALUE;
    if (lda < imax1(K) || ldb < imax1(b_trans ? K : N) || ldc < imax1(N))
        return LL_ERR_INVALID_VALUE;
    if (M == 0 || N == 0 || bt.count == 0) {
        *noop = true;
        return LL_OK;
    }
    if (C == nullptr || !aligned(C, 4))
        return LL_ERR_INVALID_VALUE;
    const int64_t c_one = span_bytes(M, N, ldc, 4);
    if (bt.count > 1 && bt.sc * 4 < c_one)
        return LL_ERR_INVALID_VALUE;
    const int64_t cb = batch_span(bt.count, bt.sc, c_one, 4);
    if (cb < 0)
        return LL_ERR_INVALID_VALUE;
    const bool reads_ab = K > 0 && alpha != 0.0f;
    if (reads_ab) {
        if (A == nullptr || B == nullptr || !aligned(A, elem_ab) || !aligned(B, elem_ab))
            return LL_ERR_INVALID_VALUE;
        const int64_t ab = batch_span(bt.count, bt.sa, span_bytes(M, K, lda, elem_ab), elem_ab);
        const int64_t bb = batch_span(bt.count, bt.sb,
                                      b_trans ? span_bytes(N, K, ldb, elem_ab)
                                              : span_bytes(K, N, ldb, elem_ab), elem_ab);
        if (ab < 0 || bb < 0 || overlap(C, cb, A, ab) || overlap(C, cb, B, bb))
            return LL_ERR_INVALID_VALUE;
    }
    return LL_OK;
}

// ---- device check (cached per device) ----

struct DevInfo {
    int status;
    int cus;
};

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DevInfo g_dev_info[kMaxDevices];

DevInfo probe_device(int dev)
{
    DevInfo d{LL_ERR_NO_DEVICE, 0};
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return d;
    }
    d.cus = prop.multiProcessorCount;
    d.status = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? LL_OK : LL_ERR_UNSUPPORTED_ARCH;
    return d;
}

int current_device(DevInfo *out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return LL_ERR_NO_DEVICE;
    }
    if (dev >= kMaxDevices) {
        *out = probe_device(dev);
    } else {
        std::call_once(g_dev_once[dev], [dev] { g_dev_info[dev] = probe_device(dev); });
        *out = g_dev_info[dev];
    }
    return out->status;
}

// ---- tile and K-split choice ----

// Plan overrides for sweeps and tests (declared in linear_layer_tuning.h).
// They are process-wide: every later call on any thread or stream plans with
// them. The four values live in one atomic word, so a call reads one
// consistent set even while another thread changes them.
struct Overrides {
    int tile[2];   // forced tile, [0] fp32, [1] 16-bit (both formats); -1 automatic
    int splits;    // forced K-split count; -1 automatic
    int sk;        // stream-K: -1 automatic, 0 never, 1 whenever possible
};
// 8 bits per value, each stored as value + 1 (so -1 .. 254)
std::atomic<uint32_t> g_overrides{0u};

Overrides load_overrides()
{
    const uint32_t w = g_overrides.load(std::memory_order_relaxed);
    return Overrides{{(int)(w & 0xff) - 1, (int)((w >> 8) & 0xff) - 1}, (int)((w >> 16) & 0xff) - 1,
                     (int)((w >> 24) & 0xff) - 1};
}

// Set field `shift` (0 fp32 tile, 8 16-bit tile, 16 splits, 24 stream-K) to v.
void store_override(int shift, int v)
{
    uint32_t w = g_overrides.load(std::memory_order_relaxed), nw;
    do {
        nw = (w & ~(0xffu << shift)) | ((uint32_t)(v + 1) << shift);
    } while (!g_overrides.compare_exchange_weak(w, nw, std::memory_order_relaxed));
}

constexpr int kSplitAlign = 64;     // K per split is a multiple of every kernel's stage depth
constexpr int kMaxSplits = 16;

// Work units are multiply-adds on one CU at the 256x256 tile's throughput.
// FP32: at the matrix peak one CU does 157.3e12 / 2 / 256 = 307e3 of them per
// microsecond. 16-bit: the 256x256 kernel's measured rate on 8192^3 products,
// about 1250e12 / 2 / 256 = 2.4e6 (the matrix peak would be 4.9e6). Fixed
// costs (passes, atomic traffic) are converted to units at the same rate.
constexpr double kUnitsPerUs[2] = {307e3, 2.4e6};
// Effective rate (bytes per microsecond) of the atomic partial sums and
// passes of a K-split or stream-K plan. 16-bit: fitted to stream-K on
// 5120^3 and 6144^3, whose shared phases took 72-87 us beyond their MFMA
// work for 84-105 MB of atomic traffic; the FP32 kernels' longer tiles hide
// more of it.
constexpr double kAtomicBytesPerUs[2] = {3.0e6, 1.2e6};
// Fixed cost (us) of the extra launches a K-split or stream-K plan makes: the
// pass that prepares C (or Y) and, for ReLU, the pass after. Through the
// Python binding a 256^3 product measured 8.6 us per call as one launch and
// 10.3 us split four ways, so a pass is charged more than its GPU time.
constexpr double kPassUs = 5.0, kReluPassUs = 3.0;

// Estimated time of a launch with `wgs` workgroups of `work` units each: the
// dispatcher deals workgroups round-robin, so the busiest CU gets
// ceil(wgs/CUs). With one workgroup per CU they run one after another at
// eff_alone; with two they run in pairs at eff_paired (a pair takes twice a
// workgroup's work), and an odd last one runs alone.
// A tile of more than two workgroups per CU (the two-wave 32x128 tile) runs
// up to wg_per_cu of them side by side in rounds; a round of r takes as long
// as one workgroup alone (eff_alone: each is bound by its own latency) or as
// r at the CU's full rate (eff_paired), whichever is longer.
double wg_cost(const TileInfo &t, int64_t wgs, double work, int cus)
{
    const int64_t per_cu = (wgs + cus - 1) / cus;
    if (t.wg_per_cu > 2) {
        const int64_t full = per_cu / t.wg_per_cu, last = per_cu % t.wg_per_cu;
        const auto round = [&](int64_t r) {
            const double alone = work / t.eff_alone, shared = (double)r * work / t.eff_paired;
            return alone > shared ? alone : shared;
        };
        return (double)full * round(t.wg_per_cu) + (last > 0 ? round(last) : 0.0);
    }
    if (t.wg_per_cu <= 1 || per_cu == 1)
        return per_cu * work / t.eff_alone;
    const int64_t pairs = per_cu / 2, single = per_cu % 2;
    return pairs * 2.0 * work / t.eff_paired + single * work / t.eff_alone;
}

// The cost factor of a K-sliced tile (or of the 32x128 tile) at a K range of
// k values per workgroup, relative to its measured rate (eff_alone at
// k_ref): each of its KS slices walks k/KS values and its pipeline fill and
// drain cost about kFillK of them, so the rate scales as x / (x + kFillK)
// with x = k/KS, up to the tile's eff_max. Fitted to FP32 products of 128 to 512 rows on MI355X (e.g.
// 512 x 2048 x 2048: 37.8 us on 64x64 in four slices against 52.8 on 128x128
// in two slices split four ways, which K-independent rates ranked the other
// way round).
constexpr double kFillK = 128.0;
double k_factor(const TileInfo &t, double k)
{
    if (t.k_ref <= 0 || k <= 0.0)
        return 1.0;
    const double x = k / t.k_slices, r = (double)t.k_ref / t.k_slices;
    const double cap = t.eff_max > 0.0f ? t.eff_max : t.eff_alone;
    double rate = t.eff_alone * (x / (x + kFillK)) / (r / (r + kFillK));
    rate = rate < cap ? rate : cap;
    return t.eff_alone / rate;
}

struct Plan {
    int tile;
    int splits;
    int k_split;
    int dp_tiles;   // stream-K hybrid: tiles run whole (data-parallel); the rest are shared out
    int sk_grid;    // workgroups of the stream-K share; 0 when the plan has none
};

// Whether a plan may share tiles out with stream-K on tile shape `ti`: it
// needs a direct kernel (128-bit-aligned operands) and no K-slices.
bool sk_tile_ok(const TileInfo &ti)
{
    return ti.stream_k && ti.k_slices == 1;
}

// The skinny kernels (a few rows of A, memory-bound; `tile` is the FP32 or
// the 16-bit one): one workgroup per 256 columns and K-split. The K-splits
// give about two workgroups per CU (B given K-by-N) or three (N-by-K, whose
// waves stream fewer bytes at a time), as measured fastest on MI355X, and
// keep each split within the A block the kernel stages whole (kmax); at most
// kMaxSkinnySplits (the atomic partial sums of a few rows cost little), each
// a multiple of `align` long: kSplitAlign, or the k-values one load of the
// 16-bit kernel covers (128), so that no load of a split is partial.
constexpr int kMaxSkinnySplits = 64;
Plan skinny_plan(int tile, int kmax, int align, int M, int N, int K, int cus, int s_ov, bool bt)
{
    const int64_t nblk = cdiv(N, kSkinnyCols);
    if (nblk > max_grid_x(256) || nblk * kSkinnyCols > ((int64_t)1 << 31))
        return Plan{-1, 1, K, 0, 0};   // more workgroups than one launch holds
    int64_t s = s_ov;
    if (s_ov < 1) {
        const int64_t fill = ((bt ? 3 : 2) * (int64_t)(cus > 0 ? cus : 1) + nblk - 1) / nblk;
        const int64_t fit = ((int64_t)K + kmax - 1) / kmax;
        const int64_t smax = ((int64_t)K + align - 1) / align;
        s = fill > fit ? fill : fit;
        s = s > kMaxSkinnySplits ? kMaxSkinnySplits : s;
        s = s > smax ? smax : s;
    }
    if (s <= 1 || K <= 0)
        return Plan{tile, 1, K, 0, 0};
    const int k_split = (int)((((int64_t)K + s - 1) / s + align - 1) / align * align);
    return Plan{tile, (int)(((int64_t)K + k_split - 1) / k_split), k_split, 0, 0};
}

// Choose the tile shape and the number of K-splits minimising the estimate:
// big tiles for big problems; smaller ones, or several workgroups along K
// whose partial sums are added atomically into C, when big tiles would leave
// CUs idle (wave quantisation). This is the size-dependent choice of page
// "GEMM 优化详解", section "矩阵大小选择策略", re-derived for 256 CUs.
// A split costs a pre-pass over C (beta*C, or the bias), the atomic traffic of
// every split's partial tile and, for ReLU, a pass afterwards. `vec`: the
// operands allow the 128-bit-load kernels; without it the tiles that exist
// only as direct kernels (whose calls would run a staged kernel of another
// shape) and stream-K are not considered, unless a tile is forced.
Plan plan(int dtype, const TileInfo *tiles, int ntiles, int M, int N, int K, int cus, bool relu,
          int batch, bool vec, bool bt)
{
    const int items = batch < kMaxGridZ ? batch : kMaxGridZ;   // items per launch
    const Overrides ov = load_overrides();
    const int t_ov = ov.tile[dtype], s_ov = ov.splits, sk_ov = ov.sk;
    // single products of a few rows of A run a skinny kernel (FP32, or 16-bit
    // with B given N-by-K); it runs others only when forced
    const bool skinny = M <= kSkinnyMaxM || (M <= kSkinnyMaxMLarge && (int64_t)K * N >= kSkinnyLargeKN);
    if (dtype == LL_DTYPE_F32 && (t_ov == kSkinnyTile || (t_ov < 0 && skinny && batch == 1))) {
        const Plan sp = skinny_plan(kSkinnyTile, skinny_kmax(M), kSplitAlign, M, N, K, cus, s_ov, bt);
        if (sp.tile >= 0 || t_ov == kSkinnyTile)
            return sp;
    }
    const bool skinny16 = M <= kSkinny16MaxM && (int64_t)K * N >= kSkinnyLargeKN && bt;
    if (dtype != LL_DTYPE_F32 && (t_ov == kSkinny16Tile || (t_ov < 0 && skinny16 && batch == 1))) {
        const Plan sp = skinny_plan(kSkinny16Tile, skinny16_kmax(M), kSkinny16Align, M, N, K, cus, s_ov, bt);
        if (sp.tile >= 0 || t_ov == kSkinny16Tile)
            return sp;
    }
    const bool allow_sk = vec && batch == 1 && s_ov < 1 && sk_ov != 0 && K > 0;
    Plan best{0, 1, K, 0, 0}, best_sk{0, 1, K, 0, 0};
    double best_cost = 0.0, best_sk_cost = 0.0;
    bool have = false, have_sk = false;
    for (int t = 0; t < ntiles; ++t) {
        if ((t_ov >= 0 && t != t_ov) || (dtype == LL_DTYPE_F32 ? t == kSkinnyTile : t == kSkinny16Tile))
            continue;
        if (dtype == LL_DTYPE_F32 && t == kThinTile && M > tiles[t].bm && t_ov != t)
            continue;   // a second row of 32x128 tiles reads B again
        const TileInfo &ti = tiles[t];
        const int64_t tiles_mn = (int64_t)cdiv(M, ti.bm) * cdiv(N, ti.bn);
        if (tiles_mn > max_grid_x(ti.threads))
            continue;   // more workgroups than one launch can hold
        if ((int64_t)cdiv(M, ti.bm) * ti.bm > (int64_t)1 << 31 ||
            (int64_t)cdiv(N, ti.bn) * ti.bn > (int64_t)1 << 31)
            continue;   // a row or column index inside the last tile would pass 2^31 - 1
        if (K < ti.min_k && t_ov != t)
            continue;   // K too short for the tile's K-slices (unless forced)
        if (!vec && ti.direct_only && t_ov != t)
            continue;   // unaligned operands would run another tile's staged kernel
        // K per split: whole stages of every K-slice (KS slices of BK = 32
        // FP32 or 64 16-bit values), so that the launch can take the
        // unchecked kernel when K allows it (a 64x64 tile in four slices split
        // 4 ways over K = 11008: 74 us in 2752-long splits, 57 us in 2816)
        const int kslice = ti.k_slices * (dtype == LL_DTYPE_F16 ? 64 : 32);
        const int align = kslice > kSplitAlign ? kslice : kSplitAlign;
        for (int s = 1; s <= kMaxSplits; ++s) {
            if (s_ov >= 1 && s != s_ov)
                continue;
            if (s_ov < 1 && s > 1 && (int64_t)K < (int64_t)s * align)
                break;
            int k_split = K;
            int splits = 1;
            if (s > 1) {
                k_split = (int)((((int64_t)K + s - 1) / s + align - 1) / align * align);
                splits = (int)(((int64_t)K + k_split - 1) / k_split);
                if (splits != s && s_ov < 1)
                    continue;   // the same partition is reached with fewer splits
                if (dtype == LL_DTYPE_F32 && t == kThinTile && k_split < kThinMinSplit && s_ov < 1)
                    break;      // 32x128 splits shorter than this measured slower than 64x64
            }
            double cost = wg_cost(ti, tiles_mn * splits * items,
                                  (double)ti.bm * ti.bn * k_split * k_factor(ti, k_split), cus);
            if (splits > 1) {
                const double mn = (double)M * N * items;
                const double bytes = 8.0 * mn * (relu ? 2 : 1) + 4.0 * mn * splits;
                cost += ((relu ? kPassUs + kReluPassUs : kPassUs) + bytes / kAtomicBytesPerUs[dtype]) *
                        kUnitsPerUs[dtype];
            }
            if (!have || cost < best_cost) {
                best = Plan{t, splits, k_split, 0, 0};
                best_cost = cost;
                have = true;
            }
        }
        // Stream-K hybrid: the full rounds of tiles run whole; the leftover
        // tiles' k-units are shared out evenly over one round of workgroups,
        // which add their partial sums atomically (framed by a pass that
        // prepares those tiles and, for ReLU, one that finishes them).
        if (allow_sk && sk_tile_ok(ti)) {
            const int64_t slots = (int64_t)cus * ti.wg_per_cu;
            const int64_t rounds = tiles_mn / slots, rest = tiles_mn - rounds * slots;
            const int64_t units = ((int64_t)K + kSkUnit - 1) / kSkUnit;
            if (rest > 0 && units >= 2 && tiles_mn + slots <= max_grid_x(ti.threads)) {
                const int64_t grid = rest * units < slots ? rest * units : slots;
                const int64_t per_wg = (rest * units + grid - 1) / grid;
                const double work = (double)ti.bm * ti.bn * K;
                double cost = rounds > 0 ? wg_cost(ti, rounds * slots, work * k_factor(ti, K), cus) : 0.0;
                cost += wg_cost(ti, grid, work * (double)per_wg / (double)units *
                                              k_factor(ti, (double)per_wg * kSkUnit), cus);
                // atomics: one partial tile per segment (at most grid + rest of
                // them); passes: the prepare write and, for ReLU, a read and write
                const double area = 4.0 * ti.bm * ti.bn;
                const double bytes = area * (double)(grid + rest) + area * rest * (relu ? 3 : 1);
                cost += ((relu ? kPassUs + kReluPassUs : kPassUs) + bytes / kAtomicBytesPerUs[dtype]) *
                        kUnitsPerUs[dtype];
                if (!have_sk || cost < best_sk_cost) {
                    best_sk = Plan{t, 1, K, (int)(rounds * slots), (int)grid};
                    best_sk_cost = cost;
                    have_sk = true;
                }
            }
        }
    }
    // stream-K forced: its best plan whenever the shape allows one
    if (have_sk && (sk_ov == 1 || !have || best_sk_cost < best_cost))
        best = best_sk;
    else if (!have)
        best.tile = -1;   // no tile's grid fits one launch (or the forced one does not)
    if (best.k_split <= 0)
        best.k_split = 1;
    return best;
}

int launch_status(hipError_t e) { return e == hipSuccess ? LL_OK : LL_ERR_LAUNCH; }

// Stream-K workspace of a plan sharing out `rest` tiles of ti: one int counter
// per shared tile (the block rounded up to 256 bytes), then one FP32 tile each.
int64_t sk_counter_bytes(int64_t rest) { return (4 * rest + 255) / 256 * 256; }
int64_t sk_workspace_bytes(int64_t rest, const TileInfo &ti)
{
    return rest > 0 ? sk_counter_bytes(rest) + rest * ti.bm * ti.bn * 4 : 0;
}

GemmParams make_params(int M, int N, int K, float alpha, const void *A, int lda, const void *B,
                       int ldb, float beta, float *C, int ldc)
{
    GemmParams p;
    memset(&p, 0, sizeof p);
    p.A = A;
    p.B = B;
    p.C = C;
    p.bias = nullptr;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.M = M;
    p.N = N;
    p.K = K;
    p.alpha = alpha;
    p.beta = beta;
    p.act = 0;
    p.group_m = 4;
    p.k_split = K > 0 ? K : 1;
    p.batch = 1;
    return p;
}

typedef hipError_t (*launch_fn)(const GemmParams &, int, int, bool, hipStream_t);

// One GEMM per plan: a single launch with the alpha/beta write-back, or, when
// K is split, C = beta*C followed by the split launch adding alpha*partials.
hipError_t run_one(GemmParams p, const Plan &pl, bool vec, hipStream_t s, launch_fn launch)
{
    if (pl.splits == 1)
        return launch(p, pl.tile, p.beta == 0.0f ? EPI_GEMM_BETA0 : EPI_GEMM_BETA, vec, s);
    if (p.beta != 1.0f) {
        const hipError_t e = launch_scale(p.C, p.ldc, p.M, p.N, p.beta, s, p.batch, p.stride_c);
        if (e != hipSuccess)
            return e;
    }
    p.k_split = pl.k_split;
    return launch(p, pl.tile, EPI_ATOMIC, vec, s);
}

// Tile grid of a plan's tile shape, for the per-tile passes.
GemmParams with_tile_grid(GemmParams p, const TileInfo &ti)
{
    p.tiles_m = cdiv(p.M, ti.bm);
    p.tiles_n = cdiv(p.N, ti.bn);
    return p;
}

// A stream-K hybrid plan: prepare the shared-out tiles (pre_pass), then one
// launch whose first dp_tiles workgroups run whole tiles with `epi` and whose
// sk_grid others share out the rest (they start as whole tiles finish), then
// (ReLU) finish the shared-out tiles.
hipError_t run_stream_k(GemmParams p, const Plan &pl, const TileInfo &ti, int epi, int pre_pass,
                        bool relu_after, bool vec, hipStream_t s, launch_fn launch,
                        void *ws = nullptr)
{
    const GemmParams g = with_tile_grid(p, ti);
    const int64_t tiles_mn = (int64_t)g.tiles_m * g.tiles_n;
    const int rest = (int)(tiles_mn - pl.dp_tiles);
    GemmParams q = p;
    q.grid_x = pl.dp_tiles + pl.sk_grid;
    q.sk_block = pl.dp_tiles;
    q.sk_tiles = rest;
    if (ws != nullptr) {
        // one launch: the sharing workgroups add into the workspace tiles and
        // the last contributor of each tile writes it, epilogue fused
        q.ws_cnt = static_cast<int *>(ws);
        q.ws = reinterpret_cast<float *>(static_cast<char *>(ws) + sk_counter_bytes(rest));
        return launch(q, pl.tile, epi, vec, s);
    }
    hipError_t e = hipSuccess;
    if (pre_pass >= 0)
        e = launch_tile_pass(g, ti.bm, ti.bn, pl.dp_tiles, rest, pre_pass, s);
    if (e == hipSuccess)
        e = launch(q, pl.tile, epi, vec, s);
    if (e == hipSuccess && relu_after)
        e = launch_tile_pass(g, ti.bm, ti.bn, pl.dp_tiles, rest, TILE_RELU, s);
    return e;
}

// A strided batch in launches of at most kMaxGridZ items (grid z).
hipError_t run_gemm(GemmParams p, const Plan &pl, bool vec, hipStream_t s, launch_fn launch,
                    int64_t elem_ab, const Batch &bt = kSingle, const TileInfo *ti = nullptr)
{
    if (pl.sk_grid > 0)   // single products only (the planner offers it for batch 1)
        return run_stream_k(p, pl, *ti, p.beta == 0.0f ? EPI_GEMM_BETA0 : EPI_GEMM_BETA,
                            p.beta == 1.0f ? -1 : TILE_SCALE, false, vec, s, launch);
    p.stride_a = bt.sa * elem_ab;
    p.stride_b = bt.sb * elem_ab;
    p.stride_c = bt.sc * 4;
    for (int64_t done = 0; done < bt.count; done += kMaxGridZ) {
        GemmParams q = p;
        q.batch = (int)(bt.count - done < kMaxGridZ ? bt.count - done : kMaxGridZ);
        q.A = static_cast<const char *>(p.A) + done * p.stride_a;
        q.B = static_cast<const char *>(p.B) + done * p.stride_b;
        q.C = reinterpret_cast<float *>(reinterpret_cast<char *>(p.C) + done * p.stride_c);
        const hipError_t e = run_one(q, pl, vec, s, launch);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// C = beta*C for every item of a batch (K == 0 or alpha == 0).
hipError_t scale_batch(float *C, int ldc, int M, int N, float beta, hipStream_t s, const Batch &bt)
{
    for (int64_t done = 0; done < bt.count; done += kMaxGridZ) {
        const int n = (int)(bt.count - done < kMaxGridZ ? bt.count - done : kMaxGridZ);
        const hipError_t e = launch_scale(C + done * bt.sc, ldc, M, N, beta, s, n, bt.sc * 4);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// 16-byte operand loads need every item's base 16-byte aligned.
bool batch_aligned(const Batch &bt, int64_t elem_ab)
{
    return bt.count <= 1 || ((bt.sa * elem_ab) % 16 == 0 && (bt.sb * elem_ab) % 16 == 0 &&
                             (bt.sc * 4) % 16 == 0);
}

}  // namespace

extern "C" {

static int gemm_f32_impl(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                         int ldb, float beta, float *C, int ldc, void *stream, bool bt,
                         const Batch &bat = kSingle)
{
    bool noop;
    int st = check_gemm(M, N, K, alpha, A, lda, B, ldb, C, ldc, 4, &noop, bt, bat);
    if (st != LL_OK || noop)
        return st;
    DevInfo dev;
    if ((st = current_device(&dev)) != LL_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0 || alpha == 0.0f)
        return launch_status(scale_batch(C, ldc, M, N, beta, s, bat));
    const bool vec = aligned(A, 16) && aligned(B, 16) && aligned(C, 16) && lda % 4 == 0 &&
                     ldb % 4 == 0 && ldc % 4 == 0 && K % 4 == 0 && (bt || N % 4 == 0) &&
                     batch_aligned(bat, 4);
    GemmParams p = make_params(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    const Plan pl =
        plan(0, kF32Tiles, kF32NumTiles, M, N, K, dev.cus, false, bat.count, vec, bt);
    if (pl.tile < 0)
        return LL_ERR_INVALID_VALUE;
    return launch_status(run_gemm(p, pl, vec, s, bt ? launch_gemm_f32_bt : launch_gemm_f32, 4, bat,
                                  &kF32Tiles[pl.tile]));
}

int gemm_f32(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, void *stream)
{
    return gemm_f32_impl(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, false);
}

int gemm_f32_nt(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
                float beta, float *C, int ldc, void *stream)
{
    return gemm_f32_impl(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, true);
}

// Both 16-bit formats and both B layouts share the kernels, tiles and checks.
static int gemm_16(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B,
                   int ldb, float beta, float *C, int ldc, void *stream, launch_fn launch, bool bt,
                   const Batch &bat = kSingle)
{
    bool noop;
    int st = check_gemm(M, N, K, alpha, A, lda, B, ldb, C, ldc, 2, &noop, bt, bat);
    if (st != LL_OK || noop)
        return st;
    DevInfo dev;
    if ((st = current_device(&dev)) != LL_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0 || alpha == 0.0f)
        return launch_status(scale_batch(C, ldc, M, N, beta, s, bat));
    const bool vec = aligned(A, 16) && aligned(B, 16) && aligned(C, 16) && lda % 8 == 0 &&
                     ldb % 8 == 0 && ldc % 4 == 0 && K % 8 == 0 && (bt || N % 8 == 0) &&
                     batch_aligned(bat, 2);
    GemmParams p = make_params(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    const Plan pl = plan(1, kF16Tiles, kF16NumTiles, M, N, K, dev.cus, false, bat.count, vec, bt);
    if (pl.tile < 0)
        return LL_ERR_INVALID_VALUE;
    return launch_status(run_gemm(p, pl, vec, s, launch, 2, bat, &kF16Tiles[pl.tile]));
}

int gemm_f16f32(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B,
                int ldb, float beta, float *C, int ldc, void *stream)
{
    return gemm_16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, launch_gemm_f16, false);
}

int gemm_bf16f32(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B,
                 int ldb, float beta, float *C, int ldc, void *stream)
{
    return gemm_16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, launch_gemm_bf16, false);
}

int gemm_f16f32_nt(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B,
                   int ldb, float beta, float *C, int ldc, void *stream)
{
    return gemm_16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, launch_gemm_f16_bt, true);
}

int gemm_bf16f32_nt(int M, int N, int K, float alpha, const uint16_t *A, int lda, const uint16_t *B,
                    int ldb, float beta, float *C, int ldc, void *stream)
{
    return gemm_16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, launch_gemm_bf16_bt, true);
}

int gemm_f32_batched(int trans_b, int M, int N, int K, float alpha, const float *A, int lda,
                     int64_t stride_a, const float *B, int ldb, int64_t stride_b, float beta, float *C,
                     int ldc, int64_t stride_c, int batch, void *stream)
{
    if (trans_b != 0 && trans_b != 1)
        return LL_ERR_INVALID_VALUE;
    return gemm_f32_impl(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, trans_b == 1,
                         Batch{batch, stride_a, stride_b, stride_c});
}

int gemm_f16f32_batched(int trans_b, int M, int N, int K, float alpha, const uint16_t *A, int lda,
                        int64_t stride_a, const uint16_t *B, int ldb, int64_t stride_b, float beta,
                        float *C, int ldc, int64_t stride_c, int batch, void *stream)
{
    if (trans_b != 0 && trans_b != 1)
        return LL_ERR_INVALID_VALUE;
    return gemm_16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                   trans_b ? launch_gemm_f16_bt : launch_gemm_f16, trans_b == 1,
                   Batch{batch, stride_a, stride_b, stride_c});
}

int gemm_bf16f32_batched(int trans_b, int M, int N, int K, float alpha, const uint16_t *A, int lda,
                         int64_t stride_a, const uint16_t *B, int ldb, int64_t stride_b, float beta,
                         float *C, int ldc, int64_t stride_c, int batch, void *stream)
{
    if (trans_b != 0 && trans_b != 1)
        return LL_ERR_INVALID_VALUE;
    return gemm_16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                   trans_b ? launch_gemm_bf16_bt : launch_gemm_bf16, trans_b == 1,
                   Batch{batch, stride_a, stride_b, stride_c});
}

// The workspace a fused-layer call would use (0: its plan needs none).
static int64_t linear_ws_need(const Plan &pl, int M, int N)
{
    if (pl.tile < 0 || pl.sk_grid <= 0)
        return 0;
    const TileInfo &ti = kF32Tiles[pl.tile];
    const int64_t rest = (int64_t)cdiv(M, ti.bm) * cdiv(N, ti.bn) - pl.dp_tiles;
    return sk_workspace_bytes(rest, ti);
}

// ws_strict: a plan needing more workspace than ws_bytes is an error (the
// no-allocation entry point), not a reason to run the plan without one.
static int linear_impl(int M, int N, int K, const float *X, int ldx, const float *W, int ldw,
                       const float *bias, int act, float *Y, int ldy, void *stream, bool wt,
                       void *ws = nullptr, int64_t ws_bytes = 0, bool ws_strict = false)
{
    if (act != LL_ACT_NONE && act != LL_ACT_RELU)
        return LL_ERR_INVALID_VALUE;
    bool noop;
    int st = check_gemm(M, N, K, 1.0f, X, ldx, W, ldw, Y, ldy, 4, &noop, wt);
    if (st != LL_OK || noop)
        return st;
    if (bias != nullptr) {
        if (!aligned(bias, 4) || overlap(Y, span_bytes(M, N, ldy, 4), bias, (int64_t)N * 4))
            return LL_ERR_INVALID_VALUE;
    }
    DevInfo dev;
    if ((st = current_device(&dev)) != LL_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0)
        return launch_status(launch_bias_fill(Y, ldy, M, N, bias, act, s));
    const bool vec = aligned(X, 16) && aligned(W, 16) && aligned(Y, 16) && ldx % 4 == 0 &&
                     ldw % 4 == 0 && ldy % 4 == 0 && K % 4 == 0 && (wt || N % 4 == 0);
    GemmParams p = make_params(M, N, K, 1.0f, X, ldx, W, ldw, 0.0f, Y, ldy);
    p.bias = bias;
    p.act = act;
    const launch_fn launch = wt ? launch_gemm_f32_bt : launch_gemm_f32;
    const Plan pl = plan(0, kF32Tiles, kF32NumTiles, M, N, K, dev.cus, act == LL_ACT_RELU, 1, vec, wt);
    if (pl.tile < 0)
        return LL_ERR_INVALID_VALUE;
    if (pl.sk_grid > 0) {
        // with a large enough workspace, one launch with the epilogue fused
        // into every tile; without, the bias pass, the launch and a ReLU pass
        const int64_t need = linear_ws_need(pl, M, N);
        if (ws_strict && need > ws_bytes)
            return LL_ERR_INVALID_VALUE;
        void *use = ws != nullptr && ws_bytes >= need ? ws : nullptr;
        return launch_status(run_stream_k(p, pl, kF32Tiles[pl.tile], EPI_LINEAR, TILE_BIAS,
                                          act == LL_ACT_RELU, vec, s, launch, use));
    }
    if (pl.splits == 1)
        return launch_status(launch(p, pl.tile, EPI_LINEAR, vec, s));
    // split-K: Y = bias, then every split adds its partial product, then ReLU
    hipError_t e = launch_bias_fill(Y, ldy, M, N, bias, LL_ACT_NONE, s);
    if (e == hipSuccess) {
        p.k_split = pl.k_split;
        e = launch(p, pl.tile, EPI_ATOMIC, vec, s);
    }
    if (e == hipSuccess && act == LL_ACT_RELU)
        e = launch_relu(Y, ldy, M, N, s);
    return launch_status(e);
}

int linear_bias_act(int M, int N, int K, const float *X, int ldx, const float *W, int ldw,
                    const float *bias, int act, float *Y, int ldy, void *stream)
{
    return linear_impl(M, N, K, X, ldx, W, ldw, bias, act, Y, ldy, stream, false);
}

int linear_bias_act_nt(int M, int N, int K, const float *X, int ldx, const float *W, int ldw,
                       const float *bias, int act, float *Y, int ldy, void *stream)
{
    return linear_impl(M, N, K, X, ldx, W, ldw, bias, act, Y, ldy, stream, true);
}

int linear_bias_act_ws(int M, int N, int K, const float *X, int ldx, const float *W, int ldw,
                       int w_layout, const float *bias, int act, float *Y, int ldy, void *workspace,
                       int64_t workspace_bytes, void *stream)
{
    if ((w_layout != LL_W_K_BY_N && w_layout != LL_W_N_BY_K) || workspace_bytes < 0 ||
        (workspace == nullptr && workspace_bytes != 0) || !aligned(workspace, 256))
        return LL_ERR_INVALID_VALUE;
    const bool wt = w_layout == LL_W_N_BY_K;
    if (workspace != nullptr && workspace_bytes > 0 && M > 0 && N > 0) {
        // the workspace may not overlap the operands or the output
        const int64_t xb = span_bytes(M, K, ldx, 4);
        const int64_t wb = wt ? span_bytes(N, K, ldw, 4) : span_bytes(K, N, ldw, 4);
        if (overlap(workspace, workspace_bytes, X, xb) || overlap(workspace, workspace_bytes, W, wb) ||
            overlap(workspace, workspace_bytes, Y, span_bytes(M, N, ldy, 4)) ||
            (bias != nullptr && overlap(workspace, workspace_bytes, bias, (int64_t)N * 4)))
            return LL_ERR_INVALID_VALUE;
    }
    return linear_impl(M, N, K, X, ldx, W, ldw, bias, act, Y, ldy, stream, wt, workspace,
                       workspace_bytes);
}

// ---- the no-allocation entry point ----
//
// linear_bias_act_noalloc runs linear_bias_act_ws on a workspace the library
// owns: `scratch`, a static device array (one copy per GPU, held until the
// process ends), zero-filled when the code object loads and left zero-filled
// by every call. Host code reaches it only through the device address
// hipGetSymbolAddress returns for the current device, looked up once per
// device; the array's own name is a host-side stand-in, never an address.
static __device__ __align__(256) unsigned char scratch[LL_NOALLOC_SCRATCH_BYTES];

static std::once_flag g_scratch_once[kMaxDevices];
static void *g_scratch_ptr[kMaxDevices];
// the part of `scratch` calls may use (ll_set_noalloc_limit; process-wide)
static std::atomic<int64_t> g_noalloc_limit{LL_NOALLOC_SCRATCH_BYTES};

// The current device's copy of `scratch`, or nullptr.
static void *scratch_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            ptr = nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    });
    return g_scratch_ptr[dev];
}

int linear_bias_act_noalloc(int M, int N, int K, const float *X, int ldx, const float *W, int ldw,
                            int w_layout, const float *bias, int act, float *Y, int ldy,
                            void *stream)
{
    if (w_layout != LL_W_K_BY_N && w_layout != LL_W_N_BY_K)
        return LL_ERR_INVALID_VALUE;
    DevInfo dev;
    int st = current_device(&dev);
    if (st != LL_OK)
        return st;
    if (stream != nullptr) {
        // the array used is the current device's: the kernels must run there
        int sdev = -1, cur = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess ||
            hipGetDevice(&cur) != hipSuccess) {
            (void)hipGetLastError();
            return LL_ERR_INVALID_VALUE;
        }
        if (sdev != cur)
            return LL_ERR_INVALID_VALUE;
    }
    void *ws = scratch_address();
    if (ws == nullptr)
        return LL_ERR_LAUNCH;
    return linear_impl(M, N, K, X, ldx, W, ldw, bias, act, Y, ldy, stream, w_layout == LL_W_N_BY_K,
                       ws, g_noalloc_limit.load(std::memory_order_relaxed), true);
}

int ll_set_noalloc_limit(int64_t bytes)
{
    if (bytes != -1 && (bytes < 0 || bytes > LL_NOALLOC_SCRATCH_BYTES))
        return LL_ERR_INVALID_VALUE;
    g_noalloc_limit.store(bytes == -1 ? LL_NOALLOC_SCRATCH_BYTES : bytes, std::memory_order_relaxed);
    return LL_OK;
}

int64_t ll_linear_workspace_size(int M, int N, int K, int w_layout, int act, int num_cus)
{
    if ((w_layout != LL_W_K_BY_N && w_layout != LL_W_N_BY_K) || M < 0 || N < 0 || K < 0 ||
        (act != LL_ACT_NONE && act != LL_ACT_RELU))
        return -1;
    if (M == 0 || N == 0 || K == 0)
        return 0;
    const Plan pl = plan(0, kF32Tiles, kF32NumTiles, M, N, K, num_cus > 0 ? num_cus : 256,
                         act == LL_ACT_RELU, 1, true, w_layout == LL_W_N_BY_K);
    return linear_ws_need(pl, M, N);
}

const char *ll_status_string(int status)
{
    switch (status) {
    case LL_OK: return "LL_OK: success";
    case LL_ERR_INVALID_VALUE: return "LL_ERR_INVALID_VALUE: invalid argument";
    case LL_ERR_NO_DEVICE: return "LL_ERR_NO_DEVICE: no HIP device available";
    case LL_ERR_UNSUPPORTED_ARCH: return "LL_ERR_UNSUPPORTED_ARCH: device is not gfx950";
    case LL_ERR_LAUNCH: return "LL_ERR_LAUNCH: kernel launch failed";
    default: return "unknown linear_layer status";
    }
}

int ll_set_tile(int dtype, int tile)
{
    if (dtype != LL_DTYPE_F32 && dtype != LL_DTYPE_F16)
        return LL_ERR_INVALID_VALUE;
    const int n = dtype == LL_DTYPE_F32 ? kF32NumTiles : kF16NumTiles;
    if (tile < -1 || tile >= n)
        return LL_ERR_INVALID_VALUE;
    store_override(dtype == LL_DTYPE_F32 ? 0 : 8, tile);
    return LL_OK;
}

int ll_num_tiles(int dtype)
{
    if (dtype == LL_DTYPE_F32)
        return kF32NumTiles;
    if (dtype == LL_DTYPE_F16)
        return kF16NumTiles;
    return 0;
}

const char *ll_tile_name(int dtype, int tile)
{
    if (dtype == LL_DTYPE_F32 && tile >= 0 && tile < kF32NumTiles)
        return kF32Tiles[tile].name;
    if (dtype == LL_DTYPE_F16 && tile >= 0 && tile < kF16NumTiles)
        return kF16Tiles[tile].name;
    return "";
}

static Plan chosen_plan(int dtype, int M, int N, int K, int batch, int num_cus, bool *ok)
{
    const int base = dtype & 0xff, flags = dtype & ~0xff;
    const bool relu = flags & LL_PLAN_RELU, bt = flags & LL_PLAN_B_NK;
    const bool vec = !(flags & LL_PLAN_UNALIGNED);
    *ok = (base == LL_DTYPE_F32 || (base == LL_DTYPE_F16 && !relu)) &&
          (flags & ~(LL_PLAN_RELU | LL_PLAN_B_NK | LL_PLAN_UNALIGNED)) == 0 && batch >= 1;
    if (!*ok)
        return Plan{-1, -1, 0};
    const int cus = num_cus > 0 ? num_cus : 256;
    const Plan pl = base == LL_DTYPE_F32
                        ? plan(0, kF32Tiles, kF32NumTiles, M, N, K, cus, relu, batch, vec, bt)
                        : plan(1, kF16Tiles, kF16NumTiles, M, N, K, cus, false, batch, vec, bt);
    if (pl.tile < 0)
        *ok = false;
    return pl;
}

int ll_chosen_tile(int dtype, int M, int N, int K, int batch, int num_cus)
{
    bool ok;
    const Plan p = chosen_plan(dtype, M, N, K, batch, num_cus, &ok);
    return ok ? p.tile : -1;
}

int ll_chosen_split_k(int dtype, int M, int N, int K, int batch, int num_cus)
{
    bool ok;
    const Plan p = chosen_plan(dtype, M, N, K, batch, num_cus, &ok);
    return ok ? p.splits : -1;
}

int ll_chosen_stream_k(int dtype, int M, int N, int K, int batch, int num_cus)
{
    bool ok;
    const Plan p = chosen_plan(dtype, M, N, K, batch, num_cus, &ok);
    if (!ok)
        return -1;
    if (p.sk_grid == 0)
        return 0;
    const TileInfo &ti = (dtype & 0xFF) == LL_DTYPE_F32 ? kF32Tiles[p.tile] : kF16Tiles[p.tile];
    return (int)((int64_t)cdiv(M, ti.bm) * cdiv(N, ti.bn) - p.dp_tiles);
}

int ll_set_stream_k(int mode)
{
    if (mode < -1 || mode > 1)
        return LL_ERR_INVALID_VALUE;
    store_override(24, mode);
    return LL_OK;
}

int ll_set_split_k(int splits)
{
    if (splits != -1 && (splits < 1 || splits > kMaxSplits))
        return LL_ERR_INVALID_VALUE;
    store_override(16, splits);
    return LL_OK;
}

}  // extern "C"
