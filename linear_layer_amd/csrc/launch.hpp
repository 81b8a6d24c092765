// Host-side launchers exported by the kernel translation units to the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace ll {

struct TileInfo {
    int bm, bn;
    int wg_per_cu;     // workgroups resident per CU (register/LDS limited)
    float eff_alone;   // relative CU throughput with one workgroup on it
    float eff_paired;  // relative CU throughput with wg_per_cu workgroups on it
    const char *name;
    int k_slices = 1;  // K-slices inside the workgroup (such tiles take no stream-K share)
    bool stream_k = true;  // the tile's kernel can run a stream-K launch
    int threads = 256;     // largest workgroup of the tile's kernels
    int min_k = 0;         // K-sliced tiles: the K below which slices get too few stages
    bool direct_only = false;  // only the 128-bit-load kernels have this shape
    int k_ref = 0;         // K per workgroup at which eff_* were measured (0: rates independent of K)
    float eff_max = 0.0f;  // the highest rate at longer K ranges (0: eff_alone)
};

constexpr int kF32NumTiles = 8;
// The FP32 tile that is the skinny kernel (vector FMAs for a few rows of A;
// planned by rule, not by the MFMA tiles' cost model) and its column width.
// It is chosen automatically for at most kSkinnyMaxM rows of A, and for up
// to kSkinnyMaxMLarge rows when B holds at least kSkinnyLargeKN values.
// Measured on MI355X against the 64x64 MFMA plan: 1.6 to 1.8 times its rate
// up to 4 rows; 1.1 to 1.5 times for 5 to 8 rows with a 4096 x 11008 B, but
// slower with a 4096 x 4096 one (its K-splits' atomic sums and short ranges
// cost more there than the vector FMAs save); past 8 rows the MFMA tiles win.
constexpr int kSkinnyTile = 6, kSkinnyCols = 256, kSkinnyMaxM = 4, kSkinnyMaxMLarge = 8;
// The 32x128 tile: chosen automatically only when one row of its tiles covers
// M (more rows read B once per row of tiles; from 40 rows on, 64x64 measured
// faster) ...
constexpr int kThinTile = 7;
// ... and split only into K ranges of at least this many values
// (32x8192x2048 in 16 splits of 128: 30 us against 25 on 64x64 in 4).
constexpr int kThinMinSplit = 256;
constexpr int64_t kSkinnyLargeKN = (int64_t)1 << 25;
// Floats of A the skinny kernel stages in LDS at once, its rows per pass
// for a product of M rows (the fewest of 1, 2, 4, 8, 16 that cover M), and so
// the longest K range it stages whole.
constexpr int kSkinnyStage = 8192;
constexpr int skinny_rows(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }
constexpr int skinny_kmax(int M) { return kSkinnyStage / skinny_rows(M); }
constexpr int kF16NumTiles = 6;
// The 16-bit tile that is the skinny kernel (dot2 instructions for a few rows
// of A, B given N-by-K) and the 16-bit values of A it stages at once. It is
// chosen automatically for one row of A with B of at least kSkinnyLargeKN
// values. Measured on MI355X against the MFMA plan, per call: one row 0.79
// to 1.01 times its time with such a B (11008 x 4096 0.85, 28672 x 8192
// 0.79, 4096 x 8192 1.01), 1.00 to 1.03 with smaller ones (4096 x 4096,
// 5120 x 5120); two rows 0.76 to 1.06 times, four and eight 1.05 to 1.9
// (each lane reads A's values from LDS again for every group of four
// columns, and the work per byte of B grows with the rows).
constexpr int kSkinny16Tile = 5, kSkinny16MaxM = 1;
constexpr int kSkinny16Stage = 16384, kSkinny16Align = 128;
constexpr int skinny16_kmax(int M) { return kSkinny16Stage / skinny_rows(M); }
extern const TileInfo kF32Tiles[kF32NumTiles];
extern const TileInfo kF16Tiles[kF16NumTiles];

// One GEMM launch. `tile` indexes kF32Tiles / kF16Tiles, `epi` is an Epi
// value, `vec` selects the 128-bit-load kernels (the caller has checked
// alignment and divisibility). Fills p.tiles_m / p.tiles_n itself; the grid
// has ceil(K / p.k_split) K-splits along y (EPI_ATOMIC when more than one)
// and p.batch items along z (at most kMaxGridZ).
hipError_t launch_gemm_f32(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s);
// As above with B given N-by-K (C = alpha*A*B^T + beta*C).
hipError_t launch_gemm_f32_bt(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s);
hipError_t launch_gemm_f16(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s);
hipError_t launch_gemm_f16_bt(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s);
hipError_t launch_gemm_bf16_bt(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s);

// Largest grid y / z extent a launch may use, and the most workgroups along
// x a launch of `threads`-thread workgroups may have (its work-item count
// along x must fit 32 bits).
constexpr int kMaxGridZ = 65535;
constexpr int64_t max_grid_x(int threads)
{
    return (int64_t)(0xffffffffu / (unsigned)threads);
}
constexpr int64_t kMaxTiles = max_grid_x(256);

// C = beta*C over an M x N matrix (beta == 0 writes zeros without reading C),
// for each of `batch` matrices stride_c bytes apart.
hipError_t launch_scale(float *C, int64_t ldc, int M, int N, float beta, hipStream_t s,
                        int batch = 1, int64_t stride_c = 0);
// Passes over whole output tiles first_tile .. first_tile+count-1 of p's
// grouped tile order (p.tiles_m, p.tiles_n, p.group_m set for bm x bn tiles):
// C = beta*C, Y = bias (or 0), or in-place ReLU.
enum TilePass { TILE_SCALE = 0, TILE_BIAS = 1, TILE_RELU = 2 };
hipError_t launch_tile_pass(const GemmParams &p, int bm, int bn, int first_tile, int count, int mode,
                            hipStream_t s);
// In-place ReLU over an M x N matrix.
hipError_t launch_relu(float *Y, int64_t ldy, int M, int N, hipStream_t s);
// Y = act(bias) broadcast over M rows (bias may be nullptr: act(0)).
hipError_t launch_bias_fill(float *Y, int64_t ldy, int M, int N, const float *bias, int act,
                            hipStream_t s);

}  // namespace ll
