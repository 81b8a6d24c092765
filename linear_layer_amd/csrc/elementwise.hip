// Elementwise row sweeps (HBM-bound). They serve the degenerate cases of the
// GEMM definition (page "GEMM 优化详解", section "GEMM 基础理论 / 数学定义"):
// when K == 0 or alpha == 0 the product term vanishes and C = beta*C; for the
// fully-connected layer with K == 0, Y = act(bias). They also frame a split-K
// product: C = beta*C (or Y = bias) before the atomically added partial sums,
// and the ReLU after them.
#include "common.hpp"
#include "launch.hpp"

namespace ll {

// A workgroup sweeps 1024 columns of a row (four values per thread, 256
// apart, all four loads issued before the stores), grid y walks the rows and
// grid z the items of a strided batch (stride_c bytes apart); a row of a
// thousand or so values is one wave of loads, not a loop of dependent ones.
constexpr int kSweepCols = 1024;

template <class F>
__device__ __forceinline__ void sweep_rows(float *base, int64_t ld, int M, int N, bool reads, F f)
{
    const int64_t n0 = (int64_t)blockIdx.x * kSweepCols + threadIdx.x;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        float *row = base + m * ld;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = reads && n0 + 256 * j < N ? row[n0 + 256 * j] : 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (n0 + 256 * j < N)
                row[n0 + 256 * j] = f(v[j], n0 + 256 * j);
    }
}

__global__ void __launch_bounds__(256) scale_kernel(float *C, int64_t ldc, int M, int N, float beta,
                                                    int64_t stride_c)
{
    C = reinterpret_cast<float *>(reinterpret_cast<char *>(C) + (int64_t)blockIdx.z * stride_c);
    sweep_rows(C, ldc, M, N, beta != 0.0f,
               [beta](float v, int64_t) { return beta == 0.0f ? 0.0f : beta * v; });
}

__global__ void __launch_bounds__(256) bias_fill_kernel(float *Y, int64_t ldy, int M, int N,
                                                        const float *bias, int act)
{
    sweep_rows(Y, ldy, M, N, false, [bias, act](float, int64_t n) {
        const float v = bias ? bias[n] : 0.0f;
        return act == 1 ? (v > 0.0f ? v : 0.0f) : v;
    });
}

// In-place ReLU (y <= 0 and NaN -> +0), the last step of a split-K
// fully-connected layer whose partial sums were accumulated atomically.
__global__ void __launch_bounds__(256) relu_kernel(float *Y, int64_t ldy, int M, int N)
{
    sweep_rows(Y, ldy, M, N, true, [](float v, int64_t) { return v > 0.0f ? v : 0.0f; });
}

// The same three operations on whole output tiles: tiles tile_base ..
// tile_base + count - 1 of p's grouped tile order (tiles of bm x bn). They
// frame the stream-K share of a product, whose tiles receive atomic partial
// sums: C = beta*C or Y = bias before, ReLU after. A workgroup sweeps
// kPassRows rows of a tile with 128-bit accesses (stream-K runs only with C
// 16-byte aligned and ldc a multiple of 4; a column tail short of 4 values,
// possible when B is given N-by-K, is done value by value).
constexpr int kPassRows = 16;

__device__ __forceinline__ float pass_one(float v, float b, const GemmParams &p, int mode)
{
    if (mode == TILE_SCALE)
        return p.beta == 0.0f ? 0.0f : p.beta * v;
    if (mode == TILE_BIAS)
        return b;
    return v > 0.0f ? v : 0.0f;
}

__global__ void __launch_bounds__(256) tile_pass_kernel(GemmParams p, int bm, int bn, int mode)
{
    const int parts = bm / kPassRows;
    const int t = blockIdx.x / parts, part = blockIdx.x % parts;
    int tm, tn;
    tile_of(p, p.tile_base + t, tm, tn);
    const int lanes_per_row = bn / 4, rows_per_iter = 256 / lanes_per_row;
    const int m0 = tm * bm + part * kPassRows, m1 = min(p.M, m0 + kPassRows);
    const int n = tn * bn + 4 * ((int)threadIdx.x % lanes_per_row), n1 = min(p.N, tn * bn + bn);
    if (n >= n1)
        return;
    const int width = n1 - n < 4 ? n1 - n : 4;
    float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (mode == TILE_BIAS && p.bias != nullptr)
        for (int e = 0; e < width; ++e)
            b[e] = p.bias[n + e];
    for (int m = m0 + (int)threadIdx.x / lanes_per_row; m < m1; m += rows_per_iter) {
        float *dst = p.C + (int64_t)m * p.ldc + n;
        if (width == 4) {
            f32x4 v = mode == TILE_BIAS ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : *reinterpret_cast<f32x4 *>(dst);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = pass_one(v[e], b[e], p, mode);
            *reinterpret_cast<f32x4 *>(dst) = v;
        } else {
            for (int e = 0; e < width; ++e)
                dst[e] = pass_one(mode == TILE_BIAS ? 0.0f : dst[e], b[e], p, mode);
        }
    }
}

hipError_t launch_tile_pass(const GemmParams &p0, int bm, int bn, int first_tile, int count, int mode,
                            hipStream_t s)
{
    if (count <= 0)
        return hipSuccess;
    GemmParams p = p0;
    p.tile_base = first_tile;
    if (bm % kPassRows != 0 || bn % 4 != 0 || bn > 1024 || 1024 % bn != 0)
        return hipErrorInvalidValue;   // every tile shape here passes
    hipLaunchKernelGGL(tile_pass_kernel, dim3((unsigned)count * (bm / kPassRows)), dim3(256), 0, s,
                       p, bm, bn, mode);
    return hipGetLastError();
}

static dim3 sweep_grid(int M, int N, int batch = 1)
{
    return dim3((unsigned)((N + kSweepCols - 1) / kSweepCols), (unsigned)(M < 65535 ? M : 65535),
                (unsigned)batch);
}

hipError_t launch_scale(float *C, int64_t ldc, int M, int N, float beta, hipStream_t s, int batch,
                        int64_t stride_c)
{
    if (M <= 0 || N <= 0 || batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(scale_kernel, sweep_grid(M, N, batch), dim3(256), 0, s, C, ldc, M, N, beta,
                       stride_c);
    return hipGetLastError();
}

hipError_t launch_relu(float *Y, int64_t ldy, int M, int N, hipStream_t s)
{
    if (M <= 0 || N <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(relu_kernel, sweep_grid(M, N), dim3(256), 0, s, Y, ldy, M, N);
    return hipGetLastError();
}

hipError_t launch_bias_fill(float *Y, int64_t ldy, int M, int N, const float *bias, int act,
                            hipStream_t s)
{
    if (M <= 0 || N <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(bias_fill_kernel, sweep_grid(M, N), dim3(256), 0, s, Y, ldy, M, N, bias, act);
    return hipGetLastError();
}

}  // namespace ll
