// Elementwise row sweeps (HBM-bound). They serve the degenerate cases of the
// GEMM definition (page "GEMM 优化详解", section "GEMM 基础理论 / 数学定义"):
// when K == 0 or alpha == 0 the product term vanishes and C = beta*C; for the
// fully-connected layer with K == 0, Y = act(bias). They also frame a split-K
// product: C = beta*C (or Y = bias) before the atomically added partial sums,
// and the ReLU after them.
#include "common.hpp"
#include "launch.hpp"

namespace ll {

// One workgroup per row-stripe, threads striding along the row; grid z walks
// the items of a strided batch (stride_c bytes apart).
__global__ void __launch_bounds__(256) scale_kernel(float *C, int64_t ldc, int M, int N, float beta,
                                                    int64_t stride_c)
{
    C = reinterpret_cast<float *>(reinterpret_cast<char *>(C) + (int64_t)blockIdx.z * stride_c);
    for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
        float *row = C + m * ldc;
        for (int n = threadIdx.x; n < N; n += blockDim.x)
            row[n] = (beta == 0.0f) ? 0.0f : beta * row[n];
    }
}

__global__ void __launch_bounds__(256) bias_fill_kernel(float *Y, int64_t ldy, int M, int N,
                                                        const float *bias, int act)
{
    for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
        float *row = Y + m * ldy;
        for (int n = threadIdx.x; n < N; n += blockDim.x) {
            float v = bias ? bias[n] : 0.0f;
            if (act == 1)
                v = v > 0.0f ? v : 0.0f;
            row[n] = v;
        }
    }
}

// In-place ReLU (y <= 0 and NaN -> +0), the last step of a split-K
// fully-connected layer whose partial sums were accumulated atomically.
__global__ void __launch_bounds__(256) relu_kernel(float *Y, int64_t ldy, int M, int N)
{
    for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
        float *row = Y + m * ldy;
        for (int n = threadIdx.x; n < N; n += blockDim.x) {
            const float v = row[n];
            row[n] = v > 0.0f ? v : 0.0f;
        }
    }
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

static unsigned rows_grid(int M)
{
    return (unsigned)(M < 65536 ? M : 65536);
}

hipError_t launch_scale(float *C, int64_t ldc, int M, int N, float beta, hipStream_t s, int batch,
                        int64_t stride_c)
{
    hipLaunchKernelGGL(scale_kernel, dim3(rows_grid(M), 1, (unsigned)batch), dim3(256), 0, s, C, ldc,
                       M, N, beta, stride_c);
    return hipGetLastError();
}

hipError_t launch_relu(float *Y, int64_t ldy, int M, int N, hipStream_t s)
{
    hipLaunchKernelGGL(relu_kernel, dim3(rows_grid(M)), dim3(256), 0, s, Y, ldy, M, N);
    return hipGetLastError();
}

hipError_t launch_bias_fill(float *Y, int64_t ldy, int M, int N, const float *bias, int act,
                            hipStream_t s)
{
    hipLaunchKernelGGL(bias_fill_kernel, dim3(rows_grid(M)), dim3(256), 0, s, Y, ldy, M, N, bias,
                       act);
    return hipGetLastError();
}

}  // namespace ll
