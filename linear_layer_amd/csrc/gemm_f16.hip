// FP16-input GEMM with FP32 accumulation and FP32 output on the CDNA4 matrix
// cores: C = alpha*A*B + beta*C with binary16 A and B.
//
// The FP16-in / FP32-accumulate product is the tensor-core step of page
// "GPU架构下的矩阵乘法深入优化", section 6, in the general form of page
// "GEMM 优化详解", section "GEMM 基础理论 / 数学定义". The page's design
// (128x128x32 block tile, 16x16x16 fragments, A transposed in shared memory,
// 16-half skew) was made for Volta; this kernel is planned for gfx950:
//
//   * 4 waves (2x2); each wave owns (BM/2) x (BN/2) of C as 32x32 blocks, each
//     block one v_mfma_f32_32x32x16_f16 accumulator (16 fp32 per lane). One
//     MFMA takes 8 consecutive k-values per lane for both operands.
//   * Both operands sit in LDS with k contiguous ([m][k] for A, [n][k] for B),
//     so every operand fetch is one 128-bit LDS read. A arrives that way from
//     row-major memory. B (row-major K x N) is transposed on its way in: a
//     thread loads an 8x8 block of B (eight 128-bit row loads), transposes it
//     in registers with 16-bit packs, and stores eight 128-bit [n][k] rows.
//   * Rows of both LDS tiles are 128 bytes; 16-byte chunks are XOR-swizzled
//     with the row index, so eight lanes reading the same logical chunk of
//     eight rows (or writing eight k-chunks of one row) cover all 32 banks.
//   * Two LDS stages, register-staged prefetch of the next stage during the
//     MFMAs of the current one, one barrier per stage. Zero-filled loads
//     outside M, N, K; masked, fused write-back.
#include "common.hpp"
#include "launch.hpp"

namespace ll {

template <int BM_, int BN_, int BK_>
struct F16Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int NT = 256;
    static constexpr int WTM = BM / 2, WTN = BN / 2;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int KSTEPS = BK / 16;          // MFMA k-steps per stage
    static constexpr int CPR = BK / 8;              // 16-byte chunks per LDS row
    static constexpr int A_CH = BM * CPR;           // A chunks per stage
    static constexpr int A_PT = A_CH / NT;
    static constexpr int B_BLK = (BK / 8) * (BN / 8);  // 8x8 B blocks per stage
    static constexpr int B_PT = (B_BLK + NT - 1) / NT;
    static_assert(BK == 64, "LDS rows are 128 bytes");
    static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");
    static_assert(A_PT >= 1 && A_PT * NT == A_CH, "A chunks must split evenly");
};

__device__ __forceinline__ uint16_t ld_u16(const uint16_t *p) { return *p; }

template <class T, int EPI, bool VEC, int WPE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
gemm_f16_kernel(GemmParams p)
{
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK;
    constexpr int FM = T::FM, FN = T::FN, CPR = T::CPR;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const uint16_t *__restrict__ A = static_cast<const uint16_t *>(p.A);
    const uint16_t *__restrict__ B = static_cast<const uint16_t *>(p.B);
    const int M = p.M, N = p.N, K = p.K;

    // A chunk i of this thread: row a_r0 + i*A_RSTEP, 16-byte chunk a_c.
    const int a_c = tid % CPR;
    const int a_r0 = tid / CPR;
    constexpr int A_RSTEP = T::NT / CPR;
    const uint16_t *a_ptr = A + (int64_t)(m0 + a_r0) * p.lda + a_c * 8;
    const int64_t a_istep = (int64_t)A_RSTEP * p.lda;

    // B block i of this thread: id = i*NT + tid; k-block id % (BK/8) (so the
    // eight lanes of a group write eight different k-chunks of one LDS row),
    // n-block id / (BK/8).
    u32x4 ra[T::A_PT];
    u32x4 rb[T::B_PT][8];

    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < T::A_PT; ++i) {
            const bool rok = m0 + a_r0 + i * A_RSTEP < M;
            const int kk = k0 + a_c * 8;
            const uint16_t *src = a_ptr + i * a_istep + k0;
            if (VEC) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (rok && kk < K)
                    v = *reinterpret_cast<const u32x4 *>(src);
                ra[i] = v;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t lo = (rok && kk + 2 * j < K) ? ld_u16(src + 2 * j) : 0u;
                    const uint32_t hi = (rok && kk + 2 * j + 1 < K) ? ld_u16(src + 2 * j + 1) : 0u;
                    ra[i][j] = lo | (hi << 16);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < T::B_PT; ++i) {
            const int id = i * T::NT + tid;
            const int kb = id % (BK / 8), nb = id / (BK / 8);
            const bool active = (T::B_PT * T::NT == T::B_BLK) || id < T::B_BLK;
            const int nn = n0 + nb * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kk = k0 + kb * 8 + j;
                const uint16_t *src = B + (int64_t)kk * p.ldb + nn;
                if (VEC) {
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (active && kk < K && nn < N)
                        v = *reinterpret_cast<const u32x4 *>(src);
                    rb[i][j] = v;
                } else {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const bool ok = active && kk < K;
                        const uint32_t lo = (ok && nn + 2 * d < N) ? ld_u16(src + 2 * d) : 0u;
                        const uint32_t hi = (ok && nn + 2 * d + 1 < N) ? ld_u16(src + 2 * d + 1) : 0u;
                        rb[i][j][d] = lo | (hi << 16);
                    }
                }
            }
        }
    };

    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < T::A_PT; ++i) {
            const int row = a_r0 + i * A_RSTEP;
            const int c = a_c ^ swz<BK * 2>(row);
            *reinterpret_cast<u32x4 *>(&As[buf][row * BK + c * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < T::B_PT; ++i) {
            const int id = i * T::NT + tid;
            if ((T::B_PT * T::NT == T::B_BLK) || id < T::B_BLK) {
                const int kb = id % (BK / 8), nb = id / (BK / 8);
                // rb[i][j] holds row k = kb*8 + j, columns nb*8 .. nb*8+7 (two per
                // dword, low half first). Column c of the block becomes LDS row
                // nb*8 + c holding k = kb*8 .. kb*8+7.
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int d = c >> 1;
                    u32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t x0 = rb[i][2 * e][d], x1 = rb[i][2 * e + 1][d];
                        w[e] = (c & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u))
                                       : ((x0 & 0xffffu) | (x1 << 16));
                    }
                    const int row = nb * 8 + c;
                    const int ch = kb ^ swz<BK * 2>(row);
                    *reinterpret_cast<u32x4 *>(&Bs[buf][row * BK + ch * 8]) = w;
                }
            }
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    const int h = lane >> 5, l32 = lane & 31;
    const int nk = (K + BK - 1) / BK;

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk)
            gload((kt + 1) * BK);
#pragma unroll
        for (int s = 0; s < T::KSTEPS; ++s) {
            // Lane half h takes k = s*16 + h*8 .. +7 for both operands.
            const int ch = 2 * s + h;
            f16x8 af[FM], bf[FN];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int row = wm * T::WTM + fm * 32 + l32;
                af[fm] = *reinterpret_cast<const f16x8 *>(
                    &As[cur][row * BK + (ch ^ swz<BK * 2>(row)) * 8]);
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int row = wn * T::WTN + fn * 32 + l32;
                bf[fn] = *reinterpret_cast<const f16x8 *>(
                    &Bs[cur][row * BK + (ch ^ swz<BK * 2>(row)) * 8]);
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[fm], bf[fn],
                                                                         acc[fm][fn], 0, 0, 0);
        }
        if (kt + 1 < nk)
            lstore(cur ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            write_block<EPI>(p, acc[fm][fn], m0 + wm * T::WTM + fm * 32,
                             n0 + wn * T::WTN + fn * 32, lane);
}

using F16_L = F16Tile<256, 256, 64>;
using F16_S = F16Tile<128, 128, 64>;
using F16_XS = F16Tile<64, 64, 64>;

template <class T, int WPE>
static hipError_t launch_t(const GemmParams &p0, int epi, bool vec, hipStream_t s)
{
    GemmParams p = p0;
    p.tiles_m = (p.M + T::BM - 1) / T::BM;
    p.tiles_n = (p.N + T::BN - 1) / T::BN;
    const int64_t ntiles = (int64_t)p.tiles_m * p.tiles_n;
    if (ntiles > 0x7fffffff)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)ntiles), block(T::NT);
#define LL_F16_LAUNCH(E, V) \
    hipLaunchKernelGGL((gemm_f16_kernel<T, E, V, WPE>), grid, block, 0, s, p)
    if (vec) {
        if (epi == EPI_GEMM_BETA0) LL_F16_LAUNCH(EPI_GEMM_BETA0, true);
        else LL_F16_LAUNCH(EPI_GEMM_BETA, true);
    } else {
        if (epi == EPI_GEMM_BETA0) LL_F16_LAUNCH(EPI_GEMM_BETA0, false);
        else LL_F16_LAUNCH(EPI_GEMM_BETA, false);
    }
#undef LL_F16_LAUNCH
    return hipGetLastError();
}

// {BM, BN, workgroups per CU, relative throughput alone, paired} (see the
// FP32 table); measured on the 8192^3 product.
const TileInfo kF16Tiles[kF16NumTiles] = {
    {F16_L::BM, F16_L::BN, 1, 1.00f, 1.00f, "f16_256x256x64"},
    {F16_S::BM, F16_S::BN, 2, 0.60f, 0.79f, "f16_128x128x64"},
    {F16_XS::BM, F16_XS::BN, 2, 0.25f, 0.32f, "f16_64x64x64"},
};

hipError_t launch_gemm_f16(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s)
{
    switch (tile) {
    case 0: return launch_t<F16_L, 1>(p, epi, vec, s);
    case 1: return launch_t<F16_S, 2>(p, epi, vec, s);
    default: return launch_t<F16_XS, 2>(p, epi, vec, s);
    }
}

}  // namespace ll
