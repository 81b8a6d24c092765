// FP32 GEMM on the CDNA4 matrix cores: C = alpha*A*B + beta*C and the fused
// fully-connected write-back act(X*W + bias).
//
// The operation is the one defined on page "GEMM 优化详解", section
// "GEMM 基础理论 / 数学定义". The pages build it up as a ladder of CUDA
// kernels (shared-memory tiles, coalescing, padding, double buffering,
// register blocking, float4 loads; page "GPU架构下的矩阵乘法深入优化"
// sections 2-5); this kernel keeps the ideas that still hold on gfx950 and
// re-plans the rest for wave64 and MFMA:
//
//   * Workgroup of 4 waves (2x2) owns a BM x BN output tile; each wave owns a
//     (BM/2) x (BN/2) sub-tile made of 32x32 blocks, each block one
//     v_mfma_f32_32x32x2_f32 accumulator (16 fp32 per lane).
//   * K is walked in stages of BK. A stage of A (BM x BK) and B (BK x BN) is
//     fetched with 128-bit loads into registers, then written to the other of
//     two LDS buffers while the MFMAs consume the current one: one barrier per
//     stage (the ping-pong of page "GPU架构下的矩阵乘法深入优化", section 5).
//   * A stays row-major in LDS ([m][k]) with an XOR swizzle of its 16-byte
//     chunks, so a lane fetches its BK/2 k-values of one row with 128-bit LDS
//     reads and eight lanes of consecutive rows cover all banks (the pages pad
//     or transpose instead). B stays [k][n]; its rows are padded by 4 floats
//     so that the two half-waves, which read rows BK/2 apart, land on
//     different banks.
//   * Inside a stage, lane half h (lanes 32h..32h+31) handles k = h*BK/2 + s
//     at MFMA step s. The MFMA sums over both halves, so any pairing of k with
//     (half, step) is valid as long as A and B agree on it; this one makes a
//     lane's A values contiguous.
//   * Out-of-range rows, columns and K tails are loaded as zeros; the store is
//     masked. No barrier is ever inside a bounds branch.
//   * The write-back applies alpha/beta or bias+ReLU to the accumulators
//     before the single store of C (page "GEMM 优化详解", "Level 6: Kernel
//     Fusion").
#include "common.hpp"
#include "launch.hpp"

namespace ll {

template <int BM_, int BN_, int BK_>
struct F32Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int NT = 256;                 // 4 waves, 2 x 2
    static constexpr int WTM = BM / 2, WTN = BN / 2;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int KH = BK / 2;              // k values per lane half per stage
    static constexpr int ACPR = BK / 4;            // 16-byte chunks per A row
    static constexpr int A_PT = BM * ACPR / NT;    // A chunks per thread
    static constexpr int BCPR = BN / 4;            // 16-byte chunks per B row
    static constexpr int B_PT = BK * BCPR / NT;    // B chunks per thread
    static constexpr int BNP = BN + 4;             // padded B row (floats)
    static constexpr int A_STAGE = BM * BK;        // floats
    static constexpr int B_STAGE = BK * BNP;
    static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");
    static_assert(A_PT >= 1 && A_PT * NT == BM * ACPR, "A chunks must split evenly");
    static_assert(B_PT >= 1 && B_PT * NT == BK * BCPR, "B chunks must split evenly");
    static_assert(KH % 4 == 0, "BK must be a multiple of 8");
};

template <class T, int EPI, bool VEC, int WPE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
gemm_f32_kernel(GemmParams p)
{
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK, KH = T::KH;
    constexpr int FM = T::FM, FN = T::FN, BNP = T::BNP;
    __shared__ __attribute__((aligned(16))) float As[2][T::A_STAGE];
    __shared__ __attribute__((aligned(16))) float Bs[2][T::B_STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    int K;
    const int kb = split_range(p, K);
    const float *__restrict__ A = static_cast<const float *>(p.A) + kb;
    const float *__restrict__ B = static_cast<const float *>(p.B) + (int64_t)kb * p.ldb;
    const int M = p.M, N = p.N;

    // Fixed per-thread load assignment: A chunk i is row a_row(i), chunk a_c;
    // B chunk i is k-row b_k(i), column chunk b_c.
    const int a_c = tid % T::ACPR;
    const int a_r0 = tid / T::ACPR;
    constexpr int A_RSTEP = T::NT / T::ACPR;
    const int b_c = tid % T::BCPR;
    const int b_k0 = tid / T::BCPR;
    constexpr int B_KSTEP = T::NT / T::BCPR;

    const float *a_ptr = A + (int64_t)(m0 + a_r0) * p.lda + a_c * 4;
    const float *b_ptr = B + (int64_t)b_k0 * p.ldb + n0 + b_c * 4;
    const int64_t a_istep = (int64_t)A_RSTEP * p.lda;
    const int64_t b_istep = (int64_t)B_KSTEP * p.ldb;

    f32x4 ra[T::A_PT], rb[T::B_PT];

    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < T::A_PT; ++i) {
            const bool rok = m0 + a_r0 + i * A_RSTEP < M;
            const float *src = a_ptr + i * a_istep + k0;
            const int kk = k0 + a_c * 4;
            if (VEC) {
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (rok && kk < K)
                    v = *reinterpret_cast<const f32x4 *>(src);
                ra[i] = v;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    ra[i][j] = (rok && kk + j < K) ? src[j] : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < T::B_PT; ++i) {
            const int kk = k0 + b_k0 + i * B_KSTEP;
            const int nn = n0 + b_c * 4;
            const float *src = b_ptr + i * b_istep + (int64_t)k0 * p.ldb;
            if (VEC) {
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (kk < K && nn < N)
                    v = *reinterpret_cast<const f32x4 *>(src);
                rb[i] = v;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    rb[i][j] = (kk < K && nn + j < N) ? src[j] : 0.0f;
            }
        }
    };

    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < T::A_PT; ++i) {
            const int row = a_r0 + i * A_RSTEP;
            const int c = a_c ^ swz<BK * 4>(row);
            *reinterpret_cast<f32x4 *>(&As[buf][row * BK + c * 4]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < T::B_PT; ++i) {
            const int kr = b_k0 + i * B_KSTEP;
            *reinterpret_cast<f32x4 *>(&Bs[buf][kr * BNP + b_c * 4]) = rb[i];
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

        // A fragments for the whole stage: row = lane's row, k = h*KH .. h*KH+KH-1.
        f32x4 af[FM][KH / 4];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int row = wm * T::WTM + fm * 32 + l32;
#pragma unroll
            for (int q = 0; q < KH / 4; ++q) {
                const int c = (h * (KH / 4) + q) ^ swz<BK * 4>(row);
                af[fm][q] = *reinterpret_cast<const f32x4 *>(&As[cur][row * BK + c * 4]);
            }
        }
        const float *bsrc = &Bs[cur][(h * KH) * BNP + wn * T::WTN + l32];
#pragma unroll
        for (int s = 0; s < KH; ++s) {
            float bf[FN];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                bf[fn] = bsrc[s * BNP + fn * 32];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        af[fm][s >> 2][s & 3], bf[fn], acc[fm][fn], 0, 0, 0);
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

// Tile configurations. The 256x256 tile runs one wave per SIMD (256
// accumulators per lane); the others are compiled for two waves per SIMD, so
// two workgroups share a CU and each covers the other's barrier and memory
// waits. Measured on the 4096^3 product, 256x128 at two workgroups per CU is
// the fastest (about 83 % of the FP32 matrix peak), and it also quantises
// best on the 2047 x 11008 fully-connected layer.
using F32_L = F32Tile<256, 256, 16>;   // 128x128 per wave
using F32_M = F32Tile<256, 128, 16>;   // 128x64 per wave
using F32_S = F32Tile<128, 128, 16>;   // 64x64 per wave
using F32_XS = F32Tile<64, 64, 16>;    // 32x32 per wave

template <class T, int WPE>
static hipError_t launch_t(const GemmParams &p0, int epi, bool vec, hipStream_t s)
{
    GemmParams p = p0;
    p.tiles_m = (p.M + T::BM - 1) / T::BM;
    p.tiles_n = (p.N + T::BN - 1) / T::BN;
    const int64_t ntiles = (int64_t)p.tiles_m * p.tiles_n;
    if (ntiles > 0x7fffffff)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)ntiles, (unsigned)((p.K + p.k_split - 1) / p.k_split)), block(T::NT);
#define LL_F32_LAUNCH(E, V) \
    hipLaunchKernelGGL((gemm_f32_kernel<T, E, V, WPE>), grid, block, 0, s, p)
    if (vec) {
        if (epi == EPI_GEMM_BETA0) LL_F32_LAUNCH(EPI_GEMM_BETA0, true);
        else if (epi == EPI_GEMM_BETA) LL_F32_LAUNCH(EPI_GEMM_BETA, true);
        else if (epi == EPI_LINEAR) LL_F32_LAUNCH(EPI_LINEAR, true);
        else LL_F32_LAUNCH(EPI_ATOMIC, true);
    } else {
        if (epi == EPI_GEMM_BETA0) LL_F32_LAUNCH(EPI_GEMM_BETA0, false);
        else if (epi == EPI_GEMM_BETA) LL_F32_LAUNCH(EPI_GEMM_BETA, false);
        else if (epi == EPI_LINEAR) LL_F32_LAUNCH(EPI_LINEAR, false);
        else LL_F32_LAUNCH(EPI_ATOMIC, false);
    }
#undef LL_F32_LAUNCH
    return hipGetLastError();
}

// {BM, BN, workgroups per CU, relative throughput alone on a CU, with a
// second workgroup beside it} -- throughputs measured on MI355X relative to
// the 256x256 tile.
const TileInfo kF32Tiles[kF32NumTiles] = {
    {F32_L::BM, F32_L::BN, 1, 1.00f, 1.00f, "f32_256x256x16"},
    {F32_M::BM, F32_M::BN, 2, 0.89f, 1.01f, "f32_256x128x16"},
    {F32_S::BM, F32_S::BN, 2, 0.80f, 0.94f, "f32_128x128x16"},
    {F32_XS::BM, F32_XS::BN, 2, 0.40f, 0.72f, "f32_64x64x16"},
};

hipError_t launch_gemm_f32(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s)
{
    switch (tile) {
    case 0: return launch_t<F32_L, 1>(p, epi, vec, s);
    case 1: return launch_t<F32_M, 2>(p, epi, vec, s);
    case 2: return launch_t<F32_S, 2>(p, epi, vec, s);
    default: return launch_t<F32_XS, 2>(p, epi, vec, s);
    }
}

}  // namespace ll
