// 16-bit-input GEMM with FP32 accumulation and FP32 output on the CDNA4 matrix
// cores: C = alpha*A*B + beta*C with binary16 or bfloat16 A and B.
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
//     by (row/2)%8, so 16 lanes reading the same logical chunk of 16 rows hit
//     16 different 16-byte groups of the 64 banks.
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
    static constexpr int BT_PT = BN * CPR / NT;          // B given N-by-K: chunks per thread
    static_assert(BK == 64, "LDS rows are 128 bytes");
    static_assert(BT_PT >= 1 && BT_PT * NT == BN * CPR, "B^T chunks must split evenly");
    static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");
    static_assert(A_PT >= 1 && A_PT * NT == A_CH, "A chunks must split evenly");
};

__device__ __forceinline__ uint16_t ld_u16(const uint16_t *p) { return *p; }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// The MFMA for the 16-bit input format: binary16 or bfloat16 operands,
// 8 k-values per lane, FP32 accumulation. The operands are handled as raw
// 16-bit patterns everywhere else.
template <bool BF16>
__device__ __forceinline__ f32x16 mma16(const f16x8 &a, const f16x8 &b, const f32x16 &c)
{
    if (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The 16x16x32 form: the same 8 k-values per lane (lane l: row or column
// l%16, k = 8*(l/16) .. +7), a 16x16 block in four accumulators per lane.
template <bool BF16>
__device__ __forceinline__ f32x4 mma16(const f16x8 &a, const f16x8 &b, const f32x4 &c)
{
    if (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int MF> struct AccBlock { using type = f32x16; static constexpr int R = 16; };
template <> struct AccBlock<16> { using type = f32x4; static constexpr int R = 4; };

// BT: B is given N-by-K (k contiguous); it is then loaded and stored exactly
// like A and needs no transposition.
template <class T, int EPI, int WPE, bool BF16, bool BT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
gemm_f16_kernel(GemmParams p)
{
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK;
    constexpr int FM = T::FM, FN = T::FN, CPR = T::CPR;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    select_batch(p);
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    int K;
    const int kb = split_range(p, K);
    const uint16_t *__restrict__ A = static_cast<const uint16_t *>(p.A) + kb;
    const uint16_t *__restrict__ B =
        static_cast<const uint16_t *>(p.B) + (BT ? (int64_t)kb : (int64_t)kb * p.ldb);
    const int M = p.M, N = p.N;

    // A chunk i of this thread: row a_r0 + i*A_RSTEP, 16-byte chunk a_c; with
    // BT the same mapping over B's rows (n).
    const int a_c = tid % CPR;
    const int a_r0 = tid / CPR;
    constexpr int A_RSTEP = T::NT / CPR;
    const uint16_t *a_ptr = A + (int64_t)(m0 + a_r0) * p.lda + a_c * 8;
    const int64_t a_istep = (int64_t)A_RSTEP * p.lda;
    const uint16_t *bt_ptr = B + (int64_t)(n0 + a_r0) * p.ldb + a_c * 8;
    const int64_t bt_istep = (int64_t)A_RSTEP * p.ldb;
    u32x4 rbt[BT ? T::BT_PT : 1];

    // k-contiguous rows (A, or B given N-by-K): chunk i of this thread.
    auto load_rows = [&](const uint16_t *ptr, int64_t istep, int first, int nrows, int npt,
                         u32x4 *dst, int k0) {
        for (int i = 0; i < npt; ++i) {
            const bool rok = first + a_r0 + i * A_RSTEP < nrows;
            const int kk = k0 + a_c * 8;
            const uint16_t *src = ptr + i * istep + k0;
            // whole chunks at any alignment; the chunk that crosses K
            // element by element
            u32x4 v = {0u, 0u, 0u, 0u};
            if (rok && kk + 8 <= K) {
                v = load16<u32x4>(src);
            } else if (rok && kk < K) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t lo = kk + 2 * j < K ? ld_u16(src + 2 * j) : 0u;
                    const uint32_t hi = kk + 2 * j + 1 < K ? ld_u16(src + 2 * j + 1) : 0u;
                    v[j] = lo | (hi << 16);
                }
            }
            dst[i] = v;
        }
    };

    // B block i of this thread: id = i*NT + tid; k-block id % (BK/8) (so the
    // eight lanes of a group write eight different k-chunks of one LDS row),
    // n-block id / (BK/8).
    u32x4 ra[T::A_PT];
    u32x4 rb[T::B_PT][8];

    auto gload = [&](int k0) {
        load_rows(a_ptr, a_istep, m0, M, T::A_PT, ra, k0);
        if (BT) {
            load_rows(bt_ptr, bt_istep, n0, N, T::BT_PT, rbt, k0);
            return;
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
                u32x4 v = {0u, 0u, 0u, 0u};
                if (active && kk < K && nn + 8 <= N) {
                    v = load16<u32x4>(src);
                } else if (active && kk < K && nn < N) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t lo = nn + 2 * d < N ? ld_u16(src + 2 * d) : 0u;
                        const uint32_t hi = nn + 2 * d + 1 < N ? ld_u16(src + 2 * d + 1) : 0u;
                        v[d] = lo | (hi << 16);
                    }
                }
                rb[i][j] = v;
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
        if (BT) {
#pragma unroll
            for (int i = 0; i < (BT ? T::BT_PT : 1); ++i) {
                const int row = a_r0 + i * A_RSTEP;
                const int c = a_c ^ swz<BK * 2>(row);
                *reinterpret_cast<u32x4 *>(&Bs[buf][row * BK + c * 8]) = rbt[i];
            }
            return;
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
    const int nk = cdiv(K, BK);

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
                    acc[fm][fn] = mma16<BF16>(af[fm], bf[fn], acc[fm][fn]);
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


// ---------------------------------------------------------------------------
// Direct-to-LDS FP16 kernel (BM x BN = 256x256, 192x192 or 128x128 block
// tile, 128-bit-aligned operands).
//
// Both operands travel global -> LDS with global_load_lds_dwordx4, so no
// registers hold prefetched tiles and the accumulators (128 per lane for a
// 128x64 wave block) leave room for two register sets of MFMA operands.
//
// The inner product runs on v_mfma_f32_16x16x32 (MF = 16; MF = 32 selects
// v_mfma_f32_32x32x16, the same 8 k-values per lane over half the k-step).
// Both reach the same peak rate, but in a register-only loop over changing
// operands on all CUs the 16x16 form sustained about 1.5x the 32x32 one (the
// chip holds a higher clock), and in this kernel it measured 3-10 % faster.
//
// B keeps its row-major [k][n] layout in LDS; the MFMA's B operand (8
// consecutive k of one column per lane) is read with ds_read_b64_tr_b16, gfx950's transposing LDS load: within each
// group of 16 lanes, lane i receives element i%4 of the 8-byte rows that lanes
// i/4, 4+i/4, 8+i/4 and 12+i/4 address. If lane j points at
// B[kb + j/4][nb + 4*(j%4)], lane i therefore receives B[kb .. kb+3][nb + i].
//
// LDS, per stage of BK k-values (CPR = BK/8 16-byte chunks per A row):
//   A: BM rows x 2*BK bytes; chunks XOR-swizzled by (row / (16/CPR)) % CPR,
//      so the 16 lanes one LDS cycle serves (16 consecutive rows, one logical
//      chunk) hit 16 different 16-byte bank groups (measured conflict-free).
//      One copy (KiB) = 64/CPR rows; lane l fills row l/CPR, slot l%CPR, and
//      fetches the logical chunk that the swizzle puts in that slot.
//   B: BK rows x 2*BN bytes; 32-byte units XOR-swizzled per k-row. A
//      transposing read is served 32 lanes (256 bytes) per LDS cycle: two
//      16-lane groups, each reading one 32-byte unit of four k-rows.
//      MF = 32: the groups read units u and u+1 (u even) of the same rows;
//      XOR by 2*(k%4) sends the even group to units u^{0,2,4,6} and the odd
//      one to the odd units between, eight different 32-byte slots of the
//      256-byte bank line (XOR by k%4 would put both groups on units u..u+3:
//      a two-way conflict, measured).
//      MF = 16: the groups read the same unit u of rows k..k+3 and k+8..k+11;
//      XOR by 2*(k%4) + (k/8)%2 sends them to u^{0,2,4,6} and u^{1,3,5,7}.
//      (With BN = 128 a k-row is one bank line; with 256 the XOR stays in
//      its half; with 192 it stays in the first eight units or, within the
//      last four, uses the low two bits.) The stage is filled as one byte
//      array, 1 KiB per copy: lane l of copy c fills bytes 1024*c + 16*l,
//      which is k-row (1024*c + 16*l) / (2*BN). With BN = 192 a copy ends
//      inside a k-row; each wave's three copies cover eight whole k-rows.
// NBUF stages form a ring. A stage holds BK/32 k-steps (BK/16 with MF = 32);
// each step's operands are read while the previous step's MFMAs run. The
// stage's barrier sits before its last step, whose operands are then in
// registers: it publishes stage kt+1 and frees stage kt's buffer, which is
// refilled at once with stage kt+NBUF while the last step's MFMAs run (a few
// copies after each of the first rows of MFMAs, not one burst the matrix
// cores would wait through). The first operands of stage kt+1 are read
// during those MFMAs too, so no LDS latency is exposed after a barrier.
//
// With BT (B given N-by-K, k contiguous) B is copied and read exactly like A:
// BN rows x 2*BK bytes, the same swizzle, 128-bit operand reads, no
// transposing loads.
//
// The workgroup is a WGM x WGN grid of waves, each owning a (BM/WGM) x
// (BN/WGN) block, with WPE waves per SIMD: 256x256 runs 2 x 4 waves, two per
// SIMD, so one wave's MFMAs can run while the other waits to issue its
// copies; 192x192 runs the same 2 x 4 grid (96x48 per wave); 128x128 runs
// 2 x 2 waves and two workgroups per CU.
//
// SK: a stream-K launch (whole tiles first, then sharing workgroups that add
// partial sums of (tile, k-range) segments atomically).
//
// KS: K-slices. The workgroup holds KS wave grids; slice s runs the pipeline
// on its own LDS ring over the s-th of KS stage-aligned parts of the tile's
// K range (all slices run the same number of stages and share every
// barrier); at the end the other slices park their partial tiles in the A
// rings and slice 0 adds them in slice order and writes the tile.
//
// IN (interior): launched only when every tile lies inside M and N and every
// workgroup's (and slice's) K range is a whole number of stages; the copies
// then need no bounds selects.
template <int EPI, bool BF16, bool BT, int BM, int BN, int BK, int NBUF, int WGM, int WGN, int WPE,
          bool IN, int MF, bool SK, int KS>
__global__ void __launch_bounds__(64 * WGM * WGN * KS) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
gemm_f16_direct_kernel(GemmParams p)
{
    constexpr int NW = WGM * WGN;   // waves of one K-slice
    static_assert(BM == BN && (BN == 128 || BN == 192 || BN == 256), "square tiles of 128, 192 or 256");
    constexpr int WTM = BM / WGM, WTN = BN / WGN, FM = WTM / MF, FN = WTN / MF;
    constexpr int KSTEP = MF == 32 ? 16 : 32;             // k per MFMA
    constexpr int STEPS = BK / KSTEP;                     // MFMA k-steps per stage
    constexpr int CPR = BK / 8;                           // 16-byte chunks per A row
    constexpr int RPC = 64 / CPR;                         // A rows per copy
    constexpr int A_STAGE = BM * BK, B_STAGE = BK * BN;   // halves
    constexpr int COPIES_A = BM / RPC / NW;               // per wave per stage
    constexpr int COPIES_B = BT ? COPIES_A : B_STAGE * 2 / 1024 / NW;
    constexpr int PER_STAGE = COPIES_A + COPIES_B;        // vmcnt entries per stage
    static_assert(STEPS % 2 == 0 && PER_STAGE % FM == 0, "stage layout");
    static_assert(COPIES_A * RPC * NW == BM && RPC % 8 == 0 &&
                      (BT || COPIES_B * 1024 * NW == B_STAGE * 2) && WTM % MF == 0 &&
                      WTN % MF == 0 && (MF == 16 || MF == 32),
                  "copies cover the stage; a copy's rows start at a multiple of 8");
    static_assert((NBUF - 1) * PER_STAGE <= 63, "vmcnt range");
    static_assert(KS >= 1 && (KS == 1 || !SK), "K-slices take no stream-K share");
    static_assert((KS - 1) * NW * FM * FN * AccBlock<MF>::R * 64 * 4 <= KS * NBUF * A_STAGE * 2,
                  "slice partials fit in the A rings");
    __shared__ __attribute__((aligned(1024))) uint16_t As[KS][NBUF][A_STAGE];
    __shared__ __attribute__((aligned(1024))) uint16_t Bs[KS][NBUF][B_STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_wg = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slice = wave_wg / NW, wave = wave_wg % NW;   // wave within the slice
    const int wm = wave / WGN, wn = wave % WGN;
    select_batch(p);
    // One tile per workgroup, or (a stream-K launch's sharing workgroups, from
    // sk_block on) up to two (tile, k-range) segments, each a complete pass of
    // the pipeline below whose partial sums are added atomically.
    const bool sharing = SK && (int)blockIdx.x >= p.sk_block;
    for (int seg = 0;; ++seg) {
    int tm, tn, K, kb;
    if (sharing) {
        if (!sk_segment(p, seg, tm, tn, kb, K))
            break;
        if (seg > 0)
            __syncthreads();   // every wave is done with the previous segment's LDS
    } else {
        if (seg > 0)
            break;
        tile_coords(p, tm, tn);
        kb = split_range(p, K);
    }
    // This slice's part of the K range; every slice runs k_steps k-values.
    int k_steps = K;
    if (KS > 1) {
        k_steps = cdiv(cdiv(K, KS), BK) * BK;
        const int lo = slice * k_steps;
        kb += lo < K ? lo : K;
        K = K - lo < k_steps ? (K - lo > 0 ? K - lo : 0) : k_steps;
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const uint16_t *__restrict__ A = static_cast<const uint16_t *>(p.A) + kb;
    const uint16_t *__restrict__ B =
        static_cast<const uint16_t *>(p.B) + (BT ? (int64_t)kb : (int64_t)kb * p.ldb);
    const int M = p.M, N = p.N;
    auto swz = [](int row) { return (row / (16 / CPR)) & (CPR - 1); };
    // B (K-by-N) unit swizzle of k-row k (see the layout notes above).
    auto bsw = [](int k) { return MF == 32 ? 2 * (k & 3) : 2 * (k & 3) + ((k >> 3) & 1); };
    // Unit u of k-row k is stored in slot bunit(u, k): the XOR acts within
    // groups of eight units (a 256-byte bank line), and within the last group
    // of four when BN = 192.
    auto bunit = [&](int u, int k) {
        if constexpr (BN % 128 == 0) {
            return u ^ bsw(k);
        } else {
            constexpr int NU = BN / 16;
            const int g = u & ~7, span = NU - g < 8 ? NU - g : 8;
            return g + ((u & 7) ^ (bsw(k) & (span - 1)));
        }
    };

    // Copy sources. Row-panel copy j of this wave (A, or B given N-by-K)
    // covers rows (wave*COPIES_A + j)*RPC + lane/CPR. A copy's first row is a
    // multiple of 8, so the swizzled chunk a lane fetches depends only on
    // whether that row is a multiple of 16: two variants.
    const int r_lane = wave * COPIES_A * RPC + lane / CPR;   // row of copy 0
    const int slot = lane % CPR;
    int ch[2];
    const uint16_t *a_src[2], *bt_src[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        ch[v] = slot ^ swz(((v * RPC) & 15) + lane / CPR);
        a_src[v] = A + (int64_t)(m0 + r_lane) * p.lda + ch[v] * 8;
        bt_src[v] = B + (int64_t)(n0 + r_lane) * p.ldb + ch[v] * 8;
    }
    // B copy j (given K-by-N) fills stage bytes (wave*COPIES_B + j)*1024 +
    // 16*lane: k-row b_row(j), unit slot s = (offset within the row)/32, half
    // (offset/16)%2, holding logical unit bunit(s, k) (an involution).
    auto b_off = [&](int j) { return (wave * COPIES_B + j) * 1024 + 16 * lane; };
    auto b_row = [&](int j) { return b_off(j) / (2 * BN); };
    constexpr int NB_SRC = BT ? 1 : COPIES_B;
    const uint16_t *b_src[NB_SRC];
    bool b_col_ok[NB_SRC];
#pragma unroll
    for (int j = 0; j < NB_SRC; ++j) {
        const int kr = b_row(j), u2 = (b_off(j) % (2 * BN)) / 16;
        const int col = n0 + bunit(u2 >> 1, kr) * 16 + (u2 & 1) * 8;
        b_src[j] = B + (int64_t)kr * p.ldb + col;
        b_col_ok[j] = col < N;
    }
    const uint32_t as_base = lds_addr(&As[slice][0][0]), bs_base = lds_addr(&Bs[slice][0][0]);

    // Copy c (A: 0 .. COPIES_A-1, then B) of the stage at k0 into buffer buf.
    // Every copy is one global_load_lds on every lane: lanes whose 16 bytes
    // lie outside A or B read the zero chunk instead, so each stage is exactly
    // PER_STAGE copies per wave and the vmcnt waits below count exactly.
    auto copy = [&](int buf, int k0, int c) {
        const uint16_t *src;
        uint32_t dst;
        if (c < COPIES_A || BT) {
            const bool is_a = c < COPIES_A;
            const int j = is_a ? c : c - COPIES_A;
            // (each wave's first row is a multiple of 16 unless BM = 192)
            const int v = (((COPIES_A * RPC) % 16 == 0 ? j : wave * COPIES_A + j) * RPC & 15) != 0;
            dst = (is_a ? as_base + buf * (A_STAGE * 2) : bs_base + buf * (B_STAGE * 2)) +
                  (wave * COPIES_A + j) * 1024;
            const int64_t step = (int64_t)(j * RPC) * (is_a ? p.lda : p.ldb) + k0;
            const uint16_t *in = (is_a ? a_src[v] : bt_src[v]) + step;
            if constexpr (IN) {
                src = in;
            } else {
                const bool ok = r_lane + j * RPC < (is_a ? M - m0 : N - n0) && k0 + ch[v] * 8 < K;
                src = ok ? in : zero_chunk<uint16_t>();
            }
        } else {
            const int j = c - COPIES_A;
            dst = bs_base + buf * (B_STAGE * 2) + (wave * COPIES_B + j) * 1024;
            const uint16_t *in = b_src[j] + (int64_t)k0 * p.ldb;
            if constexpr (IN)
                src = in;
            else
                src = k0 + b_row(j) < K && b_col_ok[j]
                          ? in
                          : zero_chunk<uint16_t>();
        }
        lds_dma_16(src, dst);
    };

    using Acc = typename AccBlock<MF>::type;
    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < AccBlock<MF>::R; ++r)
                acc[i][j][r] = 0.0f;

    // Lane l supplies row (or column) l % MF of its block and k-values
    // 8*(l/MF) .. +7 of the k-step.
    const int grp = lane / MF, lrow = lane % MF;
    const int g_lo = (lane >> 4) & 1, j16 = lane & 15;
    typedef short s16x4 __attribute__((ext_vector_type(4)));

    // Operands of k-step s (k = KSTEP*s + 8*grp + 0..7) of the stage in buffer buf.
    auto read_step = [&](int buf, int s, f16x8 (&af)[FM], f16x8 (&bf)[FN]) {
        const uint16_t *as = As[slice][buf];
        const uint16_t *bs = Bs[slice][buf];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int row = wm * WTM + fm * MF + lrow;
            const int c = (KSTEP / 8 * s + grp) ^ swz(row);
            af[fm] = *reinterpret_cast<const f16x8 *>(&as[row * BK + c * 8]);
        }
        if (BT) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int row = wn * WTN + fn * MF + lrow;
                const int c = (KSTEP / 8 * s + grp) ^ swz(row);
                bf[fn] = *reinterpret_cast<const f16x8 *>(&bs[row * BK + c * 8]);
            }
            return;
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            // 16 columns per 16-lane group: a 32-wide block splits them over
            // the two groups of a half-wave, a 16-wide one repeats them
            const int n = wn * WTN + fn * MF + (MF == 32 ? g_lo * 16 : 0) + 4 * (j16 & 3);
            s16x4 v[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int k = KSTEP * s + 8 * grp + 4 * e + (j16 >> 2);
                const int addr = k * BN + (bunit(n >> 4, k) << 4) + (n & 15);
                v[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(lds_addr(&bs[addr])));
            }
            const s16x4 lo = v[0], hi = v[1];
            bf[fn] = __builtin_bit_cast(f16x8, (short __attribute__((ext_vector_type(8)))){
                lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
    };
    // The MFMA groups raise the wave's issue priority (s_setprio), so a wave
    // with MFMAs ready wins the arbitration over its SIMD's other wave while
    // that one issues reads and copies (measured about +1 %). They walk the
    // blocks row by row in alternating column order, so that consecutive
    // MFMAs always share an operand: fewer operand bits change from one to
    // the next, and the chip, power-limited at this precision, keeps a higher
    // clock (8192^3: +1.3 to 1.6 % fp16, +0.8 to 1.2 % bf16, bit-identical
    // results; columns outermost instead measured no gain).
    auto mfma_step = [&](const f16x8 (&af)[FM], const f16x8 (&bf)[FN]) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int fn = (fm & 1) ? FN - 1 - j : j;
                acc[fm][fn] = mma16<BF16>(af[fm], bf[fn], acc[fm][fn]);
            }
        __builtin_amdgcn_s_setprio(0);
    };

    // Wait until at most n stages of copies are still in flight.
    auto wait_stages = [&](int n) {
        if (n >= 3)
            __builtin_amdgcn_s_waitcnt(LL_VMCNT(3 * PER_STAGE > 63 ? 63 : 3 * PER_STAGE));
        else if (n == 2)
            __builtin_amdgcn_s_waitcnt(LL_VMCNT(2 * PER_STAGE > 63 ? 63 : 2 * PER_STAGE));
        else if (n == 1)
            __builtin_amdgcn_s_waitcnt(LL_VMCNT(PER_STAGE));
        else
            __builtin_amdgcn_s_waitcnt(LL_VMCNT(0));
    };
    static_assert(NBUF - 1 <= 3, "wait_stages covers at most three stages in flight");

    const int nk = cdiv(k_steps, BK);   // the same in every slice
    for (int st = 0; st < NBUF; ++st)
        if (st < nk) {
#pragma unroll
            for (int c = 0; c < PER_STAGE; ++c)
                copy(st, st * BK, c);
        }
    wait_stages((nk < NBUF ? nk : NBUF) - 1);   // stage 0 has landed
    __syncthreads();

    f16x8 fa[2][FM], fb[2][FN];   // operands of two consecutive k-steps
    read_step(0, 0, fa[0], fb[0]);
    int buf = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const int nbuf = buf == NBUF - 1 ? 0 : buf + 1;
#pragma unroll
        for (int s = 0; s + 1 < STEPS; ++s) {
            read_step(buf, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
            mfma_step(fa[s & 1], fb[s & 1]);
        }
        if (kt + 1 < nk) {
            // stage kt+1 has landed (stages up to kt+NBUF-1 were issued); after
            // the barrier every wave is done with this stage's buffer
            wait_stages((kt + NBUF - 1 < nk ? kt + NBUF - 1 : nk - 1) - (kt + 1));
            __syncthreads();
        }
        const int k_next = (kt + NBUF) * BK;   // refill this buffer with stage kt+NBUF
        const bool refill = kt + NBUF < nk;
        // First operands of stage kt+1. Read unconditionally (after the last
        // stage they are stale, in-bounds and unused) so that no control-flow
        // join makes the compiler's LDS wait counts conservative.
        read_step(nbuf, 0, fa[0], fb[0]);
        // The refill copies follow the first CROWS rows of MFMAs, G after
        // each. 16x16 blocks (eight rows of four 16-cycle MFMAs): two rows
        // measured 2-4 % faster than one row per copy pair or than all
        // copies before the first MFMA; one, four, or two rows starting one
        // row later all came within 1 % of it.
        constexpr int CROWS = MF == 16 ? 2 : FM;
        constexpr int G = PER_STAGE / CROWS;
        static_assert(PER_STAGE % CROWS == 0 && CROWS <= FM, "refill placement");
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {   // the same alternating order
                const int fn = (fm & 1) ? FN - 1 - j : j;
                acc[fm][fn] = mma16<BF16>(fa[1][fm], fb[1][fn], acc[fm][fn]);
            }
            if (refill && fm < CROWS) {
#pragma unroll
                for (int g = 0; g < G; ++g)
                    copy(buf, k_next, fm * G + g);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        buf = nbuf;
    }

    if constexpr (KS > 1) {
        // Slices 1.. park their partial tiles in the (now idle) A rings, one
        // float per lane per slot, then slice 0 adds them in slice order.
        float *part = reinterpret_cast<float *>(&As[0][0][0]);
        constexpr int R = AccBlock<MF>::R, SLOTS = FM * FN * R;
        __syncthreads();   // every slice is done reading its ring
        if (slice > 0) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        part[((((slice - 1) * NW + wave) * SLOTS) + (fm * FN + fn) * R + r) * 64 + lane] =
                            acc[fm][fn][r];
        }
        __syncthreads();
        if (slice > 0)
            return;   // no barrier follows
        for (int sl = 1; sl < KS; ++sl)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[fm][fn][r] +=
                            part[((((sl - 1) * NW + wave) * SLOTS) + (fm * FN + fn) * R + r) * 64 + lane];
    }

#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int r0 = m0 + wm * WTM + fm * MF, c0 = n0 + wn * WTN + fn * MF;
            if constexpr (MF == 32) {
                if (sharing)
                    write_block<EPI_ATOMIC>(p, acc[fm][fn], r0, c0, lane);
                else
                    write_block<EPI>(p, acc[fm][fn], r0, c0, lane);
            } else {
                if (sharing)
                    write_block16<EPI_ATOMIC>(p, acc[fm][fn], r0, c0, lane);
                else
                    write_block16<EPI>(p, acc[fm][fn], r0, c0, lane);
            }
        }
    }
}

// Stage depth and ring length of the direct kernel. At BK = 64 a row panel's
// copies read whole 128-byte lines and a stage holds four k-steps under one
// barrier; two 64 KiB stages measured 6-10 % faster than four 32 KiB ones
// (BK = 32) for both B layouts on 4096- and 8192-cubed products.
// Wave grid, per B layout: 2 x 4 (eight waves, two per SIMD, 128x64 each)
// measured faster than 2 x 2 (one wave per SIMD) and 4 x 2, in one process:
// with 32x32 blocks 8192^3 fp16 1079 -> 1168 TFLOP/s, bf16 1114 -> 1234,
// B given N-by-K 1171 -> 1191; with 16x16 blocks (2 x 2 then keeps its
// accumulators in AGPRs without spills) 1084 -> 1244 for fp16. A wave that
// waits to issue a copy no longer idles its SIMD's matrix core.
template <int BM> struct DirectCfg {
    static constexpr int BK = 64, NBUF = 2;
    static constexpr int WGM = 2, WGN = 4, WPE = 2;
    static constexpr int MF = 16;
};
// 128x128: four waves of 64x64 and 64 KiB of LDS, so two workgroups share a
// CU (two waves per SIMD, as with one 256x256 workgroup).
template <> struct DirectCfg<128> {
    static constexpr int BK = 64, NBUF = 2;
    static constexpr int WGM = 2, WGN = 2, WPE = 2;
    static constexpr int MF = 16;
};

using F16_L = F16Tile<256, 256, 64>;
using F16_S = F16Tile<128, 128, 64>;
using F16_XS = F16Tile<64, 64, 64>;

template <class T, int WPE, bool BF16, bool BT>
static hipError_t launch_t(const GemmParams &p0, int epi, bool vec, hipStream_t s)
{
    GemmParams p = p0;
    p.tiles_m = cdiv(p.M, T::BM);
    p.tiles_n = cdiv(p.N, T::BN);
    const int64_t ntiles = (int64_t)p.tiles_m * p.tiles_n;
    if (ntiles > kMaxTiles || p.batch < 1 || p.batch > kMaxGridZ || p.grid_x != 0 || p.sk_tiles != 0)
        return hipErrorInvalidValue;   // the register-staged kernels run whole grids only
    const dim3 grid = gemm_grid(p, ntiles), block(T::NT);
#define LL_F16_LAUNCH(E) \
    hipLaunchKernelGGL((gemm_f16_kernel<T, E, WPE, BF16, BT>), grid, block, 0, s, p)
    // 16-byte chunk loads at any alignment, the chunk that crosses K or N
    // element by element
    if (epi == EPI_GEMM_BETA0) LL_F16_LAUNCH(EPI_GEMM_BETA0);
    else if (epi == EPI_GEMM_BETA) LL_F16_LAUNCH(EPI_GEMM_BETA);
    else LL_F16_LAUNCH(EPI_ATOMIC);
#undef LL_F16_LAUNCH
    return hipGetLastError();
}

// Skinny 16-bit products with B given N-by-K (a few rows of A: memory-bound,
// so no MFMAs, which would compute a whole block of rows for every row). The
// inner product runs on dot2 instructions: two 16-bit products added into an
// FP32 sum per lane and instruction, the precision of the MFMA path. A
// workgroup of four waves covers 256 columns of C over its K range (a
// K-split), A's rows MR at a time (MR = 1, 2, 4, 8 or 16). The A block of the K
// range is staged raw in LDS (H16_XS values; the planner keeps the range
// within H16_XS / MR k-values, and a longer one, from a forced plan, is
// walked in chunks of that size). Wave w covers columns 64w .. 64w+63 in 16
// groups of four; in a group, lane l reads column 4g + l/16's row of B at
// k-values 8(l%16) + 128j, so one 16-byte load per lane covers 128
// consecutive k of four rows; the 16 lanes of a row add their sums by DPP and
// the result goes to an LDS row block of C, stored once at the end. Loads of
// B take whole 16-byte chunks at any alignment, the chunk that crosses K
// element by element.
constexpr int H16_COLS = 256;     // columns of C per workgroup
constexpr int H16_XS = 16384;     // LDS values for the staged A block (32 KiB)

template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    if constexpr (BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

// 16-bit values k .. k+7 of a row (zero from kn on) as one 16-byte chunk.
__device__ __forceinline__ u32x4 h16_chunk(const uint16_t *src, int k, int kn)
{
    if (k + 8 <= kn)
        return load16<u32x4>(src);
    uint16_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        h[j] = k + j < kn ? src[j] : (uint16_t)0;
    return __builtin_bit_cast(u32x4, h);
}

template <int EPI, bool BF16, int MR>
__global__ void __launch_bounds__(256) gemm_h16_skinny_nt_kernel(GemmParams p)
{
    constexpr int KC = H16_XS / MR;   // k-values staged at once (a multiple of 128)
    constexpr int D = MR == 16 ? 2 : 8;   // loads in flight per lane
    __shared__ __attribute__((aligned(16))) uint16_t xs[H16_XS];
    __shared__ float ys[MR * H16_COLS];   // this row block of C
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    select_batch(p);
    int K;
    const int kb = split_range(p, K);
    const uint16_t *__restrict__ A = static_cast<const uint16_t *>(p.A) + kb;
    const uint16_t *__restrict__ B = static_cast<const uint16_t *>(p.B) + kb;
    const int M = p.M, N = p.N;
    const int nblk = blockIdx.x * H16_COLS;
    const int c8 = 8 * (lane & 15), rg = lane >> 4;

    // 64-bit chunk counters and row checks: M or K may lie within one chunk of 2^31
    for (int64_t mc = 0; mc < M; mc += MR) {
        for (int i = tid; i < MR * H16_COLS; i += 256)
            ys[i] = 0.0f;
        for (int64_t kc = 0; kc < K; kc += KC) {
            const int kn = K - kc < KC ? (int)(K - kc) : KC;
            __syncthreads();   // the previous chunk's (or row block's) A values are read
            // rows mc .. mc+MR-1 (zero past M), k-values kc .. kc+kn-1 (zero up
            // to kn rounded up to 128)
            const int kq = ((kn + 127) & ~127) / 8;   // 16-byte chunks per row
            for (int i = tid; i < MR * kq; i += 256) {
                const int m = i / kq, k = (i % kq) * 8;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (mc + m < M)
                    v = h16_chunk(A + (mc + m) * p.lda + kc + k, k, kn);
                *reinterpret_cast<u32x4 *>(xs + m * KC + k) = v;
            }
            __syncthreads();
            const int steps = (kn + 127) / 128;   // 128 k-values of a row per load
            const int total = 16 * steps;         // (group, step) pairs of this wave
            auto fetch = [&](int t) -> u32x4 {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (t >= total)
                    return v;
                const int g = t / steps, k = (t - g * steps) * 128 + c8;
                const int col = nblk + 64 * wave + 4 * g + rg;
                if (col >= N)
                    return v;
                return h16_chunk(B + (int64_t)col * p.ldb + kc + k, k, kn);
            };
            u32x4 w[D];
#pragma unroll
            for (int d = 0; d < D; ++d)
                w[d] = fetch(d);
            float acc[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m)
                acc[m] = 0.0f;
            int g = 0, st = 0;
            for (int tb = 0; tb < total; tb += D) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    if (tb + d < total) {
                        const int k0 = st * 128 + c8;   // within KC: KC is a multiple of 128
#pragma unroll
                        for (int m = 0; m < MR; ++m) {
                            const u32x4 x = *reinterpret_cast<const u32x4 *>(xs + m * KC + k0);
                            float a = acc[m];
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                a = dot2<BF16>(x[j], w[d][j], a);
                            acc[m] = a;
                        }
                        w[d] = fetch(tb + d + D);
                        if (++st == steps) {
                            // group g done: the 16 lanes of each row add up, lane 0 of the
                            // row adds the sums into the C row block
#pragma unroll
                            for (int m = 0; m < MR; ++m) {
                                const float v = dpp_row_sum16(acc[m]);
                                if ((lane & 15) == 0)
                                    ys[m * H16_COLS + 64 * wave + 4 * g + rg] += v;
                                acc[m] = 0.0f;
                            }
                            st = 0;
                            ++g;
                        }
                    }
                }
            }
        }
        __syncthreads();   // every wave's groups are in ys
        const int col = nblk + tid;
        if (col < N) {
#pragma unroll
            for (int m = 0; m < MR; ++m)
                if (mc + m < M)
                    skinny_store<EPI>(p, (int)mc + m, col, ys[m * H16_COLS + tid]);
        }
        __syncthreads();   // ys is read before the next row block clears it
    }
}

template <bool BF16>
static hipError_t launch_skinny16(const GemmParams &p0, int epi, hipStream_t s)
{
    static_assert(H16_COLS == kSkinnyCols && H16_XS == kSkinny16Stage, "skinny kernel shape");
    GemmParams p = p0;
    p.tiles_m = 1;
    p.tiles_n = cdiv(p.N, H16_COLS);
    if (p.batch < 1 || p.batch > kMaxGridZ || p.grid_x != 0 || p.sk_tiles != 0)
        return hipErrorInvalidValue;   // whole grids only, no stream-K
    const dim3 grid = gemm_grid(p, p.tiles_n), block(256);
    const int mr = skinny_rows(p.M);
#define LL_SKINNY_MR(E, MR) hipLaunchKernelGGL((gemm_h16_skinny_nt_kernel<E, BF16, MR>), grid, block, 0, s, p)
#define LL_SKINNY(E) \
    do { \
        if (mr == 1) LL_SKINNY_MR(E, 1); \
        else if (mr == 2) LL_SKINNY_MR(E, 2); \
        else if (mr == 4) LL_SKINNY_MR(E, 4); \
        else if (mr == 8) LL_SKINNY_MR(E, 8); \
        else LL_SKINNY_MR(E, 16); \
    } while (0)
    if (epi == EPI_GEMM_BETA0) LL_SKINNY(EPI_GEMM_BETA0);
    else if (epi == EPI_GEMM_BETA) LL_SKINNY(EPI_GEMM_BETA);
    else LL_SKINNY(EPI_ATOMIC);
#undef LL_SKINNY
#undef LL_SKINNY_MR
    return hipGetLastError();
}

// {BM, BN, workgroups per CU, relative throughput alone, paired} (see the
// FP32 table), against the 256x256 kernel's 4096^3 rate. 128x128 (direct):
// paired 0.91 on 8192^3 and 0.86 on 4096^3; alone 0.50 on 2048^3 and 0.62
// with K = 8192, entered as 0.45 so that a last half round of lone 128x128
// workgroups (6144^3: 4.5 rounds, 1048 TFLOP/s) loses to 256x256 with
// stream-K (1140). 64x64 (register-staged): about 0.20 paired, 0.10 alone
// (1024^3). 128x128 in two K-slices (one workgroup per CU): 0.56 on 2048^3,
// 0.76 with K = 8192, 0.62-0.73 on 4096^3-8192^3.
// Stream-K runs on the 256x256 tile only: on 128x128 tiles (3072^3, 5120^3,
// 6144^3) it lost to the best other plan by 4-10 %, its many short shared
// segments paying more per atomic byte.
const TileInfo kF16Tiles[kF16NumTiles] = {
    {F16_L::BM, F16_L::BN, 1, 1.00f, 1.00f, "f16_256x256_direct", 1, true,
     64 * DirectCfg<256>::WGM * DirectCfg<256>::WGN},
    {F16_S::BM, F16_S::BN, 2, 0.45f, 0.88f, "f16_128x128x64", 1, false},
    {F16_XS::BM, F16_XS::BN, 2, 0.10f, 0.20f, "f16_64x64x64", 1, false},
    // 128x128 in two K-slices (direct kernel only; the staged fallback runs
    // the plain tile): eight waves, one workgroup per CU; only with at least
    // 8 stages of 64 per slice (below, 0.5-1 us slower than plain 128x128)
    {F16_S::BM, F16_S::BN, 1, 0.60f, 0.60f, "f16_128x128_k2", 2, false, 512, 2 * 8 * 64, true},
    // 192x192 (direct kernel; unaligned operands run the staged 128x128):
    // eight waves, one workgroup per CU; 0.74 on 3072^3, 0.79 on 8192^3,
    // 0.85 on 4096^3. It wins where 256x256 leaves CUs idle and 192x192 does
    // not (3072^2: 256 tiles against 144).
    {192, 192, 1, 0.75f, 0.75f, "f16_192x192_direct", 1, false,
     64 * DirectCfg<192>::WGM * DirectCfg<192>::WGN, 0, true},
    // the skinny kernel (B given N-by-K; forced with B given K-by-N, the
    // 128x128 tile runs in its place): 16 rows of A at a time, 256 columns
    {16, H16_COLS, 2, 1.0f, 1.0f, "f16_16x256_skinny_nt", 1, false},
};

// The direct kernel on BM x BM tiles (KS K-slices) for 128-bit-aligned
// operands; otherwise the register-staged kernel of tile T, without slices
// (the same tile, except 128x128 for 192x192).
template <bool BF16, bool BT, int BM, class T, int WPE_T, int KS = 1>
static hipError_t launch_direct(const GemmParams &p0, int epi, bool vec, hipStream_t s)
{
    static_assert(T::BM == T::BN && (T::BM == BM || (BM == 192 && T::BM == 128)), "fallback tile");
    if (!vec)
        return launch_t<T, WPE_T, BF16, BT>(p0, epi, vec, s);
    GemmParams p = p0;
    p.tiles_m = cdiv(p.M, BM);
    p.tiles_n = cdiv(p.N, BM);
    int64_t ntiles = (int64_t)p.tiles_m * p.tiles_n;
    if (ntiles > kMaxTiles || p.batch < 1 || p.batch > kMaxGridZ)
        return hipErrorInvalidValue;
    if (p.grid_x > 0)
        ntiles = p.grid_x;   // a stream-K launch: whole tiles, then the sharing workgroups
    const bool sk = p.sk_tiles > 0;
    if (sk && (BM != 256 || KS != 1 || epi == EPI_ATOMIC || p.batch != 1))
        return hipErrorInvalidValue;   // stream-K: the 256x256 tile only
    using Cfg = DirectCfg<BM>;
    static_assert(kSkUnit % Cfg::BK == 0, "stream-K segments are whole stages");
    if (ntiles > max_grid_x(64 * Cfg::WGM * Cfg::WGN * KS))
        return hipErrorInvalidValue;
    const dim3 grid = gemm_grid(p, ntiles), block(64 * Cfg::WGM * Cfg::WGN * KS);
    // every copy inside the matrices: whole tiles, whole stages in every K range
    const int kq = KS * Cfg::BK;   // every slice's K range a whole number of stages
    const bool in = p.M % BM == 0 && p.N % BM == 0 && p.K % kq == 0 && p.k_split % kq == 0;
#define LL_DIRECT_K(E, IN, SK) \
    hipLaunchKernelGGL((gemm_f16_direct_kernel<E, BF16, BT, BM, BM, Cfg::BK, Cfg::NBUF, Cfg::WGM, \
                                               Cfg::WGN, Cfg::WPE, IN, Cfg::MF, SK, KS>), \
                       grid, block, 0, s, p)
#define LL_DIRECT(E, SK) \
    do { \
        if (in) \
            LL_DIRECT_K(E, true, SK); \
        else \
            LL_DIRECT_K(E, false, SK); \
    } while (0)
    if constexpr (BM == 256 && KS == 1) {
        if (sk) {
            // whole tiles with `epi`, shared ones added atomically
            if (epi == EPI_GEMM_BETA0)
                LL_DIRECT(EPI_GEMM_BETA0, true);
            else
                LL_DIRECT(EPI_GEMM_BETA, true);
            return hipGetLastError();
        }
    }
    if (epi == EPI_GEMM_BETA0) {
        LL_DIRECT(EPI_GEMM_BETA0, false);
    } else if (epi == EPI_GEMM_BETA) {
        LL_DIRECT(EPI_GEMM_BETA, false);
    } else {
        LL_DIRECT(EPI_ATOMIC, false);
    }
#undef LL_DIRECT
#undef LL_DIRECT_K
    return hipGetLastError();
}

template <bool BF16, bool BT>
static hipError_t launch_16(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s)
{
    switch (tile) {
    case 0: return launch_direct<BF16, BT, 256, F16_L, 1>(p, epi, vec, s);
    case 1: return launch_direct<BF16, BT, 128, F16_S, 2>(p, epi, vec, s);
    case 3: return launch_direct<BF16, BT, 128, F16_S, 2, 2>(p, epi, vec, s);
    case 4: return launch_direct<BF16, BT, 192, F16_S, 2>(p, epi, vec, s);
    case 5:
        if constexpr (BT)
            return launch_skinny16<BF16>(p, epi, s);
        else
            return launch_direct<BF16, BT, 128, F16_S, 2>(p, epi, vec, s);
    default: return launch_t<F16_XS, 2, BF16, BT>(p, epi, vec, s);
    }
}

hipError_t launch_gemm_f16(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s)
{
    return launch_16<false, false>(p, tile, epi, vec, s);
}

hipError_t launch_gemm_bf16(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s)
{
    return launch_16<true, false>(p, tile, epi, vec, s);
}

hipError_t launch_gemm_f16_bt(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s)
{
    return launch_16<false, true>(p, tile, epi, vec, s);
}

hipError_t launch_gemm_bf16_bt(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s)
{
    return launch_16<true, true>(p, tile, epi, vec, s);
}

}  // namespace ll
