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
//     reads and 16 lanes of consecutive rows hit 16 different 16-byte groups
//     of the 64 banks (the pages pad or transpose instead). B stays [k][n]; its rows are padded by 4 floats
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
    static constexpr int CPR = BK / 4;             // 16-byte chunks per k-contiguous row
    static constexpr int A_PT = BM * CPR / NT;     // A chunks per thread
    static constexpr int BCPR = BN / 4;            // 16-byte chunks per B k-row (B K-by-N)
    static constexpr int B_PT = BK * BCPR / NT;    // B chunks per thread (B K-by-N)
    static constexpr int BT_PT = BN * CPR / NT;    // B chunks per thread (B N-by-K)
    static constexpr int BNP = BN + 4;             // padded B k-row (floats)
    static constexpr int A_STAGE = BM * BK;        // floats
    static constexpr int B_STAGE = BK * BNP;       // >= BN * BK, fits either B layout
    static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");
    static_assert(A_PT >= 1 && A_PT * NT == BM * CPR, "A chunks must split evenly");
    static_assert(B_PT >= 1 && B_PT * NT == BK * BCPR, "B chunks must split evenly");
    static_assert(BT_PT >= 1 && BT_PT * NT == BN * CPR, "B^T chunks must split evenly");
    static_assert(KH % 4 == 0, "BK must be a multiple of 8");
};

// A panel of ROWS rows, each BK consecutive k of one row of a k-contiguous
// matrix (A, or B given N-by-K), staged through registers into a swizzled
// [row][k] LDS tile. Thread t owns chunks (t + i*NT): row (t + i*NT)/CPR,
// 16-byte chunk t%CPR.
template <class T, int ROWS>
struct RowPanel {
    static constexpr int CPR = T::CPR, BK = T::BK;
    static constexpr int PT = ROWS * CPR / T::NT;
    static constexpr int RSTEP = T::NT / CPR;
    const float *ptr;   // chunk 0 of this thread at k = 0
    int64_t istep;      // RSTEP rows
    int r0, c, row_base, rows;
    f32x4 reg[PT];

    __device__ void init(const float *base, int64_t ld, int first_row, int nrows, int tid)
    {
        c = tid % CPR;
        r0 = tid / CPR;
        row_base = first_row;
        rows = nrows;
        ptr = base + (int64_t)(first_row + r0) * ld + c * 4;
        istep = (int64_t)RSTEP * ld;
    }
    __device__ void load(int k0, int K)
    {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const bool rok = row_base + r0 + i * RSTEP < rows;
            const float *src = ptr + i * istep + k0;
            const int kk = k0 + c * 4;
            // whole chunks at any alignment; the chunk that crosses K
            // element by element
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (rok && kk + 4 <= K) {
                v = load16<f32x4>(src);
            } else if (rok && kk < K) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = kk + j < K ? src[j] : 0.0f;
            }
            reg[i] = v;
        }
    }
    __device__ void store(float *lds) const
    {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int row = r0 + i * RSTEP;
            *reinterpret_cast<f32x4 *>(&lds[row * BK + (c ^ swz<BK * 4>(row)) * 4]) = reg[i];
        }
    }
};

// The MFMA operand of one 32-row block: the lane's row, k = h*KH .. h*KH+KH-1,
// as KH/4 vectors read from a swizzled [row][k] tile.
template <class T>
__device__ __forceinline__ void read_rows(const float *lds, int row, int h, f32x4 (&dst)[T::KH / 4])
{
#pragma unroll
    for (int q = 0; q < T::KH / 4; ++q) {
        const int c = (h * (T::KH / 4) + q) ^ swz<T::BK * 4>(row);
        dst[q] = *reinterpret_cast<const f32x4 *>(&lds[row * T::BK + c * 4]);
    }
}

// BT = false: B is K-by-N (row-major, n contiguous); its k-rows go to LDS as
// [k][n] (rows padded by 4 floats) and each lane reads one float per MFMA step.
// BT = true: B is given N-by-K (k contiguous, e.g. a fully-connected weight
// stored [out][in]); it is staged exactly like A, as swizzled [n][k] rows, and
// read with 128-bit LDS loads like A.
template <class T, int EPI, int WPE, bool BT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
gemm_f32_kernel(GemmParams p)
{
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK, KH = T::KH;
    constexpr int FM = T::FM, FN = T::FN, BNP = T::BNP;
    __shared__ __attribute__((aligned(16))) float As[2][T::A_STAGE];
    __shared__ __attribute__((aligned(16))) float Bs[2][T::B_STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    select_batch(p);
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    int K;
    const int kb = split_range(p, K);
    const float *__restrict__ A = static_cast<const float *>(p.A) + kb;
    const float *__restrict__ B =
        static_cast<const float *>(p.B) + (BT ? (int64_t)kb : (int64_t)kb * p.ldb);
    const int M = p.M, N = p.N;

    RowPanel<T, BM> pa;
    pa.init(A, p.lda, m0, M, tid);
    RowPanel<T, BN> pbt;   // B given N-by-K
    // B given K-by-N: chunk i is k-row b_k0 + i*B_KSTEP, columns n0 + 4*b_c ..
    const int b_c = tid % T::BCPR;
    const int b_k0 = tid / T::BCPR;
    constexpr int B_KSTEP = T::NT / T::BCPR;
    const float *b_ptr = B + (int64_t)b_k0 * p.ldb + n0 + b_c * 4;
    const int64_t b_istep = (int64_t)B_KSTEP * p.ldb;
    f32x4 rb[BT ? 1 : T::B_PT];
    if (BT)
        pbt.init(B, p.ldb, n0, N, tid);

    auto gload = [&](int k0) {
        pa.load(k0, K);
        if (BT) {
            pbt.load(k0, K);
            return;
        }
#pragma unroll
        for (int i = 0; i < T::B_PT; ++i) {
            const int kk = k0 + b_k0 + i * B_KSTEP;
            const int nn = n0 + b_c * 4;
            const float *src = b_ptr + i * b_istep + (int64_t)k0 * p.ldb;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (kk < K && nn + 4 <= N) {
                v = load16<f32x4>(src);
            } else if (kk < K && nn < N) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = nn + j < N ? src[j] : 0.0f;
            }
            rb[i] = v;
        }
    };

    auto lstore = [&](int buf) {
        pa.store(As[buf]);
        if (BT) {
            pbt.store(Bs[buf]);
            return;
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
    const int nk = cdiv(K, BK);

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk)
            gload((kt + 1) * BK);

        // A fragments for the whole stage.
        f32x4 af[FM][KH / 4];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            read_rows<T>(As[cur], wm * T::WTM + fm * 32 + l32, h, af[fm]);
        if (BT) {
            f32x4 bt[FN][KH / 4];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                read_rows<T>(Bs[cur], wn * T::WTN + fn * 32 + l32, h, bt[fn]);
#pragma unroll
            for (int s = 0; s < KH; ++s)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            af[fm][s >> 2][s & 3], bt[fn][s >> 2][s & 3], acc[fm][fn], 0, 0, 0);
        } else {
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

// Direct-to-LDS FP32 kernel for 128-bit-aligned operands.
//
// The same arithmetic as gemm_f32_kernel (k = 16q + 8h + s at MFMA step s of
// half-stage q, A read as eight k-values per lane per half-stage), but both
// operands travel global -> LDS with global_load_dwordx4-to-LDS copies: no
// staging registers, no LDS stores, and a ring of NBUF stages of BK = 16 or 32
// k-values (one or two half-stages).
//   A: BM rows x 4*BK bytes per stage; 16-byte chunks XOR-swizzled by
//      (row / (16/CPR)) % CPR (CPR = BK/4 chunks per row), so the 16 lanes one
//      LDS cycle serves (16 consecutive rows, one logical chunk) hit 16
//      different 16-byte bank groups. One copy (KiB) = 64/CPR rows; at
//      BK = 32 a row's stage is a whole 128-byte line.
//   B given K-by-N: BK k-rows x BN floats, unpadded; the 16-byte chunks of
//      rows with k % 16 >= 8 XOR 8, so the two half-waves (rows 16q + s and
//      16q + 8 + s of a step, 128 bytes each) fall in different halves of the
//      256-byte bank line. One copy = 1024/(4*BN) rows; each lane reads one
//      float per MFMA step.
//   B given N-by-K (BT): BN rows, copied and read exactly like A.
// A stage's barrier sits before its last k-step, when the wave holds that
// step's operands in registers: the barrier publishes stage kt+1 and frees
// stage kt's buffer, which is refilled with stage kt+NBUF while the last
// step's MFMAs run (a few copies after each row of MFMAs), and the next
// stage's first operands are read then too; a half-stage's row-panel
// operands are read at the start of the half before. Every copy is one
// global_load_lds on every lane (lanes outside A or B read the zero chunk),
// so the vmcnt waits count exactly.
// The workgroup is a WGM x WGN grid of waves, each owning a (BM/WGM) x
// (BN/WGN) block of the tile; at 2 x 4 and two waves per SIMD, one wave's
// MFMAs keep the SIMD busy while the other waits at a barrier, on an LDS read
// or on issuing a copy.
//
// K-slices (KS > 1, for problems too small to fill the CUs with tiles): the
// workgroup holds KS such grids, slice s running the pipeline above on its own
// ring over the s-th of KS equal, stage-aligned parts of the tile's K range
// (all slices run the same number of stages, past the end on zeros, so they
// share every barrier). The partial tiles are then summed through the LDS in
// slice order and slice 0 writes the result: K split without atomics, extra
// passes or a second launch, and with KS times the waves to hide each
// stage's load latency.
//
// CHK: which bounds the copies check (CHK_M: rows of A, CHK_N: columns of B,
// or rows given N-by-K, CHK_K: the K range). The launcher leaves out a check
// when every copy of the launch passes it: tiles inside M, or N, and every
// workgroup's (and slice's) K range a whole number of stages. An unchecked
// copy needs no select: interior launches save about a quarter of the
// per-stage VALU work.
template <int EPI, int BM, int BN, int BK, int NBUF, int WPE, int WGM, int WGN, int KS, bool BT,
          bool SK, int CHK, bool WS = false>
__global__ void __launch_bounds__(64 * WGM * WGN * KS) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
gemm_f32_direct_kernel(GemmParams p)
{
    static_assert(!WS || SK, "the workspace serves stream-K launches");
    constexpr int NW = WGM * WGN;                             // waves per slice
    constexpr int HALVES = BK / 16, STEPS = BK / 2;           // half-stages, MFMA k-steps
    constexpr int WTM = BM / WGM, WTN = BN / WGN, FM = WTM / 32, FN = WTN / 32;
    constexpr int A_STAGE = BM * BK, B_STAGE = BK * BN;       // floats
    constexpr int CPR = BK / 4;                               // 16-byte chunks per panel row
    constexpr int RPC = 64 / CPR;                             // panel rows per copy
    constexpr int COPIES_A = BM / RPC / NW;                   // per wave per stage
    constexpr int CPB = BN / 4;                               // 16-byte chunks per B k-row
    constexpr int RB = 64 / CPB;                              // B k-rows per copy
    constexpr int COPIES_B = BT ? BN / RPC / NW : BK / RB / NW;
    constexpr int PER_STAGE = COPIES_A + COPIES_B;
    static_assert(BK == 16 || BK == 32, "stage depth");
    static_assert(COPIES_A >= 1 && COPIES_B >= 1 && RB >= 1 && RB <= 8 && (BT || CPB >= 16),
                  "tile shape");
    static_assert(COPIES_A * RPC * NW == BM && COPIES_B * (BT ? RPC : RB) * NW == (BT ? BN : BK) &&
                      (COPIES_A * RPC) % 16 == 0 && (!BT || (COPIES_B * RPC) % 16 == 0) &&
                      FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0,
                  "copies cover the stage; each wave's panel rows start at a multiple of 16");
    static_assert((NBUF - 1) * PER_STAGE <= 63 && NBUF >= 2 && NBUF <= 4, "vmcnt range");
    static_assert(KS >= 1 && NW * KS <= 16 && (KS == 1 || !SK), "K-slices");
    static_assert((KS - 1) * NW * FM * FN * 16 * 64 <= KS * NBUF * A_STAGE, "slice partials fit");
    __shared__ __attribute__((aligned(1024))) float As[KS][NBUF][A_STAGE];
    __shared__ __attribute__((aligned(1024))) float Bs[KS][NBUF][B_STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_wg = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slice = wave_wg / NW, wave = wave_wg % NW;   // wave within the slice
    const int wm = wave / WGN, wn = wave % WGN;
    auto swz = [](int row) { return (row / (16 / CPR)) & (CPR - 1); };
    select_batch(p);
    // One tile per workgroup, or (a stream-K launch's sharing workgroups, from
    // sk_block on) up to two (tile, k-range) segments, each a complete pass of
    // the pipeline below whose partial sums are added atomically.
    const bool sharing = SK && (int)blockIdx.x >= p.sk_block;
    __shared__ int sk_last;   // stream-K with a workspace: this workgroup finishes the tile
    for (int seg = 0;; ++seg) {
    int tm, tn, K, kb, st = 0;
    if (sharing) {
        if (!sk_segment(p, seg, tm, tn, kb, K, &st))
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
    const float *__restrict__ A = static_cast<const float *>(p.A) + kb;
    const float *__restrict__ B =
        static_cast<const float *>(p.B) + (BT ? (int64_t)kb : (int64_t)kb * p.ldb);
    const int M = p.M, N = p.N;
    // beta*C with K-slices and one block per wave (the small tiles of small
    // problems): slice 0 loads its C values now, so that their latency hides
    // behind the product instead of following it
    // With K-slices whose partial tiles fit the A rings whole (SUM_ALL: the
    // 64x64 tile in four slices), every lane finishes one 128-bit group of the
    // tile, and preloads its beta*C too.
    constexpr bool SUM_ALL = KS > 1 && BN <= NBUF * BK && BN >= 64 && BN % 64 == 0;
    constexpr int SUM_GROUPS = SUM_ALL ? BM * BN / 4 / (KS * NW * 64) : 1;   // per lane
    static_assert(!SUM_ALL || SUM_GROUPS * KS * NW * 64 * 4 == BM * BN, "groups per lane");
    constexpr bool PRE_C = EPI == EPI_GEMM_BETA && KS > 1 && (SUM_ALL || FM * FN == 1);
    f32x4 cpre[PRE_C ? 4 : 1];
    if constexpr (PRE_C && SUM_ALL) {
        static_assert(SUM_GROUPS <= 4, "preloaded groups");
#pragma unroll
        for (int i = 0; i < SUM_GROUPS; ++i) {
            const int q = tid + i * (KS * NW * 64);
            cpre[i] = load_c4(p, m0 + q / (BN / 4), n0 + (q % (BN / 4)) * 4);
        }
    } else if constexpr (PRE_C) {
        if (slice == 0)
            load_c_x4(p, m0 + wm * WTM, n0 + wn * WTN, lane, cpre);
    }

    // Copy sources. Row-panel copy j (A, or B given N-by-K) covers rows
    // (wave*COPIES + j)*RPC + lane/CPR. Each wave's rows start at a multiple
    // of 16, so the swizzled chunk a lane fetches depends only on
    // (j*RPC) % 16: one variant at BK = 16, two (j even, j odd) at BK = 32.
    const int r_lane = lane / CPR, slot = lane % CPR;
    const int a_row = wave * COPIES_A * RPC + r_lane;    // row of copy 0 (A)
    const int bt_row = wave * COPIES_B * RPC + r_lane;   // row of copy 0 (B given N-by-K)
    int ch[2];
    const float *a_src[2], *bt_src[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        ch[v] = slot ^ swz(((v * RPC) & 15) + r_lane);
        a_src[v] = A + (int64_t)(m0 + a_row) * p.lda + ch[v] * 4;
        bt_src[v] = B + (int64_t)(n0 + bt_row) * p.ldb + ch[v] * 4;
    }
    // B copy j (given K-by-N): k-rows kr0 + lane/CPB with kr0 =
    // (wave*COPIES_B + j)*RB; the lane fills physical chunk lane%CPB, holding
    // logical chunk (lane%CPB) ^ (kr & 8), and kr & 8 = kr0 & 8 (kr0 is a
    // multiple of RB <= 8), so two sources cover every copy.
    const int b_r = lane / CPB, b_pc = lane % CPB;
    const float *b_src[2];
    bool b_ok[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        const int col = n0 + (b_pc ^ (8 * v)) * 4;
        b_src[v] = B + (int64_t)b_r * p.ldb + col;
        b_ok[v] = col < N;
    }
    const uint32_t as_base = lds_addr(&As[slice][0][0]), bs_base = lds_addr(&Bs[slice][0][0]);

    // Copy c (A: 0 .. COPIES_A-1, then B) of the stage at k0 into buffer buf.
    auto copy = [&](int buf, int k0, int c) {
        const float *src;
        uint32_t dst;
        if (c < COPIES_A || BT) {
            const bool is_a = c < COPIES_A;
            const int j = is_a ? c : c - COPIES_A;
            const int v = ((j * RPC) & 15) != 0;
            dst = (is_a ? as_base + buf * (A_STAGE * 4) : bs_base + buf * (B_STAGE * 4)) +
                  (wave * (is_a ? COPIES_A : COPIES_B) + j) * 1024;
            const int64_t step = (int64_t)(j * RPC) * (is_a ? p.lda : p.ldb) + k0;
            const float *in = (is_a ? a_src[v] : bt_src[v]) + step;
            const bool row_chk = is_a ? (CHK & CHK_M) != 0 : (CHK & CHK_N) != 0;
            if (!row_chk && !(CHK & CHK_K)) {
                src = in;
            } else {
                const bool ok =
                    (!row_chk || (is_a ? a_row < M - m0 - j * RPC : bt_row < N - n0 - j * RPC)) &&
                    (!(CHK & CHK_K) || k0 + ch[v] * 4 < K);
                src = ok ? in : zero_chunk<float>();
            }
        } else {
            const int j = c - COPIES_A;
            const int kr0 = (wave * COPIES_B + j) * RB;
            const int v = (kr0 & 8) != 0;
            dst = bs_base + buf * (B_STAGE * 4) + (wave * COPIES_B + j) * 1024;
            const float *in = b_src[v] + (int64_t)(k0 + kr0) * p.ldb;
            if constexpr (!(CHK & (CHK_N | CHK_K)))
                src = in;
            else
                src = (!(CHK & CHK_K) || k0 + kr0 + b_r < K) && (!(CHK & CHK_N) || b_ok[v])
                          ? in
                          : zero_chunk<float>();
        }
        lds_dma_16(src, dst);
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
    // Row-panel operands of half-stage q (A, and B given N-by-K): the lane's
    // row, k = 16q + 8h .. 16q + 8h + 7 (logical chunks 4q + 2h, 4q + 2h + 1).
    auto read_rows = [&](const float *lds, int row0, int q, auto &frag) {
        constexpr int F = sizeof(frag) / sizeof(frag[0]);
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const int row = row0 + f * 32 + l32;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int c = (4 * q + 2 * h + e) ^ swz(row);
                frag[f][e] = *reinterpret_cast<const f32x4 *>(&lds[row * BK + c * 4]);
            }
        }
    };
    auto read_a = [&](int buf, int q, f32x4 (&af)[FM][2]) {
        read_rows(As[slice][buf], wm * WTM, q, af);
    };
    auto read_bt = [&](int buf, int q, auto &bt) { read_rows(Bs[slice][buf], wn * WTN, q, bt); };
    // B operands of k-step t of a stage (B given K-by-N): k = 16(t/8) + 8h + t%8.
    auto read_b = [&](int buf, int t, float (&bf)[FN]) {
        const int k = 16 * (t / 8) + 8 * h + (t % 8);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = wn * WTN + fn * 32 + l32;
            bf[fn] = Bs[slice][buf][k * BN + (((n >> 2) ^ (8 * h)) << 2) + (n & 3)];
        }
    };
    constexpr int FT = BT ? FN : 1;   // row-panel B operands kept per half-stage
    // With several waves per SIMD, each group of MFMAs runs at raised issue
    // priority (s_setprio), so the wave with MFMAs ready wins the arbitration
    // over the others while they read, copy or wait (4096^3: +1.4 %, 2048^3
    // as two K-slices: +3.5 %).
    auto mfma_step = [&](const f32x4 (&af)[FM][2], int s, const float (&bf)[FN],
                         const f32x4 (&bt)[FT][2]) {
        if (NW * KS > 4)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                    af[fm][s >> 2][s & 3], BT ? bt[BT ? fn : 0][s >> 2][s & 3] : bf[fn], acc[fm][fn],
                    0, 0, 0);
        if (NW * KS > 4)
            __builtin_amdgcn_s_setprio(0);
    };
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

    const int nk = cdiv(k_steps, BK);   // the same in every slice
    for (int st = 0; st < NBUF; ++st)
        if (st < nk) {
#pragma unroll
            for (int c = 0; c < PER_STAGE; ++c)
                copy(st, st * BK, c);
        }
    wait_stages((nk < NBUF ? nk : NBUF) - 1);   // stage 0 has landed
    __syncthreads();

    f32x4 af[FM][2], an[FM][2];   // the current and the next half-stage's A operands
    f32x4 bt[FT][2], btn[FT][2];  // the same for B given N-by-K
    float bf[2][FN];              // B given K-by-N: two steps' operands
    read_a(0, 0, af);
    if constexpr (BT)
        read_bt(0, 0, bt);
    else
        read_b(0, 0, bf[0]);
    int buf = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const int nbuf = buf == NBUF - 1 ? 0 : buf + 1;
#pragma unroll
        for (int t = 0; t + 1 < STEPS; ++t) {
            const int q = t / 8, s = t % 8;
            if constexpr (!BT)
                read_b(buf, t + 1, bf[(t + 1) & 1]);
            if (HALVES > 1 && s == 0 && q + 1 < HALVES) {   // the next half-stage's panels
                read_a(buf, q + 1, an);
                if constexpr (BT)
                    read_bt(buf, q + 1, btn);
            }
            mfma_step(af, s, bf[t & 1], bt);
            if (HALVES > 1 && s == 7) {
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    af[fm][0] = an[fm][0];
                    af[fm][1] = an[fm][1];
                }
                if constexpr (BT) {
#pragma unroll
                    for (int fn = 0; fn < FT; ++fn) {
                        bt[fn][0] = btn[fn][0];
                        bt[fn][1] = btn[fn][1];
                    }
                }
            }
        }
        if (kt + 1 < nk) {
            // stage kt+1 has landed (stages up to kt+NBUF-1 were issued); after
            // the barrier every wave is done with this stage's buffer
            wait_stages((kt + NBUF - 1 < nk ? kt + NBUF - 1 : nk - 1) - (kt + 1));
            __syncthreads();
        }
        const int k_next = (kt + NBUF) * BK;   // refill this buffer with stage kt+NBUF
        const bool refill = kt + NBUF < nk;
        // Operands of stage kt+1 (after the last stage: stale, in-bounds, unused).
        read_a(nbuf, 0, an);
        if constexpr (BT)
            read_bt(nbuf, 0, btn);
        else
            read_b(nbuf, 0, bf[0]);
        constexpr int G = (PER_STAGE + FM - 1) / FM;   // refill copies per MFMA row
        if (NW * KS > 4)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                    af[fm][1][3], BT ? bt[BT ? fn : 0][1][3] : bf[1][fn], acc[fm][fn], 0, 0, 0);
            if (refill && fm * G < PER_STAGE) {
#pragma unroll
                for (int g = 0; g < G; ++g)
                    if (fm * G + g < PER_STAGE)
                        copy(buf, k_next, fm * G + g);
            }
        }
        if (NW * KS > 4)
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            af[fm][0] = an[fm][0];
            af[fm][1] = an[fm][1];
        }
        if constexpr (BT) {
#pragma unroll
            for (int fn = 0; fn < FT; ++fn) {
                bt[fn][0] = btn[fn][0];
                bt[fn][1] = btn[fn][1];
            }
        }
        buf = nbuf;
    }

    if constexpr (SUM_ALL) {
        // Every slice writes its partial tile into its own (now idle) A ring
        // as a BM x BN row-major array, columns XOR 32 on rows with bit 2 set
        // (the two half-waves of a write, rows r and r+4, then fill opposite
        // halves of the 64 banks); then every lane of the workgroup adds the
        // slices of its groups of four columns in slice order (the order of
        // the path below) and finishes them with 128-bit accesses.
        __syncthreads();   // every slice is done reading its ring
        float *part = &As[slice][0][0];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wm * WTM + fm * 32 + ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
                    const int col = wn * WTN + fn * 32 + (lane & 31);
                    part[row * BN + (col ^ (((row >> 2) & 1) << 5))] = acc[fm][fn][r];
                }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < SUM_GROUPS; ++i) {
            const int q = tid + i * (KS * NW * 64);
            const int row = q / (BN / 4), col = (q % (BN / 4)) * 4;
            const int pc = col ^ (((row >> 2) & 1) << 5);
            f32x4 v = *reinterpret_cast<const f32x4 *>(&As[0][0][row * BN + pc]);
#pragma unroll
            for (int sl = 1; sl < KS; ++sl) {
                const f32x4 w = *reinterpret_cast<const f32x4 *>(&As[sl][0][row * BN + pc]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] += w[e];
            }
            finish4<EPI>(p, v, m0 + row, n0 + col, PRE_C ? cpre[PRE_C ? i : 0] : v);
        }
        continue;   // (a K-sliced tile has one segment)
    } else if constexpr (KS > 1) {
        // Slices 1.. park their partial tiles in the (now idle) A rings, one
        // float per lane per slot, then slice 0 adds them in slice order.
        float *part = &As[0][0][0];
        constexpr int SLOTS = FM * FN * 16;
        __syncthreads();   // every slice is done reading its ring
        if (slice > 0) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        part[((((slice - 1) * NW + wave) * SLOTS) + (fm * FN + fn) * 16 + r) * 64 + lane] =
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
                    for (int r = 0; r < 16; ++r)
                        acc[fm][fn][r] +=
                            part[((((sl - 1) * NW + wave) * SLOTS) + (fm * FN + fn) * 16 + r) * 64 + lane];
    }

    // Stream-K with a workspace (WS): add this segment's partial sums into
    // the shared tile's workspace tile, then count the arrival. The last of
    // the tile's contributors applies the epilogue to the sums, writes the
    // tile and clears the workspace tile and counter for the next call.
    // Nobody waits for anybody: each contributor only adds and counts, and the
    // count tells the last one that all sums are in. The workspace tile is
    // kept in accumulator order (wave, block, register, lane): a lane's adds
    // are one base address plus constants, 256 bytes per wave instruction,
    // and four consecutive floats are four consecutive columns of one row.
    if (WS && sharing) {
        constexpr int NB = FM * FN;            // accumulator blocks per wave
        constexpr int NT = 64 * NW * KS;
        float *wt = p.ws + (int64_t)st * (BM * BN);
        float *mine = wt + wave * (NB * 16 * 64) + lane;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    __hip_atomic_fetch_add(mine + ((fm * FN + fn) * 16 + r) * 64, acc[fm][fn][r],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // The barrier orders every wave's adds before thread 0's count (and
        // waits for them); the count's release and acquire, one per
        // workgroup, make them visible device-wide and the other
        // contributors' adds visible here.
        __syncthreads();
        if (tid == 0) {
            const int before = __hip_atomic_fetch_add(p.ws_cnt + st, 1, __ATOMIC_ACQ_REL,
                                                      __HIP_MEMORY_SCOPE_AGENT);
            sk_last = before == sk_contributors(p, st) - 1;
        }
        __syncthreads();
        if (sk_last) {
            // eight groups in flight per lane (unrolled by 8: 2 us faster per
            // fused-layer call than no unrolling; 16 or 32 measured no faster,
            // and 32 spills registers)
#pragma unroll 8
            for (int q = tid; q < BM * BN / 4; q += NT) {
                const int e = 4 * q, l = e & 63, r = (e >> 6) & 15, blk = (e >> 10) % NB;
                const int w = (e >> 10) / NB;
                const int row = (w / WGN) * WTM + (blk / FN) * 32 + ((r >> 2) << 3) + ((l >> 5) << 2) +
                                (r & 3);
                const int col = (w % WGN) * WTN + (blk % FN) * 32 + (l & 31);
                f32x4 *src = reinterpret_cast<f32x4 *>(wt + e);
                const f32x4 v = *src;
                *src = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                const f32x4 cv = EPI == EPI_GEMM_BETA ? load_c4(p, m0 + row, n0 + col) : v;
                finish4<EPI>(p, v, m0 + row, n0 + col, cv);
            }
            if (tid == 0)
                __hip_atomic_store(p.ws_cnt + st, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    if (WS && sharing) {
        // the workspace path above wrote (or left to a later contributor) the tile
    } else if (sharing || EPI == EPI_ATOMIC || EPI == EPI_GEMM_BETA0) {
        // atomic partial sums, or alpha*acc: 32-bit stores, one column per lane
        // (alpha*acc measured no faster with 128-bit stores: 4096^3 +0.4 %,
        // 256^3 +5 % in time)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                if (sharing)
                    write_block<EPI_ATOMIC>(p, acc[fm][fn], m0 + wm * WTM + fm * 32,
                                            n0 + wn * WTN + fn * 32, lane);
                else
                    write_block<EPI>(p, acc[fm][fn], m0 + wm * WTM + fm * 32,
                                     n0 + wn * WTN + fn * 32, lane);
            }
    } else {
        // beta*C and the fused layer: 128-bit loads and stores through a
        // per-wave LDS area (2048^3 with alpha/beta 137.7 -> 133.3 us, 1024^3
        // 22.4 -> 22.1 us, the 2047x11008 layer 1.340 -> 1.327 ms): slice 0's
        // B ring with K-slices (the A rings hold the partial tiles), else the
        // A ring once every wave is done reading it
        static_assert(NW * kStageFloats <= (KS > 1 ? NBUF * B_STAGE : NBUF * A_STAGE),
                      "write-back staging fits");
        if constexpr (KS == 1)
            __syncthreads();
        float *stage = (KS > 1 ? &Bs[0][0][0] : &As[0][0][0]) + wave * kStageFloats;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                write_block_x4<EPI, PRE_C>(p, acc[fm][fn], m0 + wm * WTM + fm * 32,
                                           n0 + wn * WTN + fn * 32, lane, stage, cpre);
    }
    }
}

// Tile configurations. The staged 256x256 kernel runs one wave per SIMD (256
// accumulators per lane; the direct one's wave grid is chosen below); the
// other tiles are compiled for two waves per SIMD, so two workgroups share a
// CU and each covers the other's barrier and memory waits. With the
// direct-to-LDS kernel, 256x256 (one tile per CU) is the fastest on the
// 4096^3 product (about 89 % of the FP32 matrix peak); 256x128 at two
// workgroups per CU is the plain choice for the 2047 x 11008 fully-connected
// layer, whose leftover tiles stream-K otherwise shares out.
// Skinny products (a few rows of A): memory-bound, so vector FMAs instead of
// MFMAs, which would compute a whole 32-row block for every row. A
// workgroup of four waves covers 256 columns of C over its K range (a
// K-split), A's rows MR at a time (MR = 1, 2, 4, 8 or 16, the fewest that
// cover M). The A block of the K range is staged in LDS once (SK_XS floats: the
// planner keeps the range within SK_XS / MR k-values; a longer one, from a
// forced plan, is walked in chunks of that size). B streams from HBM with
// the next loads issued before the current ones are used.
//   B given K-by-N: lane l covers columns 4l .. 4l+3 (one 16-byte load per
//     k-row); wave w takes the runs of U k-rows numbered w mod 4, split y
//     starting at run y mod runs and wrapping around; A's values are LDS
//     broadcasts; the four waves' sums meet in LDS at the end.
//   B given N-by-K: wave w covers columns 64w .. 64w+63 in 16 groups of four;
//     in a group, lane l reads column 4g + l/16's row of B at k-values
//     4(l%16) + 64j, so a load covers 64 consecutive k of four rows; the 16
//     lanes of a row add their sums by DPP and the result goes to an LDS row
//     of C, stored once at the end.
// B's loads take whole 16-byte chunks at any alignment, the chunk that
// crosses N or K element by element. The epilogue: alpha*acc (+ beta*C),
// bias and ReLU, or atomic partial sums for a K-split.
constexpr int SK_COLS = 256;     // columns of C per workgroup
constexpr int SK_XS = 8192;      // LDS floats for the staged A block (32 KiB)

// A's rows mc .. mc+MR-1 (zero past M), k-values kc .. kc+kn-1 of the K
// range, into xs[m][0 .. kpad) (zero past kn; kpad = kn rounded up to 64).
template <int MR>
__device__ __forceinline__ void skinny_stage(float *xs, const float *A, int64_t lda, int64_t mc, int M,
                                             int64_t kc, int kn)
{
    constexpr int KC = SK_XS / MR;
    const int kq = ((kn + 63) & ~63) / 4;   // 16-byte chunks per row
    for (int i = threadIdx.x; i < MR * kq; i += 256) {
        const int m = i / kq, k = (i % kq) * 4;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (mc + m < M) {
            const float *src = A + (mc + m) * lda + kc + k;
            if (k + 4 <= kn) {
                v = load16<f32x4>(src);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = k + j < kn ? src[j] : 0.0f;
            }
        }
        *reinterpret_cast<f32x4 *>(xs + m * KC + k) = v;
    }
}

template <int EPI, bool BT, int MR>
__global__ void __launch_bounds__(256) gemm_f32_skinny_kernel(GemmParams p)
{
    constexpr int KC = SK_XS / MR;                        // k-values staged at once
    constexpr int RED = BT ? MR * SK_COLS : 3 * MR * SK_COLS;   // N-by-K: C row block; K-by-N: 3 waves' sums
    __shared__ __attribute__((aligned(16))) float lds[BT ? SK_XS + RED : (SK_XS > RED ? SK_XS : RED)];
    float *xs = lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    select_batch(p);
    int K;
    const int kb = split_range(p, K);
    const float *__restrict__ A = static_cast<const float *>(p.A) + kb;
    const float *__restrict__ B =
        static_cast<const float *>(p.B) + (BT ? (int64_t)kb : (int64_t)kb * p.ldb);
    const int M = p.M, N = p.N;
    const int nblk = blockIdx.x * SK_COLS;

    // 64-bit chunk counters and row checks: M or K may lie within one chunk of 2^31
    for (int64_t mc = 0; mc < M; mc += MR) {
        if constexpr (!BT) {
            constexpr int U = MR == 16 ? 4 : 8;   // k-rows per run (loads in flight per lane, twice)
            const int ncol = nblk + 4 * lane;
            const bool full = ncol <= N - 4, part = ncol < N;
            f32x4 acc[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m)
                acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int64_t kc = 0; kc < K; kc += KC) {
                const int kn = K - kc < KC ? (int)(K - kc) : KC;
                __syncthreads();   // the previous chunk's (or row block's) A values are read
                skinny_stage<MR>(xs, A, p.lda, mc, M, kc, kn);
                __syncthreads();
                const float *Bc = B + kc * p.ldb + ncol;
                const int runs = (kn + 4 * U - 1) / (4 * U);   // runs of all four waves
                // the K-splits walk their runs from different starting points, so
                // that the splits in flight do not read rows a multiple of the
                // split length apart (a power-of-two stride in common shapes)
                const int rot = (int)(blockIdx.y % (unsigned)runs);
                auto fetch = [&](f32x4 (&w)[U], int run) {
                    run += rot;
                    run = run >= runs ? run - runs : run;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int k = (4 * run + wave) * U + u;
                        const float *src = Bc + (int64_t)k * p.ldb;
                        f32x4 v = {0.f, 0.f, 0.f, 0.f};
                        if (k < kn && full) {
                            v = load16<f32x4>(src);
                        } else if (k < kn && part) {
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                v[j] = ncol + j < N ? src[j] : 0.0f;
                        }
                        w[u] = v;
                    }
                };
                f32x4 wc[U], wn[U];
                fetch(wc, 0);
                for (int r = 0; r < runs; ++r) {
                    if (r + 1 < runs)
                        fetch(wn, r + 1);
                    const int rr = r + rot < runs ? r + rot : r + rot - runs;
                    const int k0 = (4 * rr + wave) * U;   // within KC: KC is a multiple of 4U
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
#pragma unroll
                        for (int q = 0; q < U / 4; ++q) {
                            const f32x4 x = *reinterpret_cast<const f32x4 *>(xs + m * KC + k0 + 4 * q);
                            acc[m] += x[0] * wc[4 * q] + x[1] * wc[4 * q + 1] + x[2] * wc[4 * q + 2] +
                                      x[3] * wc[4 * q + 3];
                        }
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        wc[u] = wn[u];
                }
            }
            // the four waves' sums of the same columns, through LDS
            __syncthreads();   // xs is read; red aliases it
            f32x4 *red = reinterpret_cast<f32x4 *>(lds);
            if (wave > 0) {
#pragma unroll
                for (int m = 0; m < MR; ++m)
                    red[((wave - 1) * MR + m) * 64 + lane] = acc[m];
            }
            __syncthreads();
            if (wave == 0) {
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    const f32x4 a = acc[m] + red[m * 64 + lane] + red[(MR + m) * 64 + lane] +
                                    red[(2 * MR + m) * 64 + lane];
                    if (mc + m < M) {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (ncol + j < N)
                                skinny_store<EPI>(p, (int)mc + m, ncol + j, a[j]);
                    }
                }
            }
        } else {
            float *ys = lds + SK_XS;   // [MR][SK_COLS]: this row block of C
            for (int i = tid; i < MR * SK_COLS; i += 256)
                ys[i] = 0.0f;
            constexpr int D = MR == 16 ? 2 : 8;   // loads in flight per lane
            const int c4 = 4 * (lane & 15), rg = lane >> 4;
            for (int64_t kc = 0; kc < K; kc += KC) {
                const int kn = K - kc < KC ? (int)(K - kc) : KC;
                __syncthreads();   // the previous chunk's (or row block's) A values are read
                skinny_stage<MR>(xs, A, p.lda, mc, M, kc, kn);
                __syncthreads();
                const int steps = (kn + 63) / 64;      // 64 k-values of a row per load
                const int total = 16 * steps;          // (group, step) pairs of this wave
                auto fetch = [&](int t) -> f32x4 {
                    f32x4 v = {0.f, 0.f, 0.f, 0.f};
                    if (t >= total)
                        return v;
                    const int g = t / steps, k = (t - g * steps) * 64 + c4;
                    const int col = nblk + 64 * wave + 4 * g + rg;
                    if (col >= N)
                        return v;
                    const float *src = B + (int64_t)col * p.ldb + kc + k;
                    if (k + 4 <= kn) {
                        v = load16<f32x4>(src);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            v[j] = k + j < kn ? src[j] : 0.0f;
                    }
                    return v;
                };
                f32x4 w[D];
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
                            const int k0 = st * 64 + c4;   // within KC: KC is a multiple of 64
#pragma unroll
                            for (int m = 0; m < MR; ++m) {
                                const f32x4 x = *reinterpret_cast<const f32x4 *>(xs + m * KC + k0);
                                acc[m] += x[0] * w[d][0] + x[1] * w[d][1] + x[2] * w[d][2] + x[3] * w[d][3];
                            }
                            w[d] = fetch(tb + d + D);
                            if (++st == steps) {
                                // group g done: the 16 lanes of each row add up, lane 0 of the
                                // row adds the sums into the C row block
#pragma unroll
                                for (int m = 0; m < MR; ++m) {
                                    const float v = dpp_row_sum16(acc[m]);
                                    if ((lane & 15) == 0)
                                        ys[m * SK_COLS + 64 * wave + 4 * g + rg] += v;
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
                for (int m = 0; m < MR; ++m) {
                    if (mc + m < M)
                        skinny_store<EPI>(p, (int)mc + m, col, ys[m * SK_COLS + tid]);
                }
            }
            __syncthreads();   // ys is read before the next row block clears it
        }
    }
}

using F32_L = F32Tile<256, 256, 16>;   // 128x128 per wave
using F32_M = F32Tile<256, 128, 16>;   // 128x64 per wave
using F32_S = F32Tile<128, 128, 16>;   // 64x64 per wave
using F32_XS = F32Tile<64, 64, 16>;    // 32x32 per wave
// Ring lengths of the direct kernel: 256x256 (one workgroup per CU) and
// 256x128 (two per CU, at most 80 KiB of LDS each) measured no faster with
// longer rings (within 1 %). The 128x128 and 64x64 tiles (plain or K-sliced)
// serve problems too small to fill the CUs; they run two stages of BK = 32,
// which measured faster than four of BK = 16 in the same LDS (whole-line
// copies, half the barriers): 1024^3 as 64x64 in four K-slices 29.5 -> 27.4
// us, 2048^3 as 128x128 in two 144 -> 139 us.
constexpr int kDirectNbufL = 2, kDirectNbufM = 2;
// Stage depth of the 256x256 tile: 32 (two 64 KiB stages), so each row-panel
// copy reads whole 128-byte lines; the other tiles keep 16.
constexpr int kDirectBkL = 32;
// Wave grid of the 256x256 tile: 2 x 4, eight waves (two per SIMD, 128x64
// each), for both B layouts. Against 2 x 2 (one wave per SIMD), measured in
// one process: B given K-by-N 4096^3 138 -> 140 TFLOP/s, 8192^3 139 -> 141;
// B given N-by-K 4096^3 144 either way (with bounds-checked copies eight
// waves lost, 141 -> 129), the 2047x11008 layer with stream-K 132.4 -> 133.7.
template <bool BT> struct WaveGridL {
    static constexpr int M = 2, N = 4;
    static constexpr int WPE = M * N / 4;   // waves per SIMD
};

// The bounds checks a launch of tile BMxBN (KS K-slices of stages of BK)
// needs: rows of A unless the tiles lie inside M; the N bound unless inside
// N; the K bound unless every workgroup's and slice's K range is a whole
// number of stages (stream-K shares are whole kSkUnit units, a multiple of
// BK). Instances exist for none, M only (the 2047x11008 layer: 134.3 -> 137.9
// TFLOP/s with W given K-by-N, 133.4 -> 136.6 given N-by-K), and all three.
static int launch_checks(const GemmParams &p, int BM, int BN, int BK, int KS)
{
    const int kq = KS * BK;
    const bool k_whole = p.K % kq == 0 && p.k_split % kq == 0 &&
                         (p.sk_tiles == 0 || (KS == 1 && p.K % kSkUnit == 0 && kSkUnit % BK == 0));
    if (p.N % BN != 0 || !k_whole)
        return CHK_M | CHK_N | CHK_K;
    return p.M % BM == 0 ? 0 : CHK_M;
}

template <int BM, int BN, int BK, int NBUF, int WPE, int WGM, int WGN, bool BT, int KS = 1>
static hipError_t launch_direct(const GemmParams &p, int64_t ntiles, int epi, hipStream_t s)
{
    if (ntiles > max_grid_x(64 * WGM * WGN * KS))
        return hipErrorInvalidValue;
    const dim3 grid = gemm_grid(p, ntiles), block(64 * WGM * WGN * KS);
    const int chk = launch_checks(p, BM, BN, BK, KS);
#define LL_F32_DIRECT_C(E, SK, C) \
    hipLaunchKernelGGL((gemm_f32_direct_kernel<E, BM, BN, BK, NBUF, WPE, WGM, WGN, KS, BT, SK, C>), \
                       grid, block, 0, s, p)
#define LL_F32_DIRECT_WS(C) \
    hipLaunchKernelGGL((gemm_f32_direct_kernel<EPI_LINEAR, BM, BN, BK, NBUF, WPE, WGM, WGN, KS, BT, \
                                               true, C, true>), \
                       grid, block, 0, s, p)
#define LL_F32_DIRECT(E, SK) \
    do { \
        if (chk == 0) \
            LL_F32_DIRECT_C(E, SK, 0); \
        else if (chk == CHK_M) \
            LL_F32_DIRECT_C(E, SK, CHK_M); \
        else \
            LL_F32_DIRECT_C(E, SK, CHK_M | CHK_N | CHK_K); \
    } while (0)
    if (KS > 1 && p.sk_tiles > 0)
        return hipErrorInvalidValue;
    if constexpr (KS > 1) {
        if (epi == EPI_GEMM_BETA0) LL_F32_DIRECT(EPI_GEMM_BETA0, false);
        else if (epi == EPI_GEMM_BETA) LL_F32_DIRECT(EPI_GEMM_BETA, false);
        else if (epi == EPI_LINEAR) LL_F32_DIRECT(EPI_LINEAR, false);
        else LL_F32_DIRECT(EPI_ATOMIC, false);
    } else if (p.sk_tiles > 0 && p.ws != nullptr) {
        // the fused layer's stream-K with a workspace: every tile finished in
        // this launch, epilogue fused
        if (epi != EPI_LINEAR)
            return hipErrorInvalidValue;
        if (chk == 0) LL_F32_DIRECT_WS(0);
        else if (chk == CHK_M) LL_F32_DIRECT_WS(CHK_M);
        else LL_F32_DIRECT_WS(CHK_M | CHK_N | CHK_K);
    } else if (p.sk_tiles > 0) {
        // whole tiles with `epi`, shared ones added atomically
        if (epi == EPI_GEMM_BETA0) LL_F32_DIRECT(EPI_GEMM_BETA0, true);
        else if (epi == EPI_GEMM_BETA) LL_F32_DIRECT(EPI_GEMM_BETA, true);
        else if (epi == EPI_LINEAR) LL_F32_DIRECT(EPI_LINEAR, true);
        else return hipErrorInvalidValue;
    } else {
        if (epi == EPI_GEMM_BETA0) LL_F32_DIRECT(EPI_GEMM_BETA0, false);
        else if (epi == EPI_GEMM_BETA) LL_F32_DIRECT(EPI_GEMM_BETA, false);
        else if (epi == EPI_LINEAR) LL_F32_DIRECT(EPI_LINEAR, false);
        else LL_F32_DIRECT(EPI_ATOMIC, false);
    }
#undef LL_F32_DIRECT
#undef LL_F32_DIRECT_C
#undef LL_F32_DIRECT_WS
    return hipGetLastError();
}

template <class T, int WPE, bool BT, int KS = 1>
static hipError_t launch_t(const GemmParams &p0, int epi, bool vec, hipStream_t s)
{
    GemmParams p = p0;
    p.tiles_m = cdiv(p.M, T::BM);
    p.tiles_n = cdiv(p.N, T::BN);
    int64_t ntiles = (int64_t)p.tiles_m * p.tiles_n;
    if (ntiles > kMaxTiles || p.batch < 1 || p.batch > kMaxGridZ)
        return hipErrorInvalidValue;
    if (p.grid_x > 0)
        ntiles = p.grid_x;   // part of the tiles, or a stream-K launch
    if (p.sk_tiles > 0 && !vec)
        return hipErrorInvalidValue;   // stream-K runs on the direct kernel only
    // 128-bit-aligned operands take the direct-to-LDS kernel.
    static_assert(KS == 1 || (T::BM == T::BN && T::BM <= 128), "K-slices: the small tiles only");
    if (vec) {
        if constexpr (T::BM == 256 && T::BN == 256)
            return launch_direct<256, 256, kDirectBkL, kDirectNbufL, WaveGridL<BT>::WPE,
                                 WaveGridL<BT>::M, WaveGridL<BT>::N, BT>(p, ntiles, epi, s);
        else if constexpr (T::BM == 256 && T::BN == 128)
            return launch_direct<256, 128, 16, kDirectNbufM, 2, 2, 2, BT>(p, ntiles, epi, s);
        else if constexpr (T::BM == 128 && T::BN == 128)
            return launch_direct<128, 128, 32, 2, 2 * KS, 2, 2, BT, KS>(p, ntiles, epi, s);
        else if constexpr (T::BM == 64 && T::BN == 64)
            return launch_direct<64, 64, 32, 2, (KS > 1 ? KS : 4), 2, 2, BT, KS>(p, ntiles, epi, s);
    }
    const dim3 grid = gemm_grid(p, ntiles), block(T::NT);
#define LL_F32_LAUNCH(E) \
    hipLaunchKernelGGL((gemm_f32_kernel<T, E, WPE, BT>), grid, block, 0, s, p)
    // register-staged: 16-byte chunk loads at any alignment, the chunk that
    // crosses K or N element by element
    if (epi == EPI_GEMM_BETA0) LL_F32_LAUNCH(EPI_GEMM_BETA0);
    else if (epi == EPI_GEMM_BETA) LL_F32_LAUNCH(EPI_GEMM_BETA);
    else if (epi == EPI_LINEAR) LL_F32_LAUNCH(EPI_LINEAR);
    else LL_F32_LAUNCH(EPI_ATOMIC);
#undef LL_F32_LAUNCH
    return hipGetLastError();
}

// This file builds the instances for B given K-by-N and the tile table; the
// translation unit gemm_f32_nt.hip includes it with LL_F32_NT_UNIT defined to
// build the instances for B given N-by-K, so the two compile in parallel.
#ifndef LL_F32_NT_UNIT
// {BM, BN, workgroups per CU, relative throughput alone on a CU, with a
// second workgroup beside it} -- throughputs measured on MI355X relative to
// the 256x256 tile.
// For the K-sliced tiles (and the 32x128 one), the last two fields are the K
// per workgroup of those measurements and the rate they reach at long K
// ranges: each slice walks K/KS values with its own pipeline fill and drain,
// so their rates depend on K (64x64 in four slices: 0.57 at K = 1024, 0.72 at 2048, 0.78
// at 4096; 128x128 in two: 0.69 at 512, 0.75 at 1024, 0.90 at 2048, no
// higher at 4096). The other tiles' rates stand at any K.
const TileInfo kF32Tiles[kF32NumTiles] = {
    {F32_L::BM, F32_L::BN, 1, 1.00f, 1.00f, "f32_256x256", 1, true, 64 * WaveGridL<false>::M * WaveGridL<false>::N},
    {F32_M::BM, F32_M::BN, 2, 0.89f, 0.985f, "f32_256x128"},
    {F32_S::BM, F32_S::BN, 2, 0.80f, 0.94f, "f32_128x128"},
    {F32_XS::BM, F32_XS::BN, 2, 0.52f, 0.72f, "f32_64x64"},
    // K-sliced tiles (direct kernel only; the staged fallback runs the plain
    // tile): four slices of 64x64 (1024^3: 0.57), two of 128x128 (2048^3: 0.90),
    // each only when every slice gets at least 8 stages of 32 (smaller K: the
    // partial-sum exchange costs more than the slices save; 256^3 8.9 us with
    // slices against 8.3 plain, 512^3 11.1 against 10.3 split across workgroups).
    {F32_XS::BM, F32_XS::BN, 1, 0.57f, 0.57f, "f32_64x64_k4", 4, true, 1024, 4 * 8 * 32, true, 1024, 0.80f},
    {F32_S::BM, F32_S::BN, 1, 0.90f, 0.90f, "f32_128x128_k2", 2, true, 512, 2 * 8 * 32, true, 2048},
    // the skinny kernel: 16 rows of A at a time, 256 columns per workgroup
    {16, SK_COLS, 2, 1.0f, 1.0f, "f32_16x256_skinny", 1, false},
    // 32x128 for a few tens of rows of A (direct kernel only): two waves per
    // workgroup, up to four workgroups per CU. A few per CU each run at about
    // the same speed (16x4096x4096 in 16 K-splits: 2 per CU, 16.8 us of
    // kernel); four fill the CU at about 0.70 (16x11008x4096 in 11 splits,
    // 27.7 us; 2048x2048x1024, 80 us). Its rate was measured at K = 256 per
    // workgroup and falls with shorter ranges as the K-sliced tiles' do
    // (32x8192x1024 in 16 splits, 64 k-values each: 21 us against 16 on
    // 64x64 in 4).
    {32, 128, 4, 0.185f, 0.70f, "f32_32x128", 1, false, 128, 0, true, 256, 0.21f},
};
#endif

template <bool BT>
static hipError_t launch_skinny(const GemmParams &p0, int epi, hipStream_t s)
{
    static_assert(SK_COLS == kSkinnyCols && SK_XS == kSkinnyStage, "skinny kernel shape");
    GemmParams p = p0;
    p.tiles_m = 1;
    p.tiles_n = cdiv(p.N, SK_COLS);
    if (p.batch < 1 || p.batch > kMaxGridZ || p.grid_x != 0 || p.sk_tiles != 0)
        return hipErrorInvalidValue;   // whole grids only, no stream-K
    const dim3 grid = gemm_grid(p, p.tiles_n), block(256);
    const int mr = skinny_rows(p.M);
#define LL_SKINNY_MR(E, MR) hipLaunchKernelGGL((gemm_f32_skinny_kernel<E, BT, MR>), grid, block, 0, s, p)
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
    else if (epi == EPI_LINEAR) LL_SKINNY(EPI_LINEAR);
    else LL_SKINNY(EPI_ATOMIC);
#undef LL_SKINNY
#undef LL_SKINNY_MR
    return hipGetLastError();
}

// The 32-row tile (a few tens of rows of A): 32x128, two waves of 32x64, no
// stream-K. Direct kernel only; unaligned operands run the staged 64x64
// kernel instead.
template <bool BT>
static hipError_t launch_thin(const GemmParams &p0, int epi, bool vec, hipStream_t s)
{
    if (!vec)
        return launch_t<F32_XS, 2, BT>(p0, epi, vec, s);
    GemmParams p = p0;
    p.tiles_m = cdiv(p.M, 32);
    p.tiles_n = cdiv(p.N, 128);
    const int64_t ntiles = (int64_t)p.tiles_m * p.tiles_n;
    if (ntiles > max_grid_x(128) || p.batch < 1 || p.batch > kMaxGridZ || p.sk_tiles != 0 || p.grid_x != 0)
        return hipErrorInvalidValue;
    const dim3 grid = gemm_grid(p, ntiles), block(128);
    const int chk = launch_checks(p, 32, 128, 32, 1);
#define LL_THIN_C(E, C) \
    hipLaunchKernelGGL((gemm_f32_direct_kernel<E, 32, 128, 32, 2, 2, 1, 2, 1, BT, false, C>), grid, block, 0, s, p)
#define LL_THIN(E) \
    do { \
        if (chk == 0) LL_THIN_C(E, 0); \
        else if (chk == CHK_M) LL_THIN_C(E, CHK_M); \
        else LL_THIN_C(E, CHK_M | CHK_N | CHK_K); \
    } while (0)
    if (epi == EPI_GEMM_BETA0) LL_THIN(EPI_GEMM_BETA0);
    else if (epi == EPI_GEMM_BETA) LL_THIN(EPI_GEMM_BETA);
    else if (epi == EPI_LINEAR) LL_THIN(EPI_LINEAR);
    else LL_THIN(EPI_ATOMIC);
#undef LL_THIN
#undef LL_THIN_C
    return hipGetLastError();
}

template <bool BT>
static hipError_t launch_f32(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s)
{
    switch (tile) {
    case 0: return launch_t<F32_L, 1, BT>(p, epi, vec, s);
    case 1: return launch_t<F32_M, 2, BT>(p, epi, vec, s);
    case 2: return launch_t<F32_S, 2, BT>(p, epi, vec, s);
    case 3: return launch_t<F32_XS, 2, BT>(p, epi, vec, s);
    case 4: return launch_t<F32_XS, 2, BT, 4>(p, epi, vec, s);
    case 5: return launch_t<F32_S, 2, BT, 2>(p, epi, vec, s);
    case 7: return launch_thin<BT>(p, epi, vec, s);
    default: return launch_skinny<BT>(p, epi, s);
    }
}

#ifndef LL_F32_NT_UNIT
hipError_t launch_gemm_f32(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s)
{
    return launch_f32<false>(p, tile, epi, vec, s);
}
#else
hipError_t launch_gemm_f32_bt(const GemmParams &p, int tile, int epi, bool vec, hipStream_t s)
{
    return launch_f32<true>(p, tile, epi, vec, s);
}
#endif

}  // namespace ll
