// Device-side building blocks shared by the FP32 and FP16 GEMM kernels:
// parameter block, workgroup -> output-tile mapping, LDS swizzle and the
// fused write-back (alpha/beta, bias, ReLU).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ll {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Write-back variants. The write-back is fused into the GEMM kernel, so the
// product never makes a round trip through memory before bias and activation
// are applied (page "GEMM 优化详解", section "Level 6: Kernel Fusion").
enum Epi : int {
    EPI_GEMM_BETA0 = 0,  // C = alpha*acc            (C not read)
    EPI_GEMM_BETA = 1,   // C = alpha*acc + beta*C
    EPI_LINEAR = 2,      // Y = act(acc + bias[n])   (Y not read)
    EPI_ATOMIC = 3,      // C += alpha*acc atomically (one K-split's share)
};

struct GemmParams {
    const void *A;        // M x K, row-major, leading dimension lda (elements)
    const void *B;        // K x N, row-major, leading dimension ldb
    float *C;             // M x N, row-major, leading dimension ldc (in/out)
    const float *bias;    // N values or nullptr (EPI_LINEAR)
    int64_t lda, ldb, ldc;
    int M, N, K;
    float alpha, beta;
    int act;              // 0 none, 1 ReLU (EPI_LINEAR)
    int tiles_m, tiles_n; // output tiles along M and N
    int group_m;          // tile rows per group in the grouped ordering
    int k_split;          // K per split (a multiple of 64); K itself when not split
    int batch;            // batch items in this launch (grid z); 1 for a single product
    int64_t stride_a, stride_b, stride_c;  // byte distance between batch items (0: shared)
    int tile_base;        // index (in the grouped order) of this launch's first tile
    int grid_x;           // workgroups along x; 0: one per tile of the whole grid
    int sk_tiles;         // stream-K: the number of tiles shared out; 0: none
    int sk_block;         // stream-K: workgroups below this run whole tiles, the rest share
    // stream-K with a workspace (nullptr: none): a zero-filled FP32 tile per
    // shared tile, into which the sharing workgroups add their partial sums,
    // and an arrival counter per shared tile; the last contributor applies
    // the epilogue and clears both
    float *ws;
    int *ws_cnt;
};

// A 16-byte load from an address of any alignment. The target allows
// unaligned global accesses (the compiler itself emits one dwordx4 load for
// this copy even at 2-byte alignment).
template <class V>
__device__ __forceinline__ V load16(const void *src)
{
    static_assert(sizeof(V) == 16, "16-byte vector");
    V v;
    __builtin_memcpy(&v, src, 16);
    return v;
}

// Bounds a direct kernel's copies check (a template mask; see the launchers).
enum : int { CHK_M = 1, CHK_N = 2, CHK_K = 4 };

// K granularity of a stream-K share: a multiple of every kernel's stage depth.
constexpr int kSkUnit = 64;

// Strided batch: workgroups with blockIdx.z = i compute item i, whose A, B and
// C start stride_{a,b,c}*i bytes after the first item's (page "GEMM 优化详解",
// section "矩阵大小选择策略": small products are run as one batched GEMM).
// ceil(a / b) for a >= 0, b > 0, without the overflow of (a + b - 1) / b
// when a is close to INT_MAX.
__host__ __device__ constexpr int cdiv(int a, int b)
{
    return a / b + (a % b != 0);
}

__device__ __forceinline__ void select_batch(GemmParams &p)
{
    const int64_t z = blockIdx.z;
    p.A = static_cast<const char *>(p.A) + z * p.stride_a;
    p.B = static_cast<const char *>(p.B) + z * p.stride_b;
    p.C = reinterpret_cast<float *>(reinterpret_cast<char *>(p.C) + z * p.stride_c);
}

// Launch grid of a product: x = output tiles, y = K-splits, z = batch items.
inline dim3 gemm_grid(const GemmParams &p, int64_t ntiles)
{
    return dim3((unsigned)ntiles, (unsigned)cdiv(p.K, p.k_split), (unsigned)p.batch);
}

// The K range of this workgroup: split blockIdx.y covers
// [blockIdx.y*k_split, min(K, (blockIdx.y+1)*k_split)). Returns the offset;
// `k_len` receives the length.
__device__ __forceinline__ int split_range(const GemmParams &p, int &k_len)
{
    const int kb = blockIdx.y * p.k_split;
    k_len = min(p.K - kb, p.k_split);
    return kb;
}

// Workgroup -> output tile.
//
// The dispatcher hands consecutive workgroup ids to the 8 XCDs in turn, and
// each XCD has its own L2. block_index() renumbers the nwg ids so that the ids one
// XCD receives are consecutive; tile_of() walks tiles in groups of group_m
// tile rows, column by column, so that the tiles resident on one XCD at a
// time form a compact block and share their A rows and B columns in that
// XCD's L2.
__device__ __forceinline__ int block_index(int wg, int nwg)
{
    const int q = nwg >> 3, r = nwg & 7, x = wg & 7;
    return x * q + (x < r ? x : r) + (wg >> 3);
}

// Tile `lid` of the grouped order -> (tile_m, tile_n).
__device__ __forceinline__ void tile_of(const GemmParams &p, int lid, int &tm, int &tn)
{
    const int group = p.group_m * p.tiles_n;
    const int g = lid / group;
    const int first_m = g * p.group_m;
    const int rows = min(p.tiles_m - first_m, p.group_m);
    const int within = lid - g * group;
    tm = first_m + within % rows;
    tn = within / rows;
}

// The tile of this workgroup in a data-parallel launch (tiles tile_base ..),
// or of a whole-tile workgroup (blockIdx.x < sk_block) of a stream-K launch.
__device__ __forceinline__ void tile_coords(const GemmParams &p, int &tm, int &tn)
{
    const int nwg = p.sk_tiles > 0 ? p.sk_block : (int)gridDim.x;
    tile_of(p, p.tile_base + block_index(blockIdx.x, nwg), tm, tn);
}

// Stream-K: the sk_tiles tiles after the whole ones (from tile_base + sk_block
// on) are cut into units of kSkUnit k-values, and sharing workgroup w (of the
// gridDim.x - sk_block from sk_block on) takes the w-th of equal contiguous
// runs of those (tile, unit) pairs -- less than one tile's worth, so at most
// two segments. Segment `seg` of this workgroup: returns false if there is
// none, else its tile and k-range [kb, kb + k_len).
__device__ __forceinline__ bool sk_segment(const GemmParams &p, int seg, int &tm, int &tn, int &kb,
                                           int &k_len, int *shared_tile = nullptr)
{
    const int units = cdiv(p.K, kSkUnit);
    const int64_t total = (int64_t)p.sk_tiles * units;
    const int64_t w = (int64_t)blockIdx.x - p.sk_block, nw = (int64_t)gridDim.x - p.sk_block;
    int64_t u0 = total * w / nw;
    const int64_t u1 = total * (w + 1) / nw;
    for (int s = 0; s < seg && u0 < u1; ++s)
        u0 = (u0 / units + 1) * units;   // skip to the next tile's first unit
    if (u0 >= u1)
        return false;
    const int t = (int)(u0 / units), lo = (int)(u0 % units);
    const int64_t tile_end = (int64_t)(t + 1) * units;
    const int hi = (int)((u1 < tile_end ? u1 : tile_end) - (int64_t)t * units);
    tile_of(p, p.tile_base + p.sk_block + t, tm, tn);
    kb = lo * kSkUnit;
    k_len = min(p.K, hi * kSkUnit) - kb;
    if (shared_tile != nullptr)
        *shared_tile = t;
    return true;
}

// The number of sharing workgroups whose runs meet shared tile t. Workgroup w
// covers units [total*w/nw, total*(w+1)/nw), every run at least one unit
// long (the planner shares out at least as many units as it has sharing
// workgroups), so the workgroup holding unit u is floor(((u+1)*nw - 1)/total).
__device__ __forceinline__ int sk_contributors(const GemmParams &p, int t)
{
    const int64_t units = cdiv(p.K, kSkUnit);
    const int64_t total = (int64_t)p.sk_tiles * units;
    const int64_t nw = (int64_t)gridDim.x - p.sk_block;
    auto owner = [&](int64_t u) { return ((u + 1) * nw - 1) / total; };
    return (int)(owner((int64_t)(t + 1) * units - 1) - owner((int64_t)t * units) + 1);
}

// XOR swizzle of 16-byte chunks inside an LDS row of ROW_BYTES bytes. The
// LDS has 64 banks of 4 bytes and serves a 128-bit read 16 lanes per cycle,
// so 16 lanes reading the same logical chunk of 16 consecutive rows must hit
// 16 different 16-byte bank groups of the 256-byte bank line: RPL rows share
// a line, and the chunk index is XORed with the row's line number (mod the
// chunks per row, at most 16). (Measured with the bank-conflict counter: for
// 64-byte rows, XOR by (row/4)%4 is conflict-free, by (row/2)%4 two-way.)
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int row)
{
    constexpr int CPR = ROW_BYTES / 16;
    constexpr int RPL = ROW_BYTES >= 256 ? 1 : 256 / ROW_BYTES;
    constexpr int MASK = (CPR < 16 ? CPR : 16) - 1;
    return (row / RPL) & MASK;
}

// ---- direct global -> LDS copies ----

// Byte address of an LDS object.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// global_load_lds_dwordx4: this lane's 16 bytes at `src` are written to LDS
// byte address lds_base + 16*lane, without passing through registers (so one
// wave instruction fills one contiguous KiB). Issued as inline assembly so the
// compiler does not treat it as an LDS store that every later barrier must
// wait for; the caller counts these copies itself (s_waitcnt vmcnt) before
// the barrier that publishes them. Lanes masked off by EXEC copy nothing. One
// wait state separates the scalar write of M0 from the load that reads it
// (the compiler's hazard checks do not look inside inline assembly).
__device__ __forceinline__ void lds_dma_16(const void *src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(src)
                 : "memory", "m0");
}

// Sixteen zero bytes in device memory: the source of every direct copy whose
// elements lie outside the matrix. Such a copy is still issued on every lane
// (so each wave's vmcnt counts a fixed number of copies per stage) and fills
// its LDS slot with zeros.
static __device__ __attribute__((aligned(16))) const uint32_t kZeroChunk[4] = {0u, 0u, 0u, 0u};

template <class T>
__device__ __forceinline__ const T *zero_chunk()
{
    return reinterpret_cast<const T *>(kZeroChunk);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
#define LL_VMCNT(n) ((((n) & 0xF) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 3) << 14)))

// The fused write-back of one MFMA accumulator block (page "GEMM 优化详解",
// "Level 6: Kernel Fusion": alpha/beta, or bias by output column then ReLU,
// applied to the accumulators before the single store).
//
// Accumulator layouts (wave64): v_mfma_f32_32x32x* (MF = 32, 16 registers):
// lane l holds column l % 32, register r row 8*(r/4) + 4*(l/32) + r%4;
// v_mfma_f32_16x16x* (MF = 16, 4 registers): lane l holds column l % 16,
// register r row 4*(l/16) + r.
//
// The values are computed first, with the loads they need (beta*C, the
// bias) issued together from in-bounds addresses (row and column clamped to
// the matrix), and stored afterwards. A masked store is a branch, and a load
// whose result is first used inside one would make every later store wait
// for all earlier memory operations (loads and stores share one counter), so
// no store may depend on a load that was not consumed before the first store.
// Rows of a block that lies inside the matrix (a uniform test) need no mask.
template <int EPI, int MF, class Acc>
__device__ __forceinline__ void write_acc(const GemmParams &p, const Acc &acc, int row0, int col0,
                                          int lane)
{
    constexpr int R = MF == 32 ? 16 : 4;
    const int col = col0 + (lane % MF);
    const int rbase = row0 + (lane / MF) * 4;
    auto row = [&](int r) { return MF == 32 ? rbase + ((r >> 2) << 3) + (r & 3) : rbase + r; };
    const bool full = row0 <= p.M - MF;
    const bool col_ok = col < p.N;
    float *dst = p.C + col;
    auto put = [&](int r, float v) {
        if (col_ok && (full || row(r) < p.M))
            dst[(int64_t)row(r) * p.ldc] = v;
    };
    if (EPI == EPI_ATOMIC) {
        // split-K / stream-K share: every contributor adds alpha times its
        // partial sum; C was prepared (beta*C, or the bias) beforehand
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (col_ok && row(r) < p.M)
                __hip_atomic_fetch_add(dst + (int64_t)row(r) * p.ldc, p.alpha * acc[r],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (EPI == EPI_GEMM_BETA) {
        // beta*C in groups of G rows (loads, then stores): at most G values of
        // C are held at once
        constexpr int G = R < 4 ? R : 4;
        const int64_t cc = col_ok ? col : p.N - 1;
#pragma unroll
        for (int g = 0; g < R; g += G) {
            float c[G];
#pragma unroll
            for (int r = 0; r < G; ++r) {
                const int rr = row(g + r);
                c[r] = p.C[(int64_t)(rr < p.M ? rr : p.M - 1) * p.ldc + cc];
            }
#pragma unroll
            for (int r = 0; r < G; ++r)
                c[r] = __builtin_fmaf(p.alpha, acc[g + r], p.beta * c[r]);
#pragma unroll
            for (int r = 0; r < G; ++r)
                put(g + r, c[r]);
        }
    } else if (EPI == EPI_LINEAR) {
        const float bv = p.bias != nullptr ? p.bias[col_ok ? col : p.N - 1] : 0.0f;
        float v[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float y = acc[r] + bv;
            v[r] = (p.act == 1 && !(y > 0.0f)) ? 0.0f : y;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            put(r, v[r]);
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
            put(r, p.alpha * acc[r]);
    }
}

template <int EPI>
__device__ __forceinline__ void write_block(const GemmParams &p, const f32x16 &acc,
                                            int row0, int col0, int lane)
{
    write_acc<EPI, 32>(p, acc, row0, col0, lane);
}

// LDS floats one wave needs for write_block_x4.
constexpr int kStageFloats = 608;

// The fused write-back of one 32x32 block with 128-bit stores (C 16-byte
// aligned, ldc a multiple of 4). A lane holds one column of the block, so
// each half of 16 rows goes through `stage` (kStageFloats floats of LDS
// owned by this wave) to give every lane four consecutive columns of two
// rows: local row lr sits at float (lr + lr/4)*32, so the two half-waves of
// a 32-bit write (rows lr and lr+4) hit opposite halves of the 64 banks and
// the 16 lanes of a 128-bit read (rows 2i, 2i+1) eight 16-byte groups each.
// The epilogue is the one of write_acc; four columns that cross N are
// stored one by one.
// The fused epilogue of four consecutive outputs C(row, col .. col+3), whose
// accumulated sums are v (cv: their beta*C inputs, for EPI_GEMM_BETA), stored
// with one 128-bit access when all four lie inside N, else one by one; rows
// outside M store nothing. EPI_ATOMIC adds alpha*v atomically.
template <int EPI>
__device__ __forceinline__ void finish4(const GemmParams &p, f32x4 v, int row, int col,
                                        const f32x4 &cv)
{
    if (row >= p.M)
        return;
    const bool vec = col + 3 < p.N;
    float *dst = p.C + (int64_t)row * p.ldc + col;
    if (EPI == EPI_ATOMIC) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (col + e < p.N)
                __hip_atomic_fetch_add(dst + e, p.alpha * v[e], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (EPI == EPI_GEMM_BETA) {
            v[e] = __builtin_fmaf(p.alpha, v[e], p.beta * cv[e]);
        } else if (EPI == EPI_LINEAR) {
            const float bv = p.bias != nullptr ? p.bias[col + e < p.N ? col + e : p.N - 1] : 0.0f;
            const float y = v[e] + bv;
            v[e] = (p.act == 1 && !(y > 0.0f)) ? 0.0f : y;
        } else {
            v[e] = p.alpha * v[e];
        }
    }
    if (vec) {
        *reinterpret_cast<f32x4 *>(dst) = v;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (col + e < p.N)
                dst[e] = v[e];
    }
}

// The four values of C at (row, col .. col+3), the row and columns clamped to
// the matrix (beta*C inputs of finish4).
__device__ __forceinline__ f32x4 load_c4(const GemmParams &p, int row, int col)
{
    const int64_t rr = row < p.M ? row : p.M - 1;
    f32x4 c;
    if (col + 3 < p.N) {
        c = *reinterpret_cast<const f32x4 *>(&p.C[rr * p.ldc + col]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            c[e] = p.C[rr * p.ldc + (col + e < p.N ? col + e : p.N - 1)];
    }
    return c;
}

// The values of C (beta*C) that write_block_x4 combines into this lane's
// stores, index 2*h + j: rows row0 + 16h + 8j + lane/8, columns col0 +
// 4*(lane%8) .. +3 (rows and columns clamped to the matrix). A kernel may
// load them early, so their latency hides behind the product.
__device__ __forceinline__ void load_c_x4(const GemmParams &p, int row0, int col0, int lane,
                                          f32x4 (&cv)[4])
{
    const int col = col0 + ((lane & 7) << 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = row0 + 16 * (i >> 1) + 8 * (i & 1) + (lane >> 3);
        const int64_t rr = row < p.M ? row : p.M - 1;
        if (col + 3 < p.N) {
            cv[i] = *reinterpret_cast<const f32x4 *>(&p.C[rr * p.ldc + col]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                cv[i][e] = p.C[rr * p.ldc + (col + e < p.N ? col + e : p.N - 1)];
        }
    }
}

template <int EPI, bool PRE = false>
__device__ __forceinline__ void write_block_x4(const GemmParams &p, const f32x16 &acc, int row0,
                                               int col0, int lane, float *stage,
                                               const f32x4 *cpre = nullptr)
{
    const int c = lane & 31, rb = (lane >> 5) << 2;
    const int cq = (lane & 7) << 2, rq = lane >> 3;
    const int col = col0 + cq;
    const bool vec = col + 3 < p.N;
    // beta*C of both halves, loaded before the first LDS round trip (or
    // earlier, by the caller: PRE)
    f32x4 cv[4];
    if (EPI == EPI_GEMM_BETA) {
        if constexpr (PRE) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                cv[i] = cpre[i];
        } else {
            load_c_x4(p, row0, col0, lane, cv);
        }
    }
    f32x4 bv = {0.0f, 0.0f, 0.0f, 0.0f};
    if (EPI == EPI_LINEAR && p.bias != nullptr) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            bv[e] = p.bias[col + e < p.N ? col + e : p.N - 1];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int lr = ((r >> 2) << 3) + rb + (r & 3);
            stage[(lr + (lr >> 2)) * 32 + c] = acc[8 * h + r];
        }
        f32x4 v[2];
        int row[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int lr = rq + 8 * j;
            v[j] = *reinterpret_cast<const f32x4 *>(&stage[(lr + (lr >> 2)) * 32 + cq]);
            row[j] = row0 + 16 * h + lr;
        }
        if (EPI == EPI_GEMM_BETA) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[j][e] = __builtin_fmaf(p.alpha, v[j][e], p.beta * cv[2 * h + j][e]);
        } else if (EPI == EPI_LINEAR) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y = v[j][e] + bv[e];
                    v[j][e] = (p.act == 1 && !(y > 0.0f)) ? 0.0f : y;
                }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[j][e] = p.alpha * v[j][e];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (row[j] >= p.M)
                continue;
            float *dst = p.C + (int64_t)row[j] * p.ldc + col;
            if (vec) {
                *reinterpret_cast<f32x4 *>(dst) = v[j];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col + e < p.N)
                        dst[e] = v[j][e];
            }
        }
    }
}

template <int EPI>
__device__ __forceinline__ void write_block16(const GemmParams &p, const f32x4 &acc,
                                              int row0, int col0, int lane)
{
    write_acc<EPI, 16>(p, acc, row0, col0, lane);
}

// The skinny kernels' helpers. dpp_row_sum16: the sum of v over each row of
// 16 lanes, in every lane of the row (quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror, row_mirror). skinny_store: one output value
// through the epilogue (alpha*a, + beta*C, bias and ReLU, or an atomic
// partial sum of a K-split).
__device__ __forceinline__ float dpp_row_sum16(float v)
{
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, false));
    return v;
}

template <int EPI>
__device__ __forceinline__ void skinny_store(const GemmParams &p, int row, int col, float a)
{
    float *dst = p.C + (int64_t)row * p.ldc + col;
    if constexpr (EPI == EPI_ATOMIC) {
        __hip_atomic_fetch_add(dst, p.alpha * a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (EPI == EPI_GEMM_BETA) {
        *dst = __builtin_fmaf(p.alpha, a, p.beta * *dst);
    } else if constexpr (EPI == EPI_LINEAR) {
        const float y = a + (p.bias != nullptr ? p.bias[col] : 0.0f);
        *dst = (p.act == 1 && !(y > 0.0f)) ? 0.0f : y;
    } else {
        *dst = p.alpha * a;
    }
}

}  // namespace ll
