/*
 * linear_layer.h — C ABI of the MI355X (gfx950) GEMM / fully-connected library.
 *
 * Every entry point enqueues work on the caller's HIP stream and returns at
 * once; it never synchronises, never allocates device memory and keeps no
 * state between calls beyond a read-only cache of device properties. All
 * matrix pointers are DEVICE pointers owned by the caller. Matrices are
 * row-major: element (r, c) of a matrix with leading dimension ld is at
 * ptr[r * ld + c]. Dimensions and leading dimensions are int; offsets are
 * computed in 64 bits inside.
 *
 * Errors are never fatal: no abort, no exception crosses this boundary. Each
 * call returns one of the LL_* status codes below. Argument errors are found
 * on the host before anything is enqueued; faults during execution surface
 * on the stream like those of any other kernel.
 *
 * `stream` is a hipStream_t passed as void* (NULL = the default stream), so
 * that this header needs no HIP header.
 */
#ifndef LINEAR_LAYER_H
#define LINEAR_LAYER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define LL_OK 0
#define LL_ERR_INVALID_VALUE 1   /* negative dimension, leading dimension too small,
                                    NULL pointer that would be dereferenced, pointer not
                                    aligned to its element size, unknown activation,
                                    an output range overlapping an input range, or an
                                    output whose tiles exceed one launch's grid (only
                                    extreme shapes: M or N within about 2^8 of 2^31
                                    with the other one small) */
#define LL_ERR_NO_DEVICE 2       /* no HIP device is current / visible */
#define LL_ERR_UNSUPPORTED_ARCH 3/* the current device is not gfx950 (MI355X class) */
#define LL_ERR_LAUNCH 4          /* the HIP runtime reported an error at launch */

/* Activations for linear_bias_act. */
#define LL_ACT_NONE 0
#define LL_ACT_RELU 1

/*
 * gemm_f32 — C = alpha * A * B + beta * C in FP32.
 *
 * Defined on page "GEMM 优化详解" (GEMM optimisation in detail), section
 * "GEMM 基础理论 / 数学定义" (mathematical definition): the general form
 * C = alpha*A*B + beta*C with A M-by-K, B K-by-N, C M-by-N and
 * C(m,n) = sum_k A(m,k) * B(k,n). The same sum is on page "第5章-基础Kernel",
 * section 1.1.
 *
 *   M, N, K   >= 0. M == 0 or N == 0: returns LL_OK, touches nothing.
 *   A         M-by-K fp32, lda >= max(1, K). Read only if K > 0 and alpha != 0.
 *   B         K-by-N fp32, ldb >= max(1, N). Read only if K > 0 and alpha != 0.
 *   C         M-by-N fp32, ldc >= max(1, N), in/out. Read only if beta != 0, so
 *             with beta == 0 any bit pattern (NaN included) in C is ignored.
 *   alpha, beta  fp32 scalars (host values). K == 0 or alpha == 0 gives C = beta*C.
 *   stream    hipStream_t (void*), NULL for the default stream.
 *
 * Products are accumulated in FP32 on the matrix cores (MFMA), in an order of
 * the kernel's choosing. C must not overlap A or B. Pointers need only be
 * 4-byte aligned; 16-byte aligned pointers with lda, ldb, ldc, K and N all
 * multiples of 4 take the direct-to-LDS kernels; anything else the
 * register-staged kernels, which load 128-bit chunks at any alignment and
 * the chunk that crosses K or N element by element.
 */
int gemm_f32(int M, int N, int K, float alpha,
             const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, void *stream);

/*
 * gemm_f16f32 — C = alpha * A * B + beta * C with IEEE binary16 A and B,
 * FP32 accumulation and FP32 C.
 *
 * The FP16-input / FP32-accumulate product of page
 * "GPU架构下的矩阵乘法深入优化" (in-depth matrix-multiply optimisation on
 * GPU architecture), section 6 (tensor-core implementation), in the general
 * form of page "GEMM 优化详解", section "GEMM 基础理论 / 数学定义".
 *
 *   A  M-by-K binary16 bit patterns (uint16_t), lda >= max(1, K).
 *   B  K-by-N binary16 bit patterns, ldb >= max(1, N).
 *   C  M-by-N fp32, ldc >= max(1, N).
 * Every other argument, rule and error as gemm_f32. Pointers to A and B need
 * only be 2-byte aligned; the direct-to-LDS kernels need 16-byte aligned
 * pointers and lda, ldb, K, N multiples of 8 (ldc a multiple of 4), other
 * operands run the register-staged kernels.
 */
int gemm_f16f32(int M, int N, int K, float alpha,
                const uint16_t *A, int lda, const uint16_t *B, int ldb,
                float beta, float *C, int ldc, void *stream);

/*
 * gemm_bf16f32 — C = alpha * A * B + beta * C with bfloat16 A and B, FP32
 * accumulation and FP32 C.
 *
 * Page "GEMM 优化详解", section "进一步优化方向" (further directions),
 * item "Tensor Core (WMMA)": the matrix units take FP16 or BF16 inputs. Same
 * product as gemm_f16f32 with the inputs in bfloat16 (1 sign, 8 exponent,
 * 7 fraction bits) instead of binary16.
 *
 *   A  M-by-K bfloat16 bit patterns (uint16_t), lda >= max(1, K).
 *   B  K-by-N bfloat16 bit patterns, ldb >= max(1, N).
 * Every other argument, rule and error as gemm_f16f32 (same kernels and tile
 * shapes, selected by LL_DTYPE_F16 below).
 */
int gemm_bf16f32(int M, int N, int K, float alpha,
                 const uint16_t *A, int lda, const uint16_t *B, int ldb,
                 float beta, float *C, int ldc, void *stream);

/*
 * linear_bias_act — Y = act(X * W + bias), the fused fully-connected layer.
 *
 * Page "GEMM 优化详解", table "为什么 GEMM 重要" (an FC layer is
 * Y = X*W + b) and section "Level 6: Kernel Fusion" (the bias, indexed by
 * output column, and then the ReLU are applied in the GEMM's write-back, so
 * the intermediate never goes to memory). The page's four flag combinations
 * map to (bias != NULL) x (act).
 *
 *   X     M-by-K fp32 (a batch of M input rows), ldx >= max(1, K).
 *   W     K-by-N fp32 weights, row-major K-by-N, ldw >= max(1, N).
 *   bias  N fp32 values, or NULL for no bias.
 *   act   LL_ACT_NONE or LL_ACT_RELU; ReLU maps y <= 0 (and NaN) to +0.0.
 *   Y     M-by-N fp32 output, ldy >= max(1, N); never read.
 * K == 0 gives Y = act(bias) (or act(0)). Y must not overlap X, W or bias.
 * Alignment rules as gemm_f32.
 */
int linear_bias_act(int M, int N, int K,
                    const float *X, int ldx, const float *W, int ldw,
                    const float *bias, int act,
                    float *Y, int ldy, void *stream);

/*
 * Transposed-B forms: B (or W) is given N-by-K, row-major, leading dimension
 * ldb >= max(1, K) (ldw for W), so that its element (k, n) is at B[n*ldb + k]:
 *
 *   gemm_f32_nt, gemm_f16f32_nt, gemm_bf16f32_nt:  C = alpha * A * B^T + beta * C
 *   linear_bias_act_nt:                            Y = act(X * W^T + bias)
 *
 * This is how a fully-connected weight is usually stored ([out][in]) and the
 * shape of products such as Q * K^T (page "GEMM 优化详解", table
 * "为什么 GEMM 重要"). B is then k-contiguous like A and the kernels stage and
 * read it exactly like A. Every other argument, rule and error is that of the
 * corresponding function above; the 128-bit kernels need ldb (ldw) to be a
 * multiple of 4 (fp32) or 8 (16-bit) instead of N.
 */
int gemm_f32_nt(int M, int N, int K, float alpha,
                const float *A, int lda, const float *B, int ldb,
                float beta, float *C, int ldc, void *stream);
int gemm_f16f32_nt(int M, int N, int K, float alpha,
                   const uint16_t *A, int lda, const uint16_t *B, int ldb,
                   float beta, float *C, int ldc, void *stream);
int gemm_bf16f32_nt(int M, int N, int K, float alpha,
                    const uint16_t *A, int lda, const uint16_t *B, int ldb,
                    float beta, float *C, int ldc, void *stream);
int linear_bias_act_nt(int M, int N, int K,
                       const float *X, int ldx, const float *W, int ldw,
                       const float *bias, int act,
                       float *Y, int ldy, void *stream);

/*
 * linear_bias_act_ws — the fused layer of linear_bias_act (w_layout
 * LL_W_K_BY_N) or linear_bias_act_nt (LL_W_N_BY_K) with a caller-provided
 * workspace, so that the bias and ReLU stay fused into the write-back of
 * every output tile (page "GEMM 优化详解", "Level 6: Kernel Fusion").
 *
 * Without a workspace, a plan that shares the K range of leftover tiles out
 * over several workgroups (stream-K; e.g. 2047 x 11008 x 4096, 88 of 344
 * tiles) adds their partial sums atomically into Y, which a pass fills with
 * the bias first and another pass finishes with the ReLU: three launches.
 * With a workspace of at least ll_linear_workspace_size bytes, the partial
 * sums go to a workspace tile and the last workgroup to contribute to a tile
 * applies bias and ReLU and writes it: one launch, no pass over Y.
 *
 *   workspace        device memory owned by the caller, 256-byte aligned, not
 *                    overlapping X, W, bias or Y; it must hold zeros before
 *                    its first use (e.g. hipMemset to 0), and every call that
 *                    completes leaves it holding zeros again. NULL (with
 *                    workspace_bytes 0) or a workspace smaller than the plan
 *                    needs: the three-launch plan runs, with the same result
 *                    up to the order of the atomic additions.
 *   workspace_bytes  its size in bytes.
 * Calls that use one workspace must not overlap in time (on one stream they
 * never do); calls with different workspaces are independent. Everything
 * else as linear_bias_act / linear_bias_act_nt; LL_ERR_INVALID_VALUE also for
 * an unknown w_layout or a misaligned or overlapping workspace.
 */
#define LL_W_K_BY_N 0
#define LL_W_N_BY_K 1
int linear_bias_act_ws(int M, int N, int K,
                       const float *X, int ldx, const float *W, int ldw, int w_layout,
                       const float *bias, int act,
                       float *Y, int ldy, void *workspace, int64_t workspace_bytes,
                       void *stream);
/* Bytes of workspace linear_bias_act_ws uses for this shape on a device with
 * num_cus compute units (num_cus <= 0: 256), assuming 128-bit-aligned
 * operands (other calls use less or none); 0 if its plan needs none; -1 for
 * a negative size or an unknown w_layout or act. Honours the overrides of
 * linear_layer_tuning.h. For 2047 x 11008 x 4096 on 256 CUs: 88 tiles of
 * 256 KiB plus counters, about 22 MiB. */
int64_t ll_linear_workspace_size(int M, int N, int K, int w_layout, int act, int num_cus);

/*
 * linear_bias_act_noalloc — linear_bias_act_ws for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the workspace is the library's own
 * static device array of LL_NOALLOC_SCRATCH_BYTES (one per GPU, held until
 * the process ends), so the call allocates nothing and takes no workspace
 * argument. The array covers every plan on a device of up to 256 compute
 * units (a stream-K plan shares out less than one round of tiles: at most
 * 64 MiB of partial tiles plus their counters). A shape whose plan needs more
 * workspace than that (see ll_linear_workspace_size) returns
 * LL_ERR_INVALID_VALUE and runs nothing.
 * Every call on one GPU uses that GPU's single array: calls that overlap in
 * time on one GPU (other streams, other threads) race and give wrong
 * results; calls on one stream never overlap. Each call leaves the array
 * zero-filled, as the next one needs it. The array used is the current
 * device's, so `stream` must belong to the current device (else
 * LL_ERR_INVALID_VALUE). Arguments and results otherwise as
 * linear_bias_act_ws.
 */
#define LL_NOALLOC_SCRATCH_BYTES (65ll << 20)
int linear_bias_act_noalloc(int M, int N, int K,
                            const float *X, int ldx, const float *W, int ldw, int w_layout,
                            const float *bias, int act,
                            float *Y, int ldy, void *stream);

/*
 * Strided-batched products (page "GEMM 优化详解", section "矩阵大小选择策略":
 * small matrices are best run as one batched GEMM). For i in [0, batch):
 *
 *   C_i = alpha * A_i * op(B_i) + beta * C_i,   op(B) = B (trans_b 0) or B^T (trans_b 1)
 *
 * with A_i = A + i*stride_a, B_i = B + i*stride_b, C_i = C + i*stride_c
 * (strides in ELEMENTS of the operand's type). Each item follows the rules of
 * gemm_f32 / gemm_f16f32 / gemm_bf16f32 (trans_b 0: B_i K-by-N, ldb >= N;
 * trans_b 1: B_i N-by-K, ldb >= K). A stride of 0 shares one A or B among all
 * items; C items must not overlap (stride_c >= (M-1)*ldc + N when batch > 1),
 * and the address range spanned by all C items must not meet that of A's or
 * B's items. batch == 0 returns LL_OK with no launch; negative strides or
 * batch, or trans_b outside {0, 1}, give LL_ERR_INVALID_VALUE. All items run
 * in one launch (several when batch exceeds 65535), their tiles sharing the
 * CUs. The 128-bit kernels also need stride_a, stride_b (in bytes) and
 * stride_c*4 to be multiples of 16.
 */
int gemm_f32_batched(int trans_b, int M, int N, int K, float alpha,
                     const float *A, int lda, int64_t stride_a,
                     const float *B, int ldb, int64_t stride_b,
                     float beta, float *C, int ldc, int64_t stride_c,
                     int batch, void *stream);
int gemm_f16f32_batched(int trans_b, int M, int N, int K, float alpha,
                        const uint16_t *A, int lda, int64_t stride_a,
                        const uint16_t *B, int ldb, int64_t stride_b,
                        float beta, float *C, int ldc, int64_t stride_c,
                        int batch, void *stream);
int gemm_bf16f32_batched(int trans_b, int M, int N, int K, float alpha,
                         const uint16_t *A, int lda, int64_t stride_a,
                         const uint16_t *B, int ldb, int64_t stride_b,
                         float beta, float *C, int ldc, int64_t stride_c,
                         int batch, void *stream);

/* A static, human-readable string for a status code (never NULL). */
const char *ll_status_string(int status);

/*
 * Tile and K-split selection. Each data type has a small set of block-tile
 * shapes; by default the library picks, per call, a tile shape and a number
 * of K-splits from M, N, K and the CU count, minimising an estimate of the
 * run time: large problems get the largest tiles, and problems too small to
 * fill the device get smaller tiles or several workgroups along K (the
 * size-dependent strategy of page "GEMM 优化详解", section "矩阵大小选择策略"
 * (matrix-size strategy), re-derived for 256 CUs).
 *
 * With K-splits (split-K), each split computes alpha * A[:, Ks] * B[Ks, :]
 * for its range Ks of K and adds it into C with hardware FP32 atomics, after
 * a pass that scales C by beta (for linear_bias_act: fills Y with the bias,
 * then applies the ReLU in a pass afterwards). The result is the same sum in
 * a different, run-dependent order; it still allocates nothing.
 *
 * Some shapes split K inside the workgroup instead ("K-sliced" tiles, named
 * *_k4 and *_k2: f32_64x64_k4, f32_128x128_k2, f16_128x128_k2): the
 * workgroup's slices sum disjoint stage-aligned K ranges and add their
 * partial tiles through on-chip memory in a fixed order, so the result does
 * not depend on the run; no atomics, no extra pass. They serve problems too
 * small to fill the device (e.g. 1024^3), and the automatic choice takes them
 * only when each slice gets at least 8 stages (a forced tile is always used).
 *
 * FP32 products of at most 32 rows of A may take f32_32x128: two-wave
 * workgroups of 32x128, up to four per CU, for the rows that the 64-row
 * tiles would mostly pad.
 *
 * Single FP32 products with a few rows of A (at most 4, or at most 8 when B
 * holds at least 2^25 values) are bound by reading B from HBM, not by the
 * matrix units (page "GEMM 优化详解", table "计算复杂度分析": the intensity
 * 2MNK / (MK + KN + MN) / 4 is about M/2 FLOP per byte). They take the tile
 * f32_16x256_skinny: vector FMAs over 256 columns of C per workgroup with
 * A's rows staged in LDS, and up to 64 K-splits (added atomically, framed by
 * the same passes as above). Forced on more rows it walks them 16 at a time.
 * Single 16-bit products of one row of A with B given N-by-K and holding at
 * least 2^25 values likewise take f16_16x256_skinny_nt: dot2 instructions
 * (two 16-bit products added into an FP32 sum) over 256 columns of C per
 * workgroup, the same K-splits; forced with B given K-by-N, the 128x128 tile
 * runs in its place.
 *
 * The calls below report the choice; they touch only host memory and never
 * the GPU. (linear_layer_tuning.h declares process-wide overrides of the
 * choice for benchmarks and tests.)
 */
#define LL_DTYPE_F32 0 /* gemm_f32, linear_bias_act and their _nt forms */
#define LL_DTYPE_F16 1 /* gemm_f16f32, gemm_bf16f32 and their _nt forms */
/* Flags the ll_chosen_* queries accept OR-ed into `dtype`:
 * LL_PLAN_RELU: linear_bias_act with the ReLU, whose K-split and stream-K
 * plans pay for one more pass over Y (LL_DTYPE_F32 only);
 * LL_PLAN_B_NK: the _nt form (B given N-by-K; the FP32 skinny kernel's
 * K-split count and the 16-bit skinny kernel's choice depend on it);
 * LL_PLAN_UNALIGNED: operands that do not allow the 128-bit-load kernels
 * (a base not 16-byte aligned, or a leading dimension, K or N not a multiple
 * of 4 (fp32) or 8 (16-bit)): no stream-K, and the tiles that exist only as
 * 128-bit-load kernels (the K-sliced ones, f32_32x128 and f16_192x192_direct)
 * are not chosen automatically. */
#define LL_PLAN_RELU 0x100
#define LL_PLAN_B_NK 0x200
#define LL_PLAN_UNALIGNED 0x400

/* Number of tile shapes for a data type (0 for an unknown dtype). */
int ll_num_tiles(int dtype);
/* Name of a tile shape, e.g. "f32_256x256" ("" if out of range). Static string. */
const char *ll_tile_name(int dtype, int tile);
/* The tile / the number of K-splits the library would use for `batch`
 * M-by-N outputs (batch 1: a single product) with inner dimension K on a
 * device with num_cus compute units (num_cus <= 0: 256), honouring the
 * overrides and the LL_PLAN_* flags in dtype. -1 for an unknown dtype or
 * flag, or batch < 1. */
int ll_chosen_tile(int dtype, int M, int N, int K, int batch, int num_cus);
int ll_chosen_split_k(int dtype, int M, int N, int K, int batch, int num_cus);

/*
 * Stream-K (single products with 128-bit-aligned operands; FP32 on tiles
 * without K-slices, 16-bit on the 256x256 tile):
 * when the output tiles do not fill a whole number of rounds of the CUs, the
 * planner may run the full rounds tile by tile and share the leftover tiles'
 * K range out evenly over one round of workgroups, whose partial sums are
 * added atomically into C (prepared with beta*C, or the bias, beforehand;
 * the ReLU applied afterwards). Like a K-split, this makes the summation
 * order of those tiles run-dependent (still within the error bound; integer
 * inputs stay exact); it allocates nothing.
 *   ll_chosen_stream_k: the number of tiles the plan shares out (0: none);
 *   dtype and flags as for ll_chosen_tile; -1 for an unknown dtype or flag,
 *   or batch < 1.
 */
int ll_chosen_stream_k(int dtype, int M, int N, int K, int batch, int num_cus);

#ifdef __cplusplus
}
#endif

#endif /* LINEAR_LAYER_H */
