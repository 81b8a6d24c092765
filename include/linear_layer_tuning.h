/*
 * linear_layer_tuning.h — plan overrides of the MI355X GEMM library, for
 * benchmarks, sweeps and tests. Not for product code.
 *
 * By default every call of linear_layer.h picks its tile shape, K-split and
 * stream-K share itself (see ll_chosen_tile there). The calls below replace
 * that choice PROCESS-WIDE: once set, an override steers every later call of
 * the matching entry points from every thread and on every stream of the
 * process, until it is reset to -1. A forced K-split or stream-K share also
 * changes the summation order of the products it applies to (still within
 * the error bound; integer-valued inputs stay exact). Each call reads all
 * overrides at once, as one consistent set, so a setter running on another
 * thread never leaves a call with a mix of old and new values; which of the
 * two sets a concurrent call sees is unspecified.
 *
 * They touch only host memory and never the GPU. Each returns LL_OK or
 * LL_ERR_INVALID_VALUE (the value out of range; nothing changes then).
 */
#ifndef LINEAR_LAYER_TUNING_H
#define LINEAR_LAYER_TUNING_H

#include "linear_layer.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Force tile `tile` (0 .. ll_num_tiles(dtype)-1) for every later call of
 * that dtype; -1 restores the automatic choice. LL_DTYPE_F16 covers both
 * 16-bit formats (binary16 and bfloat16) and both B layouts. */
int ll_set_tile(int dtype, int tile);

/* Force `splits` K-splits (1 .. 16; the split length is rounded up to a
 * multiple of 64, or of 128 on the 16-bit skinny tile, and to whole stages
 * of every slice on the K-sliced tiles, so small K may use fewer) for every
 * later call of any dtype; -1 restores the automatic choice (which for the
 * skinny tiles may use up to 64). */
int ll_set_split_k(int splits);

/* Stream-K for leftover tiles: -1 automatic (default), 0 never, 1 whenever
 * the shape allows it (a forced K-split takes precedence; K-sliced tiles and
 * the 128x128 and 64x64 16-bit tiles never share out). */
int ll_set_stream_k(int mode);

/* Lower the workspace linear_bias_act_noalloc may use to `bytes` (0 ..
 * LL_NOALLOC_SCRATCH_BYTES) for every later call, so that its refusal of
 * larger needs can be exercised on a device where no plan reaches the full
 * array; -1 restores the full array. */
int ll_set_noalloc_limit(int64_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* LINEAR_LAYER_TUNING_H */
