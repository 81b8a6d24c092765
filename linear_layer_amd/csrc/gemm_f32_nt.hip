// The FP32 kernels' instances for B given N-by-K (the _nt entry points):
// gemm_f32.hip built a second time, as a translation unit of its own, so that
// the two B layouts' instances compile in parallel.
#define LL_F32_NT_UNIT 1
#include "gemm_f32.hip"
