// Instantiations of the fused-epilogue GEMM kernels for one output type (EPI_F32); one file per
// output type so that the four compile in parallel.
#include "gemm_kernels.h"

namespace sfp8 {
int gemm_fused_f32(int mode, int fa, int fb, const uint8_t* A, const uint8_t* B, const void* sa, const void* sb,
                  const EpiParams& ep, int M, int N, int K, hipStream_t st) {
  return dispatch_mode<EPI_F32, true>(mode, fa, fb, A, B, sa, sb, ep, M, N, K, st, "fp8_gemm_fused");
}
}  // namespace sfp8
