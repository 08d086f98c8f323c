// Instantiations of the fused-epilogue GEMM kernels for one output type (EPI_E4M3) and the
// per-tensor and MX modes; one file per (output type, mode pair) so that they compile in parallel.
#include "gemm_kernels.h"

namespace sfp8 {
int gemm_fused_e4m3_tm(int mode, int fa, int fb, const uint8_t* A, const uint8_t* B, const void* sa,
                      const void* sb, const EpiParams& ep, int M, int N, int K, hipStream_t st) {
  if (mode == MODE_TENSOR) return dispatch_fmt<MODE_TENSOR, EPI_E4M3, true>(fa, fb, A, B, sa, sb, ep, M, N, K, st, "fp8_gemm_fused");
  return dispatch_fmt<MODE_MX, EPI_E4M3, true>(fa, fb, A, B, sa, sb, ep, M, N, K, st, "fp8_gemm_fused");
}
}  // namespace sfp8
