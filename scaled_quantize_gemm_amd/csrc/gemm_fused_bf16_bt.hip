// Instantiations of the fused-epilogue GEMM kernels for one output type (EPI_BF16) and the
// blockwise modes; one file per (output type, mode pair) so that they compile in parallel.
#include "gemm_kernels.h"

namespace sfp8 {
int gemm_fused_bf16_bt(int mode, int fa, int fb, const uint8_t* A, const uint8_t* B, const void* sa,
                      const void* sb, const EpiParams& ep, int M, int N, int K, hipStream_t st) {
  if (mode == MODE_BLOCK) return dispatch_fmt<MODE_BLOCK, EPI_BF16, true>(fa, fb, A, B, sa, sb, ep, M, N, K, st, "fp8_gemm_fused");
  return dispatch_fmt<MODE_TILE2, EPI_BF16, true>(fa, fb, A, B, sa, sb, ep, M, N, K, st, "fp8_gemm_fused");
}
}  // namespace sfp8
