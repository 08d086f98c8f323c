// fp8_gemm: the FP8 x FP8 GEMM with the plain dequantising epilogue (C = the fp32 result,
// stored as fp32 or bf16).  The kernels are in gemm_kernels.h.
#include "gemm_kernels.h"

using namespace sfp8;

extern "C" int fp8_gemm(const uint8_t* A, int fmt_a, const void* a_scale_inv, int gran_a, const uint8_t* B, int fmt_b,
                        const void* b_scale_inv, int gran_b, void* C, int c_dtype, int64_t M, int64_t N, int64_t K,
                        void* stream) {
  int mode = -1;
  const int rc = gemm_check("fp8_gemm", A, fmt_a, a_scale_inv, gran_a, B, fmt_b, b_scale_inv, gran_b, M, N, K, mode);
  if (rc != FP8_OK) return rc;
  SFP8_REQUIRE(c_dtype == OUT_F32 || c_dtype == OUT_BF16, FP8_ERR_DTYPE, "fp8_gemm: c_dtype %d", c_dtype);
  if (M == 0 || N == 0) return FP8_OK;
  SFP8_REQUIRE(C != nullptr, FP8_ERR_ARG, "fp8_gemm: null C");
  SFP8_REQUIRE(aligned4(C), FP8_ERR_ARG, "fp8_gemm: C must be 4-byte aligned");
  EpiParams ep{};
  ep.C = C;
  ep.act = FP8_ACT_NONE;
  hipStream_t st = (hipStream_t)stream;
  const int m = (int)M, n = (int)N, k = (int)K;
  if (c_dtype == OUT_F32)
    return dispatch_mode<EPI_F32, false>(mode, fmt_a, fmt_b, A, B, a_scale_inv, b_scale_inv, ep, m, n, k, st, "fp8_gemm");
  return dispatch_mode<EPI_BF16, false>(mode, fmt_a, fmt_b, A, B, a_scale_inv, b_scale_inv, ep, m, n, k, st, "fp8_gemm");
}
