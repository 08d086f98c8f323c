// fp8_gemm_fused: the FP8 x FP8 GEMM with the fused epilogue of gemm_epilogue.h (bias,
// pre-activation copy, GELU or SwiGLU, fp32 / bf16 / FP8 output with amax).
#include "gemm_kernels.h"

namespace sfp8 {
// one per (output type, mode pair), each in its own translation unit (gemm_fused_<type>_<pair>.hip):
// tm = per-tensor and MX, bt = the two blockwise modes
#define SFP8_FUSED_DECL(name)                                                                                   \
  int name(int mode, int fa, int fb, const uint8_t* A, const uint8_t* B, const void* sa, const void* sb,        \
           const EpiParams& ep, int M, int N, int K, hipStream_t st);
SFP8_FUSED_DECL(gemm_fused_f32_tm)
SFP8_FUSED_DECL(gemm_fused_f32_bt)
SFP8_FUSED_DECL(gemm_fused_bf16_tm)
SFP8_FUSED_DECL(gemm_fused_bf16_bt)
SFP8_FUSED_DECL(gemm_fused_e4m3_tm)
SFP8_FUSED_DECL(gemm_fused_e4m3_bt)
SFP8_FUSED_DECL(gemm_fused_e5m2_tm)
SFP8_FUSED_DECL(gemm_fused_e5m2_bt)
#undef SFP8_FUSED_DECL
}  // namespace sfp8

using namespace sfp8;

extern "C" int fp8_gemm_fused(const uint8_t* A, int fmt_a, const void* a_scale_inv, int gran_a, const uint8_t* B,
                              int fmt_b, const void* b_scale_inv, int gran_b, const void* bias, int bias_dtype, int act,
                              void* aux, void* C, int c_dtype, const float* c_scale, float* c_amax, int64_t M,
                              int64_t N, int64_t K, void* stream) {
  const char* what = "fp8_gemm_fused";
  int mode = -1;
  const int rc = gemm_check(what, A, fmt_a, a_scale_inv, gran_a, B, fmt_b, b_scale_inv, gran_b, M, N, K, mode);
  if (rc != FP8_OK) return rc;
  SFP8_REQUIRE(fmt_b == FP8_E4M3, FP8_ERR_ARG, "%s: B must be E4M3 (weights and activations are E4M3 in every recipe)",
               what);
  SFP8_REQUIRE(c_dtype == OUT_F32 || c_dtype == OUT_BF16 || c_dtype == OUT_E4M3 || c_dtype == OUT_E5M2,
               FP8_ERR_DTYPE, "%s: c_dtype %d", what, c_dtype);
  SFP8_REQUIRE(act == FP8_ACT_NONE || act == FP8_ACT_GELU || act == FP8_ACT_SWIGLU, FP8_ERR_ARG, "%s: act %d", what,
               act);
  SFP8_REQUIRE(bias == nullptr || bias_dtype == HP_F32 || bias_dtype == HP_BF16, FP8_ERR_DTYPE, "%s: bias_dtype %d",
               what, bias_dtype);
  SFP8_REQUIRE(act != FP8_ACT_SWIGLU || N % 2 == 0, FP8_ERR_SHAPE,
               "%s: SwiGLU needs an even N (interleaved gate/up rows), N=%lld", what, (long long)N);
  const bool fp8_out = c_dtype == OUT_E4M3 || c_dtype == OUT_E5M2;
  if (M == 0 || N == 0) return FP8_OK;
  SFP8_REQUIRE(C != nullptr && aligned16(C), FP8_ERR_ARG, "%s: C must be non-null and 16-byte aligned", what);
  SFP8_REQUIRE(aux == nullptr || aligned16(aux), FP8_ERR_ARG, "%s: aux must be 16-byte aligned", what);
  SFP8_REQUIRE(bias == nullptr || (bias_dtype == HP_F32 ? aligned4(bias) : (reinterpret_cast<uintptr_t>(bias) & 1) == 0),
               FP8_ERR_ARG, "%s: misaligned bias", what);
  SFP8_REQUIRE(!fp8_out || (c_scale != nullptr && c_amax != nullptr && aligned4(c_scale) && aligned4(c_amax)),
               FP8_ERR_ARG, "%s: FP8 output needs 4-byte aligned c_scale and c_amax", what);
  EpiParams ep{};
  ep.C = C;
  ep.bias = bias;
  ep.aux = aux;
  ep.c_scale = c_scale;
  ep.c_amax = c_amax;
  ep.bias_bf16 = bias_dtype == HP_BF16;
  ep.act = act;
  hipStream_t st = (hipStream_t)stream;
  const int m = (int)M, n = (int)N, k = (int)K;
  const bool tm = mode == MODE_TENSOR || mode == MODE_MX;
  switch (c_dtype) {
    case OUT_F32:
      return (tm ? gemm_fused_f32_tm : gemm_fused_f32_bt)(mode, fmt_a, fmt_b, A, B, a_scale_inv, b_scale_inv, ep, m,
                                                        n, k, st);
    case OUT_BF16:
      return (tm ? gemm_fused_bf16_tm : gemm_fused_bf16_bt)(mode, fmt_a, fmt_b, A, B, a_scale_inv, b_scale_inv, ep, m,
                                                          n, k, st);
    case OUT_E4M3:
      return (tm ? gemm_fused_e4m3_tm : gemm_fused_e4m3_bt)(mode, fmt_a, fmt_b, A, B, a_scale_inv, b_scale_inv, ep, m,
                                                          n, k, st);
    default:
      return (tm ? gemm_fused_e5m2_tm : gemm_fused_e5m2_bt)(mode, fmt_a, fmt_b, A, B, a_scale_inv, b_scale_inv, ep, m,
                                                          n, k, st);
  }
}
