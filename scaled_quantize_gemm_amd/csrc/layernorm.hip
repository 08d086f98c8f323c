// LayerNorm fused with the FP8 cast of its output: the step before the GEMM.
//
// Transformer Engine tutorial, module tour cell (te.LayerNorm, te.LayerNormLinear and
// te.LayerNormMLP: the norm feeds the FP8 linear directly) and plain-PyTorch block cell
// (nn.LayerNorm before attention and before the MLP).  Per row of x [rows][cols]:
//   mean = sum(x) / cols,  var = sum((x - mean)^2) / cols  (biased),  rs = 1 / sqrt(var + eps)
//   y = (x - mean) * rs * gamma + beta
// and y goes straight to FP8 under the cast rules of quantize.hip at one of three
// granularities: per tensor (delayed scale, amax of y max-reduced into a slot), 1x128 runs
// or MX 1x32 runs (current scales from the run's amax).  y never exists in HBM: the kernel
// reads x once and writes the codes (and scales) once, instead of a bf16 round trip.
//
// One wave per row, the row held in registers: lane l takes the 8-element chunks l, l+64,
// l+128, ... (NCH of them, cols <= 512 NCH), so every load and code store of the wave is a
// contiguous 512-element segment of the row, a 1x32 run is 4 adjacent lanes and a 1x128 run
// 16 adjacent lanes (shuffle reductions within the group).  Mean and variance are two
// passes over the registers (no cancellation from a one-pass sum of squares).  8 rows per
// block; row groups are dealt to the XCDs in contiguous ranges (block b runs on XCD b % 8),
// so the narrow [cols/32][rows] e8m0 and [cols/128][rows] scale columns of neighbouring row
// groups fill their cache lines in one L2.
#include "quant_rules.h"

namespace sfp8 {

constexpr int kLnRows = 8;  // rows (waves) per block

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// 8 consecutive gamma / beta values (ordinary loads: every row reads them, they stay cached)
__device__ __forceinline__ void load8_param(const void* __restrict__ p, bool bf16, int e0, float (&v)[8]) {
  if (bf16) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p) + e0);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + e0);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + e0 + 4);
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  }
}

template <int FMT, bool BF16, int GRAN, int NCH>
__global__ void __launch_bounds__(64 * kLnRows) ln_quant_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma, const void* __restrict__ beta, int w_bf16, float eps,
    int64_t rows, int cols, int row_blocks, const float* __restrict__ scale_p, uint32_t* __restrict__ amax_slot,
    uint8_t* __restrict__ q, void* __restrict__ sinv, float* __restrict__ mu_out, float* __restrict__ rs_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x, xcd = b & 7, idx = b >> 3, per = row_blocks >> 3, rem = row_blocks & 7;
  const int rb = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int64_t row = (int64_t)rb * kLnRows + wave;
  const bool live = row < rows;   // waves past the last row idle until the block's amax reduction
  const int nch = live ? cols >> 3 : 0;
  const int64_t base = row * cols;

  float v[NCH][8];
  float sum = 0.0f;
#pragma unroll
  for (int p = 0; p < NCH; ++p) {
    const int c = lane + 64 * p;
    if (c < nch) {
      load8<BF16>(x, base + 8 * c, v[p]);
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += v[p][i];
    }
  }
  const float mean = wave_sum(sum) / (float)cols;
  float ssq = 0.0f;
#pragma unroll
  for (int p = 0; p < NCH; ++p)
    if (lane + 64 * p < nch) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[p][i] -= mean;
        ssq += v[p][i] * v[p][i];
      }
    }
  const float rs = 1.0f / sqrtf(wave_sum(ssq) / (float)cols + eps);
  if (lane == 0 && live) {
    if (mu_out != nullptr) mu_out[row] = mean;
    if (rs_out != nullptr) rs_out[row] = rs;
  }

  float s = 1.0f;
  if constexpr (GRAN == FP8_SCALE_TENSOR) s = *scale_p;
  uint32_t lane_amax = 0u;
#pragma unroll
  for (int p = 0; p < NCH; ++p) {
    const int c = lane + 64 * p;
    // whole 4- and 16-lane groups share the branch: nch is a multiple of 4 (MX) / 16 (1x128)
    if (c >= nch) continue;
    float g[8];
    load8_param(gamma, w_bf16, 8 * c, g);
    if (beta != nullptr) {
      float bb[8];
      load8_param(beta, w_bf16, 8 * c, bb);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[p][i] = fmaf(v[p][i] * rs, g[i], bb[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[p][i] = v[p][i] * rs * g[i];
    }
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = m > abs_bits(v[p][i]) ? m : abs_bits(v[p][i]);
    u32x2 codes;
    if constexpr (GRAN == FP8_SCALE_TENSOR) {
      codes = cast8<FMT>(v[p], s, m);
      lane_amax = lane_amax > m ? lane_amax : m;
    } else if constexpr (GRAN == FP8_SCALE_TILE_1x128) {
      const bool nan_here = m > 0x7F800000u;
      m = group_max_u32<16>(m);
      float sc, sc_inv;
      current_scale<FMT>(m, sc, sc_inv);
      codes = cast8<FMT>(v[p], sc, nan_here ? m : 0u);
      if ((lane & 15) == 0) static_cast<float*>(sinv)[(int64_t)(c >> 4) * rows + row] = sc_inv;
    } else {
      const bool nan_here = m > 0x7F800000u;
      m = group_max_u32<4>(m);
      uint32_t code;
      float mult;
      mx_rule<FMT>(m, code, mult);
      codes = cast8<FMT>(v[p], mult, nan_here ? m : 0u);
      if ((lane & 3) == 0) static_cast<uint8_t*>(sinv)[(int64_t)(c >> 2) * rows + row] = (uint8_t)code;
    }
    __builtin_nontemporal_store(codes, reinterpret_cast<u32x2*>(q + base + 8 * c));
  }
  // per tensor: the block's amax goes to the slot with one atomic (one per wave measured 3.7x
  // slower over the whole kernel on 8192 x 4096)
  if constexpr (GRAN == FP8_SCALE_TENSOR) {
    if (amax_slot != nullptr) {
      __shared__ uint32_t red[kLnRows];
      const uint32_t m = wave_max_u32(lane_amax);
      if (lane == 0) red[wave] = m;
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t r = red[0];
#pragma unroll
        for (int i = 1; i < kLnRows; ++i) r = r > red[i] ? r : red[i];
        if (r != 0u) atomicMax(amax_slot, r);
      }
    }
  }
}

template <int FMT, bool BF16, int GRAN>
static void launch_ln(int nch_blocks, const void* x, const void* gamma, const void* beta, int w_bf16, float eps,
                      int64_t rows, int cols, const float* scale, float* amax_slot, uint8_t* q, void* sinv, float* mu,
                      float* rs, hipStream_t st) {
  const int row_blocks = (int)((rows + kLnRows - 1) / kLnRows);
  const dim3 grid(row_blocks), block(64 * kLnRows);
  uint32_t* slot = reinterpret_cast<uint32_t*>(amax_slot);
#define SFP8_LN(N)                                                                                              \
  hipLaunchKernelGGL((ln_quant_kernel<FMT, BF16, GRAN, N>), grid, block, 0, st, x, gamma, beta, w_bf16, eps, rows, \
                     cols, row_blocks, scale, slot, q, sinv, mu, rs)
  switch (nch_blocks) {
    case 1: SFP8_LN(1); break;
    case 2: SFP8_LN(2); break;
    case 4: SFP8_LN(4); break;
    case 8: SFP8_LN(8); break;
    default: SFP8_LN(16); break;
  }
#undef SFP8_LN
}

template <int FMT, bool BF16>
static void launch_ln_gran(int gran, int nchb, const void* x, const void* gamma, const void* beta, int w_bf16, float eps,
                           int64_t rows, int cols, const float* scale, float* amax_slot, uint8_t* q, void* sinv,
                           float* mu, float* rs, hipStream_t st) {
  if (gran == FP8_SCALE_TENSOR)
    launch_ln<FMT, BF16, FP8_SCALE_TENSOR>(nchb, x, gamma, beta, w_bf16, eps, rows, cols, scale, amax_slot, q, sinv, mu,
                                           rs, st);
  else if (gran == FP8_SCALE_TILE_1x128)
    launch_ln<FMT, BF16, FP8_SCALE_TILE_1x128>(nchb, x, gamma, beta, w_bf16, eps, rows, cols, scale, amax_slot, q, sinv,
                                               mu, rs, st);
  else
    launch_ln<FMT, BF16, FP8_SCALE_MX_1x32>(nchb, x, gamma, beta, w_bf16, eps, rows, cols, scale, amax_slot, q, sinv, mu,
                                            rs, st);
}

}  // namespace sfp8

using namespace sfp8;

extern "C" int fp8_layernorm_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, const void* gamma,
                                      const void* beta, int w_dtype, float eps, int fmt, int granularity,
                                      const float* scale, float* amax_slot, uint8_t* q, void* scale_inv_out,
                                      float* mu, float* rsigma, void* stream) {
  const char* what = "fp8_layernorm_quantize";
  SFP8_REQUIRE(x_dtype == HP_F32 || x_dtype == HP_BF16, FP8_ERR_DTYPE, "%s: x_dtype %d", what, x_dtype);
  SFP8_REQUIRE(w_dtype == HP_F32 || w_dtype == HP_BF16, FP8_ERR_DTYPE, "%s: w_dtype %d", what, w_dtype);
  SFP8_REQUIRE(fmt == FP8_E4M3 || fmt == FP8_E5M2, FP8_ERR_ARG, "%s: fmt %d", what, fmt);
  SFP8_REQUIRE(granularity == FP8_SCALE_TENSOR || granularity == FP8_SCALE_TILE_1x128 ||
                   granularity == FP8_SCALE_MX_1x32,
               FP8_ERR_ARG, "%s: granularity %d (TENSOR, TILE_1x128 or MX_1x32)", what, granularity);
  SFP8_REQUIRE(rows >= 0 && cols >= 0, FP8_ERR_SHAPE, "%s: negative shape", what);
  SFP8_REQUIRE(rows < (1ll << 31) / kLnRows, FP8_ERR_SHAPE, "%s: rows >= 2^28", what);
  const int64_t need = granularity == FP8_SCALE_TILE_1x128 ? 128 : (granularity == FP8_SCALE_MX_1x32 ? 32 : 8);
  SFP8_REQUIRE(cols % need == 0 && cols <= 8192, FP8_ERR_SHAPE,
               "%s: cols=%lld must be a multiple of %lld and at most 8192", what, (long long)cols, (long long)need);
  SFP8_REQUIRE(eps >= 0.0f, FP8_ERR_ARG, "%s: eps must be >= 0", what);
  if (rows == 0 || cols == 0) return FP8_OK;
  SFP8_REQUIRE(x != nullptr && q != nullptr && gamma != nullptr, FP8_ERR_ARG, "%s: null x, q or gamma", what);
  SFP8_REQUIRE(aligned16(x) && aligned16(q) && aligned16(gamma) && (beta == nullptr || aligned16(beta)), FP8_ERR_ARG,
               "%s: x, q, gamma, beta must be 16-byte aligned", what);
  if (granularity == FP8_SCALE_TENSOR) {
    SFP8_REQUIRE(scale != nullptr && aligned4(scale), FP8_ERR_ARG, "%s: TENSOR needs a 4-byte aligned scale", what);
    SFP8_REQUIRE(amax_slot == nullptr || aligned4(amax_slot), FP8_ERR_ARG, "%s: misaligned amax_slot", what);
  } else {
    SFP8_REQUIRE(scale_inv_out != nullptr, FP8_ERR_ARG, "%s: null scale_inv_out", what);
    SFP8_REQUIRE(granularity == FP8_SCALE_MX_1x32 || aligned4(scale_inv_out), FP8_ERR_ARG,
                 "%s: misaligned scale_inv_out", what);
  }
  SFP8_REQUIRE((mu == nullptr || aligned4(mu)) && (rsigma == nullptr || aligned4(rsigma)), FP8_ERR_ARG,
               "%s: misaligned mu / rsigma", what);
  const int nch = (int)(cols >> 3);
  const int nchb = nch <= 64 ? 1 : nch <= 128 ? 2 : nch <= 256 ? 4 : nch <= 512 ? 8 : 16;
  const int wb = w_dtype == HP_BF16;
  const int c = (int)cols;
  hipStream_t st = (hipStream_t)stream;
  if (fmt == FP8_E4M3) {
    if (x_dtype == HP_BF16)
      launch_ln_gran<FP8_E4M3, true>(granularity, nchb, x, gamma, beta, wb, eps, rows, c, scale, amax_slot, q,
                                     scale_inv_out, mu, rsigma, st);
    else
      launch_ln_gran<FP8_E4M3, false>(granularity, nchb, x, gamma, beta, wb, eps, rows, c, scale, amax_slot, q,
                                      scale_inv_out, mu, rsigma, st);
  } else {
    if (x_dtype == HP_BF16)
      launch_ln_gran<FP8_E5M2, true>(granularity, nchb, x, gamma, beta, wb, eps, rows, c, scale, amax_slot, q,
                                     scale_inv_out, mu, rsigma, st);
    else
      launch_ln_gran<FP8_E5M2, false>(granularity, nchb, x, gamma, beta, wb, eps, rows, c, scale, amax_slot, q,
                                      scale_inv_out, mu, rsigma, st);
  }
  return check_launch(what);
}
