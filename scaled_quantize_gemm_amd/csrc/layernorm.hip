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
// passes over the registers (no cancellation from a one-pass sum of squares).
#include <algorithm>

#include "quant_rules.h"

namespace sfp8 {

constexpr int kLnRows = 4;  // waves per block, one row each per step (small blocks pack the CU)

// sum over the 64 lanes, the same in every lane (each step adds a lane and its partner, which
// adds them in the other order: fp32 addition commutes); 6 levels, as the error bound assumes
__device__ __forceinline__ float wave_sum(float v) {
  auto partner = [](float x, auto ctrl) {
    return __uint_as_float(dpp_partner<decltype(ctrl)::value>(__float_as_uint(x)));
  };
  v += partner(v, std::integral_constant<int, kDppQuadXor1>{});
  v += partner(v, std::integral_constant<int, kDppQuadXor2>{});
  v += partner(v, std::integral_constant<int, kDppHalfMirror>{});
  v += partner(v, std::integral_constant<int, kDppMirror>{});
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// raw 16-byte pieces of one 8-element chunk: 1 for bf16, 2 for fp32
template <bool BF16>
struct Chunk {
  u32x4 w[BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ void load_chunk(const void* __restrict__ x, int64_t e0, Chunk<BF16>& c) {
  if constexpr (BF16) {
    c.w[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + e0));
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + e0);
    c.w[0] = __builtin_nontemporal_load(p);
    c.w[1] = __builtin_nontemporal_load(p + 1);
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack_chunk(const Chunk<BF16>& c, float (&v)[8]) {
  if constexpr (BF16) {
    const uint32_t w[4] = {c.w[0].x, c.w[0].y, c.w[0].z, c.w[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const uint32_t w[8] = {c.w[0].x, c.w[0].y, c.w[0].z, c.w[0].w, c.w[1].x, c.w[1].y, c.w[1].z, c.w[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
  }
}

// Persistent blocks: the grid is 8 x (blocks per XCD); XCD x (block b runs on XCD b % 8) owns
// the contiguous range of 8-row groups [G x / 8, G (x + 1) / 8), which its blocks walk with a
// stride of their count, so the narrow scale columns ([cols/32][rows] e8m0, [cols/128][rows]
// fp32) of neighbouring groups fill their cache lines in one L2.  gamma and beta sit in LDS as
// fp32 for the block's lifetime; each wave loads its next row while it normalises the current
// one, so the row's HBM latency overlaps the reductions and the cast.
template <int FMT, bool BF16, int GRAN, int NCH, bool FULL>
__global__ void __launch_bounds__(64 * kLnRows) ln_quant_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma, const void* __restrict__ beta, int w_bf16, float eps,
    int64_t rows, int cols, int64_t groups, const float* __restrict__ scale_p, uint32_t* __restrict__ amax_slot,
    uint8_t* __restrict__ q, void* __restrict__ sinv, float* __restrict__ mu_out, float* __restrict__ rs_out) {
  extern __shared__ __attribute__((aligned(16))) float ln_smem[];
  float* g_s = ln_smem;         // [cols]
  float* b_s = ln_smem + cols;  // [cols] (zeros without beta)
  // gamma and beta to LDS as fp32, 8 columns per thread and pass (cols is a multiple of 8;
  // both are 16-byte aligned); each wave issues its first row's loads before the fill, so
  // that their latency overlaps it
  auto fill = [&](const void* src, float* dst) {
    for (int i = 8 * threadIdx.x; i < cols; i += 8 * 64 * kLnRows) {
      float w[8];
      if (src == nullptr) {
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = 0.0f;
      } else if (w_bf16) {
        const u32x4 h = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + i);
        const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          w[2 * k] = bf16_lo(hw[k]);
          w[2 * k + 1] = bf16_hi(hw[k]);
        }
      } else {
        const float4 f0 = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + i);
        const float4 f1 = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + i + 4);
        w[0] = f0.x; w[1] = f0.y; w[2] = f0.z; w[3] = f0.w;
        w[4] = f1.x; w[5] = f1.y; w[6] = f1.z; w[7] = f1.w;
      }
      *reinterpret_cast<float4*>(dst + i) = make_float4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<float4*>(dst + i + 4) = make_float4(w[4], w[5], w[6], w[7]);
    }
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: row addresses in SGPRs
  const int nbx = gridDim.x >> 3, xcd = blockIdx.x & 7;
  const int64_t g_end = groups * (xcd + 1) / 8;
  // FULL: cols == 512 NCH, every lane holds NCH whole chunks (no per-chunk tests)
  const int nch = FULL ? 64 * NCH : cols >> 3;
  float s = 1.0f;
  if constexpr (GRAN == FP8_SCALE_TENSOR) s = *scale_p;
  // this lane's scale column: run (lane + 64p) / 4 of MX
  uint8_t* const sinv_mx = static_cast<uint8_t*>(sinv) + (int64_t)(lane >> 2) * rows;
  uint32_t lane_amax = 0u;

  // the next row is prefetched when its raw chunks fit beside the current row's values (rows
  // of at most 4096 columns)
  constexpr bool PF = NCH <= 8;
  int64_t grp = groups * xcd / 8 + (blockIdx.x >> 3);
  int64_t row = grp * kLnRows + wave;
  Chunk<BF16> raw[PF ? NCH : 1];
  if constexpr (PF) {
    if (grp < g_end && row < rows) {
#pragma unroll
      for (int p = 0; p < NCH; ++p)
        if (lane + 64 * p < nch) load_chunk<BF16>(x, row * cols + 8 * (lane + 64 * p), raw[p]);
    }
  }
  fill(gamma, g_s);
  fill(beta, b_s);
  __syncthreads();
  for (; grp < g_end; grp += nbx) {
    const bool live = row < rows;
    float v[NCH][8];
    if constexpr (PF) {
#pragma unroll
      for (int p = 0; p < NCH; ++p) unpack_chunk<BF16>(raw[p], v[p]);
    } else if (live) {
#pragma unroll
      for (int p = 0; p < NCH; ++p)
        if (lane + 64 * p < nch) {
          Chunk<BF16> c1;
          load_chunk<BF16>(x, row * cols + 8 * (lane + 64 * p), c1);
          unpack_chunk<BF16>(c1, v[p]);
        }
    }
    // the next row of this wave, in flight while this one is processed
    const int64_t row_n = (grp + nbx) * kLnRows + wave;
    if constexpr (PF) {
      if (grp + nbx < g_end && row_n < rows) {
#pragma unroll
        for (int p = 0; p < NCH; ++p)
          if (lane + 64 * p < nch) load_chunk<BF16>(x, row_n * cols + 8 * (lane + 64 * p), raw[p]);
      }
    }
    if (live) {
      const int64_t base = row * cols;
      float sum = 0.0f;
#pragma unroll
      for (int p = 0; p < NCH; ++p)
        if (lane + 64 * p < nch) {
#pragma unroll
          for (int i = 0; i < 8; ++i) sum += v[p][i];
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
      if (lane == 0) {
        if (mu_out != nullptr) mu_out[row] = mean;
        if (rs_out != nullptr) rs_out[row] = rs;
      }
      // A NaN or inf anywhere in the row makes mean or rs non-finite, and then every y of the
      // row is NaN; otherwise no y is NaN.  So NaN handling (unsigned amax over |y| bits, code
      // rewrite) is a per-row, wave-uniform branch, and finite rows take the float max with an
      // abs modifier and no rewrite.
      const bool nan_row = __builtin_amdgcn_readfirstlane(__builtin_isfinite(mean) && __builtin_isfinite(rs) ? 0 : 1);
      // y = fma((x - mean) rs, gamma, beta) of chunk c from the centred values xc, rs given
      auto normalise = [&](const float (&xc)[8], int c, float rs, float (&y)[8]) {
        const float4 g0 = *reinterpret_cast<const float4*>(g_s + 8 * c);
        const float4 g1 = *reinterpret_cast<const float4*>(g_s + 8 * c + 4);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        if (beta != nullptr) {
          const float4 b0 = *reinterpret_cast<const float4*>(b_s + 8 * c);
          const float4 b1 = *reinterpret_cast<const float4*>(b_s + 8 * c + 4);
          const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) y[i] = fmaf(xc[i] * rs, g[i], bb[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) y[i] = xc[i] * rs * g[i];
        }
      };
      // 1x128: each chunk's group max and this lane's own max, kept for the cast after the scales
      uint32_t run_max[GRAN == FP8_SCALE_TILE_1x128 ? NCH : 1], own_max[GRAN == FP8_SCALE_TILE_1x128 ? NCH : 1];
#pragma unroll
      for (int p = 0; p < NCH; ++p) {
        const int c = lane + 64 * p;
        // whole 4- and 16-lane groups share the branch: nch is a multiple of 4 (MX) / 16 (1x128)
        if (c >= nch) {
          if constexpr (GRAN == FP8_SCALE_TILE_1x128) run_max[p] = own_max[p] = 0u;
          continue;
        }
        // 1x128 keeps the centred values for a second normalisation after the row's scales
        // (holding all of y instead took 216 VGPRs, 2 waves per SIMD)
        float y[8];
        normalise(v[p], c, rs, y);
        if constexpr (GRAN != FP8_SCALE_TILE_1x128) {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[p][i] = y[i];
        }
        uint32_t m;
        if (nan_row) {
          m = 0u;
#pragma unroll
          for (int i = 0; i < 8; ++i) m = m > abs_bits(y[i]) ? m : abs_bits(y[i]);
        } else {
          float mf = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) mf = fmaxf(mf, fabsf(y[i]));
          m = __float_as_uint(mf);
        }
        const uint32_t own = m;  // this lane's |y| bits max (NaN bits only on NaN rows)
        float sc = s;
        if constexpr (GRAN == FP8_SCALE_TENSOR) {
          lane_amax = lane_amax > m ? lane_amax : m;
        } else if constexpr (GRAN == FP8_SCALE_TILE_1x128) {
          run_max[p] = group_max_u32<16>(m);
          own_max[p] = own;
          continue;  // cast below, once the row's scales are known
        } else {
          m = group_max_u32<4>(m);
          uint32_t code;
          mx_rule<FMT>(m, code, sc);
          if ((lane & 3) == 0) sinv_mx[(int64_t)(16 * p) * rows + row] = (uint8_t)code;
        }
        u32x2 codes = cast8<FMT>(v[p], sc, 0u);
        if (nan_row) codes = cast8<FMT>(v[p], sc, own);
        __builtin_nontemporal_store(codes, reinterpret_cast<u32x2*>(q + base + 8 * c));
      }
      if constexpr (GRAN == FP8_SCALE_TILE_1x128) {
        // the row's cols/128 (<= 64) run scales at once, lane L taking run L, instead of every
        // 16-lane group dividing for its own run in each chunk (two correctly rounded divisions
        // per 4 runs: 4.5 us of 28 on 8192 x 4096).  Run L's max is chunk L/4's in group L%4;
        // its scale goes back to the 16 lanes of that group.
        uint32_t a = 0u;
#pragma unroll
        for (int p = 0; p < NCH; ++p) {
          const uint32_t t = (uint32_t)__shfl((int)run_max[p], 16 * (lane & 3), 64);
          a = (lane >> 2) == p ? t : a;
        }
        float run_sc, run_sinv;
        current_scale<FMT>(a, run_sc, run_sinv);
        // the second normalisation must not be merged with the first (that would keep every y
        // live across the scale step): rs and the chunk index pass through empty asm
        float rs2 = rs;
        int lane2 = lane;
        asm volatile("" : "+v"(rs2), "+v"(lane2));
        if (lane < (nch >> 4)) static_cast<float*>(sinv)[(int64_t)lane * rows + row] = run_sinv;  // [cols/128][rows]
#pragma unroll
        for (int p = 0; p < NCH; ++p) {
          const int c = lane + 64 * p;
          const float sc = __shfl(run_sc, (lane >> 4) + 4 * p, 64);
          if (c >= nch) continue;
          float y[8];
          normalise(v[p], lane2 + 64 * p, rs2, y);
          u32x2 codes = cast8<FMT>(y, sc, 0u);
          if (nan_row) codes = cast8<FMT>(y, sc, own_max[p]);
          __builtin_nontemporal_store(codes, reinterpret_cast<u32x2*>(q + base + 8 * c));
        }
      }
    }
    row = row_n;
  }
  // per tensor: the block's amax goes to the slot with one atomic (one per wave and row
  // measured 3.7x slower over the whole kernel on 8192 x 4096)
  if constexpr (GRAN == FP8_SCALE_TENSOR) {
    if (amax_slot != nullptr) {
      // the gamma / beta area is free once every wave is past the loop (keeps the block
      // within 64 KB of LDS at 8192 columns)
      uint32_t* red = reinterpret_cast<uint32_t*>(ln_smem);
      const uint32_t m = wave_max_u32(lane_amax);
      __syncthreads();
      if (lane == 0) red[wave] = m;
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t r = red[0];
#pragma unroll
        for (int i = 1; i < kLnRows; ++i) r = r > red[i] ? r : red[i];
        // a plain read first: the blocks end together, and most do not raise the maximum
        if (r > __hip_atomic_load(amax_slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(amax_slot, r);
      }
    }
  }
}

template <int FMT, bool BF16, int GRAN>
static void launch_ln(int nch_blocks, const void* x, const void* gamma, const void* beta, int w_bf16, float eps,
                      int64_t rows, int cols, const float* scale, float* amax_slot, uint8_t* q, void* sinv, float* mu,
                      float* rs, hipStream_t st) {
  const int64_t groups = (rows + kLnRows - 1) / kLnRows;
  const size_t lds = 2 * (size_t)cols * sizeof(float);
  uint32_t* slot = reinterpret_cast<uint32_t*>(amax_slot);
  // as many blocks as are resident at once (registers and LDS decide: 2-5 waves per SIMD),
  // the same number on each of the 8 XCDs
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess || n < 8)
      n = 256;
    return n;
  }();
#define SFP8_LN_F(N, F)                                                                                              \
  do {                                                                                                               \
    int per_cu = 0;                                                                                                  \
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ln_quant_kernel<FMT, BF16, GRAN, N, F>, 64 * kLnRows,  \
                                                     lds) != hipSuccess || per_cu < 1)                              \
      per_cu = 1;                                                                                                    \
    const int64_t per_xcd = std::min<int64_t>((int64_t)per_cu * (cus / 8), (groups + 7) / 8);                        \
    hipLaunchKernelGGL((ln_quant_kernel<FMT, BF16, GRAN, N, F>), dim3((unsigned)(8 * per_xcd)), dim3(64 * kLnRows),  \
                       lds, st, x, gamma, beta, w_bf16, eps, rows, cols, groups, scale, slot, q, sinv, mu, rs);      \
  } while (0)
#define SFP8_LN(N)                          \
  do {                                      \
    if (cols == 512 * (N)) SFP8_LN_F(N, true); \
    else SFP8_LN_F(N, false);               \
  } while (0)
  switch (nch_blocks) {
    case 1: SFP8_LN(1); break;
    case 2: SFP8_LN(2); break;
    case 4: SFP8_LN(4); break;
    case 8: SFP8_LN(8); break;
    default: SFP8_LN(16); break;
  }
#undef SFP8_LN
#undef SFP8_LN_F
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
