// FP8 x FP8 GEMM on gfx950 matrix cores: C[M][N] = sum_k deq(A[m][k]) deq(B[n][k]).
//
// "Week 14" course page: matmuls run in FP8 (FP8 bullet); FP8 products are summed in a
// wider accumulator and partial sums promoted to fp32 at fixed intervals
// (accumulation-precision bullet); MX gives every 32 numbers a shared scale and DeepSeek-V3
// scales 1x128 activation runs and 128x128 weight blocks (absmax bullet).
//
// Matrix-core facts this kernel is built on (gfx950, v_mfma_*_16x16x128_f8f6f4):
//  * operand layout: lane l = 16 g + r supplies row r of its 16-row operand; its 32 bytes are
//    K = 16g .. 16g+15 (bytes 0-15) and K = 64+16g .. 64+16g+15 (bytes 16-31);
//  * result layout: lane l holds C[4g + j][r], j = 0..3;
//  * scaled form: lane l's e8m0 byte scales row r over K = 32g .. 32g+31 by 2^(e - 127);
//  * the products are exact; runs of 8 consecutive K are summed in a fixed-point window
//    below the run's largest product, and each run is promoted into the fp32 accumulator.
//
// Block tile BM x BN x 128, 4 waves in a 2 x 2 grid, each wave (BM/2) x (BN/2) built from
// 16x16x128 MFMAs.  A and B tiles are staged through LDS (double-buffered, 16-byte chunks
// XOR-swizzled by row so the fragment reads of 16 consecutive rows hit distinct banks).
//
// Scaling modes:
//  * TENSOR:  acc over all K; C = acc * (sa * sb).
//  * BLOCK:   per 128-K block kb: p = MFMA from zero; acc += p * (sa[kb][m] * sb[n/128][kb]).
//  * MX:      scaled MFMA with the e8m0 codes of A[m][4kb+g] and B[n][4kb+g]; C = acc.
#include "common.h"

namespace sfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum { MODE_TENSOR = 0, MODE_BLOCK = 1, MODE_MX = 2 };

template <int BM, int BN>
struct GemmCfg {
  static constexpr int BK = 128;
  static constexpr int WM = BM / 2, WN = BN / 2;  // wave tile
  static constexpr int TM = WM / 16, TN = WN / 16;  // MFMA tiles per wave
  static constexpr int A_CHUNKS = BM * BK / 16, B_CHUNKS = BN * BK / 16;
  static constexpr int A_PER_T = A_CHUNKS / 256, B_PER_T = B_CHUNKS / 256;
  static constexpr int LDS_A = BM * BK, LDS_B = BN * BK;  // bytes per stage
};

// byte offset of 16-byte chunk c of tile row `row` in a 128-byte-row LDS tile
__device__ __forceinline__ int swz(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }

template <int BM, int BN, int MODE, int FA, int FB, int OUT>
__global__ void __launch_bounds__(256) gemm_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                   const void* __restrict__ sa_p, const void* __restrict__ sb_p,
                                                   void* __restrict__ C, int M, int N, int K) {
  using Cfg = GemmCfg<BM, BN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* lds_a = smem;                      // [2][BM][128]
  uint8_t* lds_b = smem + 2 * Cfg::LDS_A;     // [2][BN][128]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, r = lane & 15;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int nk = K / 128;

  // ---- global -> register staging of one K-step
  uint4 ra[Cfg::A_PER_T], rb[Cfg::B_PER_T];
  auto load_step = [&](int ks) {
#pragma unroll
    for (int i = 0; i < Cfg::A_PER_T; ++i) {
      const int id = tid + 256 * i, row = id >> 3, c = id & 7;
      int gm = m0 + row;
      gm = gm < M ? gm : M - 1;
      ra[i] = *reinterpret_cast<const uint4*>(A + (size_t)gm * K + (size_t)ks * 128 + c * 16);
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_PER_T; ++i) {
      const int id = tid + 256 * i, row = id >> 3, c = id & 7;
      int gn = n0 + row;
      gn = gn < N ? gn : N - 1;
      rb[i] = *reinterpret_cast<const uint4*>(B + (size_t)gn * K + (size_t)ks * 128 + c * 16);
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < Cfg::A_PER_T; ++i) {
      const int id = tid + 256 * i, row = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(lds_a + buf * Cfg::LDS_A + swz(row, c)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_PER_T; ++i) {
      const int id = tid + 256 * i, row = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(lds_b + buf * Cfg::LDS_B + swz(row, c)) = rb[i];
    }
  };

  v4f acc[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    load_step(0);
    store_step(0);
  }
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) load_step(ks + 1);

    // ---- per-step scale operands
    float sab[Cfg::TM][4];
    int scale_a[Cfg::TM], scale_b[Cfg::TN];
    if constexpr (MODE == MODE_BLOCK) {
      const float* sa = static_cast<const float*>(sa_p);
      const float* sb = static_cast<const float*>(sb_p);
      const float sbv = sb[(size_t)(n0 / 128) * nk + ks];
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int gm = m0 + wm * Cfg::WM + 16 * i + 4 * g + j;
          gm = gm < M ? gm : M - 1;
          sab[i][j] = sa[(size_t)ks * M + gm] * sbv;
        }
    }
    if constexpr (MODE == MODE_MX) {
      const uint8_t* ea = static_cast<const uint8_t*>(sa_p);
      const uint8_t* eb = static_cast<const uint8_t*>(sb_p);
      const int kq = K / 32;
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i) {
        int gm = m0 + wm * Cfg::WM + 16 * i + r;
        gm = gm < M ? gm : M - 1;
        scale_a[i] = ea[(size_t)gm * kq + 4 * ks + g];
      }
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j) {
        int gn = n0 + wn * Cfg::WN + 16 * j + r;
        gn = gn < N ? gn : N - 1;
        scale_b[j] = eb[(size_t)gn * kq + 4 * ks + g];
      }
    }

    // ---- fragments from LDS
    v8i fa[Cfg::TM], fb[Cfg::TN];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int row = wm * Cfg::WM + 16 * i + r;
      const uint8_t* base = lds_a + buf * Cfg::LDS_A;
      uint4 lo = *reinterpret_cast<const uint4*>(base + swz(row, g));
      uint4 hi = *reinterpret_cast<const uint4*>(base + swz(row, g + 4));
      fa[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int row = wn * Cfg::WN + 16 * j + r;
      const uint8_t* base = lds_b + buf * Cfg::LDS_B;
      uint4 lo = *reinterpret_cast<const uint4*>(base + swz(row, g));
      uint4 hi = *reinterpret_cast<const uint4*>(base + swz(row, g + 4));
      fb[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }

    // ---- matrix cores
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j) {
        if constexpr (MODE == MODE_TENSOR) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], FA, FB, 0, 0, 0, 0);
        } else if constexpr (MODE == MODE_MX) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], FA, FB, 0, scale_a[i],
                                                                        0, scale_b[j]);
        } else {
          v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], v4f{0.f, 0.f, 0.f, 0.f}, FA, FB, 0,
                                                                    0, 0, 0);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[i][j][jj] = fmaf(p[jj], sab[i][jj], acc[i][j][jj]);
        }
      }

    if (ks + 1 < nk) store_step(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  float s = 1.0f;
  if constexpr (MODE == MODE_TENSOR) s = *static_cast<const float*>(sa_p) * *static_cast<const float*>(sb_p);
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int gn = n0 + wn * Cfg::WN + 16 * j + r;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int gm = m0 + wm * Cfg::WM + 16 * i + 4 * g + jj;
        if (gm < M && gn < N) {
          float v = MODE == MODE_TENSOR ? acc[i][j][jj] * s : acc[i][j][jj];
          if constexpr (OUT == OUT_F32)
            static_cast<float*>(C)[(size_t)gm * N + gn] = v;
          else
            static_cast<uint16_t*>(C)[(size_t)gm * N + gn] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
}

template <int MODE, int FA, int FB, int OUT>
static int launch_gemm(const uint8_t* A, const uint8_t* B, const void* sa, const void* sb, void* C, int M, int N, int K,
                       hipStream_t st) {
  constexpr int BM = 128, BN = 128;
  using Cfg = GemmCfg<BM, BN>;
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  const size_t lds = 2 * (Cfg::LDS_A + Cfg::LDS_B);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, MODE, FA, FB, OUT>), grid, dim3(256), lds, st, A, B, sa, sb, C, M, N, K);
  return check_launch("fp8_gemm");
}

template <int MODE, int FA, int FB>
static int dispatch_out(int out, const uint8_t* A, const uint8_t* B, const void* sa, const void* sb, void* C, int M,
                        int N, int K, hipStream_t st) {
  return out == OUT_F32 ? launch_gemm<MODE, FA, FB, OUT_F32>(A, B, sa, sb, C, M, N, K, st)
                        : launch_gemm<MODE, FA, FB, OUT_BF16>(A, B, sa, sb, C, M, N, K, st);
}

template <int MODE>
static int dispatch_fmt(int fa, int fb, int out, const uint8_t* A, const uint8_t* B, const void* sa, const void* sb,
                        void* C, int M, int N, int K, hipStream_t st) {
  if (fa == FP8_E4M3 && fb == FP8_E4M3) return dispatch_out<MODE, 0, 0>(out, A, B, sa, sb, C, M, N, K, st);
  if (fa == FP8_E5M2 && fb == FP8_E4M3) return dispatch_out<MODE, 1, 0>(out, A, B, sa, sb, C, M, N, K, st);
  if (fa == FP8_E4M3 && fb == FP8_E5M2) return dispatch_out<MODE, 0, 1>(out, A, B, sa, sb, C, M, N, K, st);
  return dispatch_out<MODE, 1, 1>(out, A, B, sa, sb, C, M, N, K, st);
}

}  // namespace sfp8

using namespace sfp8;

extern "C" int fp8_gemm(const uint8_t* A, int fmt_a, const void* a_scale_inv, int gran_a, const uint8_t* B, int fmt_b,
                        const void* b_scale_inv, int gran_b, void* C, int c_dtype, int64_t M, int64_t N, int64_t K,
                        void* stream) {
  SFP8_REQUIRE(M >= 0 && N >= 0 && K >= 0, FP8_ERR_SHAPE, "fp8_gemm: negative shape (%lld, %lld, %lld)",
               (long long)M, (long long)N, (long long)K);
  SFP8_REQUIRE(M < (1ll << 31) && N < (1ll << 31) && K < (1ll << 31), FP8_ERR_SHAPE, "fp8_gemm: dimension >= 2^31");
  SFP8_REQUIRE(K % 128 == 0, FP8_ERR_SHAPE, "fp8_gemm: K=%lld must be a multiple of 128 (pad with zero codes)",
               (long long)K);
  SFP8_REQUIRE((fmt_a == FP8_E4M3 || fmt_a == FP8_E5M2) && (fmt_b == FP8_E4M3 || fmt_b == FP8_E5M2), FP8_ERR_ARG,
               "fp8_gemm: formats (%d, %d)", fmt_a, fmt_b);
  SFP8_REQUIRE(c_dtype == OUT_F32 || c_dtype == OUT_BF16, FP8_ERR_DTYPE, "fp8_gemm: c_dtype %d", c_dtype);
  int mode;
  if (gran_a == FP8_SCALE_TENSOR && gran_b == FP8_SCALE_TENSOR) mode = MODE_TENSOR;
  else if (gran_a == FP8_SCALE_TILE_1x128 && gran_b == FP8_SCALE_BLOCK_128x128) mode = MODE_BLOCK;
  else if (gran_a == FP8_SCALE_MX_1x32 && gran_b == FP8_SCALE_MX_1x32) mode = MODE_MX;
  else
    return set_error(FP8_ERR_ARG,
                     "fp8_gemm: granularity pair (%d, %d) unsupported; use TENSORxTENSOR, TILE_1x128xBLOCK_128x128 or "
                     "MX_1x32xMX_1x32",
                     gran_a, gran_b);
  if (M == 0 || N == 0) return FP8_OK;
  SFP8_REQUIRE(C != nullptr && a_scale_inv != nullptr && b_scale_inv != nullptr, FP8_ERR_ARG,
               "fp8_gemm: null C or scale pointer");
  SFP8_REQUIRE(K == 0 || (A != nullptr && B != nullptr), FP8_ERR_ARG, "fp8_gemm: null A or B");
  SFP8_REQUIRE(K == 0 || (aligned16(A) && aligned16(B)), FP8_ERR_ARG, "fp8_gemm: A and B must be 16-byte aligned");
  SFP8_REQUIRE(mode == MODE_MX || (aligned4(a_scale_inv) && aligned4(b_scale_inv)), FP8_ERR_ARG,
               "fp8_gemm: fp32 scales must be 4-byte aligned");
  SFP8_REQUIRE(aligned4(C), FP8_ERR_ARG, "fp8_gemm: C must be 4-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const int m = (int)M, n = (int)N, k = (int)K;
  if (mode == MODE_TENSOR)
    return dispatch_fmt<MODE_TENSOR>(fmt_a, fmt_b, c_dtype, A, B, a_scale_inv, b_scale_inv, C, m, n, k, st);
  if (mode == MODE_BLOCK)
    return dispatch_fmt<MODE_BLOCK>(fmt_a, fmt_b, c_dtype, A, B, a_scale_inv, b_scale_inv, C, m, n, k, st);
  return dispatch_fmt<MODE_MX>(fmt_a, fmt_b, c_dtype, A, B, a_scale_inv, b_scale_inv, C, m, n, k, st);
}
