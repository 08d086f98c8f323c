// FP8 x FP8 GEMM on gfx950 matrix cores: C[M][N] = sum_k deq(A[m][k]) deq(B[n][k]), templated
// on the epilogue (gemm_epilogue.h) so that the plain and the fused entry points (gemm.hip,
// gemm_fused.hip) share the kernels.
//
// "Week 14" course page: matmuls run in FP8 (FP8 bullet); FP8 products are summed in a
// wider accumulator and partial sums promoted to fp32 at fixed intervals
// (accumulation-precision bullet); MX gives every 32 numbers a shared scale and DeepSeek-V3
// scales 1x128 activation runs and 128x128 weight blocks (absmax bullet).
//
// Kernels: gemm_small.h (128 x 128 tiles, any shape), gemm_w4.h (256 x 256, one wave per SIMD,
// per-tensor and MX), gemm_blk.h (256 x 128 / 256 x 64 ping-pong, blockwise and small per-tensor
// problems).
// This file routes a problem to one of them and holds the host-side checks and dispatch.
#pragma once

#include "gemm_blk.h"
#include "gemm_small.h"
#include "gemm_w4.h"

namespace sfp8 {

// per-tensor problems with fewer 256 x 128 tiles than this run on 256 x 64 tiles (at 200, the
// 144- and 192-tile GEMMs of the MiniGPT layer set moved too and its step got 5-7% slower)
constexpr int64_t kNarrowTiles = 128;
// ... and those whose 128 x 64 tiles number at most this run on them (one tile per CU)
constexpr int64_t kSmallTileMax = 256;

// the kernel for a problem: the 256 x 256 kernel (gemm_w4.h) for per-tensor problems
// of at least 256 of its tiles and for MX; the 256 x 128 / 256 x 64 kernel (gemm_blk.h) for the
// blockwise modes and smaller per-tensor problems; the 128 x 128 kernel (gemm_small.h) where
// neither applies
template <int MODE, int FA, int FB, int OUT, bool FUSED>
static int launch_gemm(const uint8_t* A, const uint8_t* B, const void* sa, const void* sb, const EpiParams& ep, int M,
                       int N, int K, hipStream_t st, const char* what) {
  if constexpr (MODE == MODE_TENSOR) {
    // fewer 256 x 256 tiles than CUs: the 256 x 128 tiles of the blockwise kernel keep twice
    // as many CUs busy (workload 2's per-tensor GEMMs 1.5x faster); from one full wave of
    // tiles on, the 256 x 256 kernel reads less per FLOP and wins
    const int64_t big_tiles = (int64_t)((M + W4_BM - 1) / W4_BM) * ((N + W4_BN - 1) / W4_BN);
    if (big_tiles < 256 && 256ll * K < (1ll << 32)) {
      const int64_t tiles = (int64_t)((M + BLK_BM - 1) / BLK_BM) * ((N + BLK_BN - 1) / BLK_BN);
      // still a fraction of the CUs: 256 x 64 tiles double the count, and 128 x 64 tiles
      // double it again where that still fits one tile per CU
      if (tiles < kNarrowTiles) {
        const int64_t small = (int64_t)((M + 127) / 128) * ((N + 63) / 64);
        if (small <= kSmallTileMax)
          return launch_blk<MODE, FA, FB, OUT, FUSED, 64, 128>(A, B, sa, sb, ep, M, N, K, st, what);
        return launch_blk<MODE, FA, FB, OUT, FUSED, 64>(A, B, sa, sb, ep, M, N, K, st, what);
      }
      return launch_blk<MODE, FA, FB, OUT, FUSED, BLK_BN>(A, B, sa, sb, ep, M, N, K, st, what);
    }
  }
  if constexpr (MODE == MODE_TENSOR || MODE == MODE_MX) {
    // every size it supports: even with a few tiles (e.g. 2048 x 2304 x 768, 72 tiles) it beats
    // the 128 x 128 kernel by 1.2-1.9x; MX scale rows are read as 4-byte runs, so M and N must be
    // multiples of 4 there
    if (M >= 4 && N >= 4 && (MODE != MODE_MX || (M % 4 == 0 && N % 4 == 0))) {
      // the large-tile kernel addresses a tile's rows and a stage's scale rows with 32-bit
      // offsets; beyond that the 128 x 128 kernel (64-bit addressing) takes the problem
      const int64_t mn = M > N ? M : N;
      const bool offsets32 = 256ll * K < (1ll << 32) && (MODE != MODE_MX || (int64_t)(K / 32) * mn < (1ll << 32));
      if (offsets32) return launch_w4<MODE, FA, FB, OUT, FUSED>(A, B, sa, sb, ep, M, N, K, st, what);
    }
  }
  if constexpr (MODE == MODE_BLOCK || MODE == MODE_TILE2) {
    // every size (1.4-3.1x over the 128 x 128 kernel at workload 2's shapes); 32-bit offsets for
    // a tile's rows and a stage's scales
    const int64_t mn = M > N ? M : N;
    const bool offsets32 = 256ll * K < (1ll << 32) && (int64_t)(K / 128) * mn * 4 < (1ll << 32);
    if (offsets32) return launch_blk<MODE, FA, FB, OUT, FUSED, BLK_BN>(A, B, sa, sb, ep, M, N, K, st, what);
  }
  constexpr int BM = 128, BN = 128;
  using Cfg = GemmCfg<BM, BN>;
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  const size_t lds = 2 * (Cfg::LDS_A + Cfg::LDS_B);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, MODE, FA, FB, OUT, FUSED>), grid, dim3(256), lds, st, A, B, sa, sb, ep, M, N, K);
  return check_launch(what);
}

// ------------------------------------------------------------------ host-side dispatch

// granularity pair -> MODE_*, or -1
static inline int gemm_mode(int gran_a, int gran_b) {
  if (gran_a == FP8_SCALE_TENSOR && gran_b == FP8_SCALE_TENSOR) return MODE_TENSOR;
  if (gran_a == FP8_SCALE_TILE_1x128 && gran_b == FP8_SCALE_BLOCK_128x128) return MODE_BLOCK;
  if (gran_a == FP8_SCALE_TILE_1x128 && gran_b == FP8_SCALE_TILE_1x128) return MODE_TILE2;
  if (gran_a == FP8_SCALE_MX_1x32 && gran_b == FP8_SCALE_MX_1x32) return MODE_MX;
  return -1;
}

// argument checks shared by the GEMM entry points (everything but C and the epilogue);
// sets `mode` on success
static inline int gemm_check(const char* what, const uint8_t* A, int fmt_a, const void* a_scale_inv, int gran_a,
                             const uint8_t* B, int fmt_b, const void* b_scale_inv, int gran_b, int64_t M, int64_t N,
                             int64_t K, int& mode) {
  SFP8_REQUIRE(M >= 0 && N >= 0 && K >= 0, FP8_ERR_SHAPE, "%s: negative shape (%lld, %lld, %lld)", what,
               (long long)M, (long long)N, (long long)K);
  SFP8_REQUIRE(M < (1ll << 31) && N < (1ll << 31) && K < (1ll << 31), FP8_ERR_SHAPE, "%s: dimension >= 2^31", what);
  SFP8_REQUIRE(K % 128 == 0, FP8_ERR_SHAPE, "%s: K=%lld must be a multiple of 128 (pad with zero codes)", what,
               (long long)K);
  SFP8_REQUIRE((fmt_a == FP8_E4M3 || fmt_a == FP8_E5M2) && (fmt_b == FP8_E4M3 || fmt_b == FP8_E5M2), FP8_ERR_ARG,
               "%s: formats (%d, %d)", what, fmt_a, fmt_b);
  mode = gemm_mode(gran_a, gran_b);
  if (mode < 0)
    return set_error(FP8_ERR_ARG,
                     "%s: granularity pair (%d, %d) unsupported; use TENSORxTENSOR, TILE_1x128xBLOCK_128x128, "
                     "TILE_1x128xTILE_1x128 or MX_1x32xMX_1x32",
                     what, gran_a, gran_b);
  if (M == 0 || N == 0) return FP8_OK;
  SFP8_REQUIRE(a_scale_inv != nullptr && b_scale_inv != nullptr, FP8_ERR_ARG, "%s: null scale pointer", what);
  SFP8_REQUIRE(K == 0 || (A != nullptr && B != nullptr), FP8_ERR_ARG, "%s: null A or B", what);
  SFP8_REQUIRE(K == 0 || (aligned16(A) && aligned16(B)), FP8_ERR_ARG, "%s: A and B must be 16-byte aligned", what);
  SFP8_REQUIRE(mode == MODE_MX || (aligned4(a_scale_inv) && aligned4(b_scale_inv)), FP8_ERR_ARG,
               "%s: fp32 scales must be 4-byte aligned", what);
  return FP8_OK;
}

template <int MODE, int OUT, bool FUSED>
static int dispatch_fmt(int fa, int fb, const uint8_t* A, const uint8_t* B, const void* sa, const void* sb,
                        const EpiParams& ep, int M, int N, int K, hipStream_t st, const char* what) {
  if (fa == FP8_E4M3 && fb == FP8_E4M3) return launch_gemm<MODE, 0, 0, OUT, FUSED>(A, B, sa, sb, ep, M, N, K, st, what);
  if (fa == FP8_E5M2 && fb == FP8_E4M3) return launch_gemm<MODE, 1, 0, OUT, FUSED>(A, B, sa, sb, ep, M, N, K, st, what);
  if constexpr (!FUSED) {  // the fused entry point takes B in E4M3 only (checked on the host)
    if (fa == FP8_E4M3 && fb == FP8_E5M2) return launch_gemm<MODE, 0, 1, OUT, FUSED>(A, B, sa, sb, ep, M, N, K, st, what);
    return launch_gemm<MODE, 1, 1, OUT, FUSED>(A, B, sa, sb, ep, M, N, K, st, what);
  }
  return set_error(FP8_ERR_ARG, "%s: B must be E4M3", what);
}

template <int OUT, bool FUSED>
static int dispatch_mode(int mode, int fa, int fb, const uint8_t* A, const uint8_t* B, const void* sa, const void* sb,
                         const EpiParams& ep, int M, int N, int K, hipStream_t st, const char* what) {
  if (mode == MODE_TENSOR) return dispatch_fmt<MODE_TENSOR, OUT, FUSED>(fa, fb, A, B, sa, sb, ep, M, N, K, st, what);
  if (mode == MODE_BLOCK) return dispatch_fmt<MODE_BLOCK, OUT, FUSED>(fa, fb, A, B, sa, sb, ep, M, N, K, st, what);
  if (mode == MODE_TILE2) return dispatch_fmt<MODE_TILE2, OUT, FUSED>(fa, fb, A, B, sa, sb, ep, M, N, K, st, what);
  return dispatch_fmt<MODE_MX, OUT, FUSED>(fa, fb, A, B, sa, sb, ep, M, N, K, st, what);
}

}  // namespace sfp8

