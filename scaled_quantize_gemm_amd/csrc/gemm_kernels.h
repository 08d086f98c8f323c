// FP8 x FP8 GEMM kernels on gfx950 matrix cores: C[M][N] = sum_k deq(A[m][k]) deq(B[n][k]),
// templated on the epilogue (gemm_epilogue.h) so that the plain and the fused entry points
// (gemm.hip, gemm_fused.hip) share them.
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
//  * TILE2:   both operands in 1x128 runs along K: acc += p * (sa[kb][m] * sb[kb][n]).
//  * MX:      scaled MFMA with the e8m0 codes of A[m][4kb+g] and B[n][4kb+g]; C = acc.
#pragma once

#include <type_traits>

#include "common.h"
#include "gemm_epilogue.h"

namespace sfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum { MODE_TENSOR = 0, MODE_BLOCK = 1, MODE_MX = 2, MODE_TILE2 = 3 };

template <int BM, int BN>
struct GemmCfg {
  static constexpr int BK = 128;
  static constexpr int WM = BM / 2, WN = BN / 2;  // wave tile
  static constexpr int TM = WM / 16, TN = WN / 16;  // MFMA tiles per wave
  static constexpr int A_CHUNKS = BM * BK / 16, B_CHUNKS = BN * BK / 16;
  static constexpr int A_PER_T = A_CHUNKS / 256, B_PER_T = B_CHUNKS / 256;
  static constexpr int LDS_A = BM * BK, LDS_B = BN * BK;  // bytes per stage
};

// byte offset of 16-byte chunk c of tile row `row` in a 128-byte-row LDS tile; the position
// c ^ ((row >> 1) ^ ((row & 1) << 2)) is distinct over any 8 consecutive rows (32 banks) and
// over 16 consecutive rows for each row parity (64 banks), so fragment reads do not conflict
__device__ __forceinline__ int swz(int row, int c) { return row * 128 + ((c ^ (((row >> 1) ^ ((row & 1) << 2)) & 7)) << 4); }

template <int BM, int BN, int MODE, int FA, int FB, int OUT, bool FUSED>
__global__ void __launch_bounds__(256) gemm_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                   const void* __restrict__ sa_p, const void* __restrict__ sb_p,
                                                   const EpiParams ep, int M, int N, int K) {
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
    float sab[Cfg::TM][4], sbc[Cfg::TN];
    int scale_a[Cfg::TM], scale_b[Cfg::TN];
    if constexpr (MODE == MODE_BLOCK || MODE == MODE_TILE2) {
      const float* sa = static_cast<const float*>(sa_p);
      const float* sb = static_cast<const float*>(sb_p);
      const float sbv = MODE == MODE_BLOCK ? sb[(size_t)(n0 / 128) * nk + ks] : 1.0f;
      if constexpr (MODE == MODE_TILE2) {
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j) {
          int gn = n0 + wn * Cfg::WN + 16 * j + r;
          gn = gn < N ? gn : N - 1;
          sbc[j] = sb[(size_t)ks * N + gn];  // [K/128][N]
        }
      }
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
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i) {
        int gm = m0 + wm * Cfg::WM + 16 * i + r;
        gm = gm < M ? gm : M - 1;
        scale_a[i] = ea[(size_t)(4 * ks + g) * M + gm];  // e8m0 layout [K/32][M]
      }
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j) {
        int gn = n0 + wn * Cfg::WN + 16 * j + r;
        gn = gn < N ? gn : N - 1;
        scale_b[j] = eb[(size_t)(4 * ks + g) * N + gn];
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
          for (int jj = 0; jj < 4; ++jj)
            acc[i][j][jj] = fmaf(p[jj], MODE == MODE_TILE2 ? sab[i][jj] * sbc[j] : sab[i][jj], acc[i][j][jj]);
        }
      }

    if (ks + 1 < nk) store_step(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane (g, r) holds column 16j + r of rows 4g + jj of tile (i, j)
  Epilogue<OUT, FUSED> epi(ep);
  float s = 1.0f;
  if constexpr (MODE == MODE_TENSOR) s = *static_cast<const float*>(sa_p) * *static_cast<const float*>(sb_p);
  epi.with_act([&](auto act_c) {
    constexpr int ACT = decltype(act_c)::value;
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int gn = n0 + wn * Cfg::WN + 16 * j + r;
      float b[1];
      epi.template bias<1>(gn, N, b);
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int gm = m0 + wm * Cfg::WM + 16 * i + 4 * g + jj;
          const bool in = gm < M && gn < N;
          float v[1] = {MODE == MODE_TENSOR ? acc[i][j][jj] * s : acc[i][j][jj]};
          epi.pre(v, b);
          if (in) epi.aux(v, gm, gn, N, true);
          if constexpr (ACT == FP8_ACT_SWIGLU) {
            // the up value of an even (gate) column is held by the next lane
            float w[2] = {v[0], __shfl_xor(v[0], 1, 64)};
            if (in && (r & 1) == 0) epi.template out<ACT>(w, gm, gn, N, true);
          } else if (in) {
            epi.template out<ACT>(v, gm, gn, N, true);
          }
        }
    }
  });
  epi.finish(lane, reinterpret_cast<uint32_t*>(smem));
}

// ------------------------------------------------------------------ large-tile kernel
//
// Definitions shared by the large-tile kernel below: a 256 x 256 block tile (per-tensor and
// MX scaling), K staged 64 at a time through LDS stages that are
// filled by direct-to-LDS loads (lane L's 16 bytes land at the instruction's LDS base + 16 L),
// so no registers hold tiles in flight.
//
// 32x32x64 operand layout: lane l = 32 g + r supplies row r; bytes 0-15 hold K = 16g..16g+15
// and bytes 16-31 K = 32+16g..; result register e of lane l is C[8(e/4) + 4g + e%4][r]; in the
// scaled form lane l's e8m0 byte scales row r over K = 32g..32g+31 of the 64-long step.
//
// LDS stage: A [256 rows][64 B], B [256][64 B], then (MX) the stage's two K-blocks of e8m0
// scales for A [2][256] and B [2][256].  16-byte chunk c of a 64-byte row sits at position
// c ^ (((row >> 2) ^ (row >> 1)) & 3): the rows one 128-bit read phase touches (8 rows over
// 32 banks, or 16 rows over 64 banks) then cover distinct banks, and rows 32 apart share it.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs (each with its own L2), so
// block b runs on XCD b % 8; each XCD gets a contiguous range of tiles, walked in groups of
// 4 tile-rows so that the tiles resident on one XCD share A rows and B columns.

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BIG_BM = 256, BIG_BN = 256, BIG_BK = 64;
constexpr int BIG_TILE_BYTES = (BIG_BM + BIG_BN) * BIG_BK;  // 32 KB
constexpr int BIG_SCALE_BYTES = 2 * (BIG_BM + BIG_BN);      // 1 KB (MX only)

__device__ __forceinline__ int bswz_pos(int row) { return ((row >> 2) ^ (row >> 1)) & 3; }
__device__ __forceinline__ int bswz(int row, int c) { return row * 64 + ((c ^ bswz_pos(row)) << 4); }

__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int xcd = b & 7, idx = b >> 3;
  const int per = T >> 3, rem = T & 7;
  const int t = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  constexpr int GM = 4;
  const int group = t / (GM * tiles_n);
  const int first = group * GM;
  const int gsz = (tiles_m - first) < GM ? (tiles_m - first) : GM;
  const int in = t - group * GM * tiles_n;
  tm = first + in % gsz;
  tn = in / gsz;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// ------------------------------------------------------------------ ping-pong large-tile kernel
//
// 256 x 256 block tile, K step 64, a 4-stage LDS ring fed by direct-to-LDS loads issued 3
// stages ahead, and 8 waves in two groups of 4.  Group p computes tile rows 128p .. 128p+127; wave i
// of a group computes tile columns 64i .. 64i+63 (a 128 x 64 wave tile: 4 x 2 MFMAs of
// 32x32x64 per K step, 128 fp32 accumulators per lane).  Waves w and w+4 share a SIMD.
//
// Every wave runs the same sequence M_0 C_0 M_1 C_1 ..., each phase closed by a workgroup
// barrier; group 1 starts one barrier late, so at any time one group computes while the
// other moves data, and each SIMD's matrix core is fed by whichever of its two waves is in
// its compute phase.
//   M_k: issue this wave's part of stage k+3 into the buffer stage k-1 used; read stage k's
//        A fragments (and A scales).
//   C_k: the 8 MFMAs of stage k; meanwhile read stage k+1's B fragments (and B scales) into
//        the other B register set, so that both waves of a SIMD keep LDS reads in flight;
//        then wait for this wave's part of stage k+2.
// Slot 2k holds M_k of group 0 and C_{k-1} of group 1; slot 2k+1 holds C_k of group 0 and
// M_k of group 1.  Stage k+2 is complete (both groups waited for it by the ends of slots
// 2k+1 and 2k+2) and published by the barrier closing slot 2k+2, before group 0 reads its B
// fragments in slot 2k+3.  Stage k-1's buffer is last read in slot 2k-1 (group 1's M_{k-1}),
// and every read is waited for (lgkmcnt) before the barrier that closes the reading wave's
// next memory phase, so the refill issued from slot 2k on overwrites nothing still needed.
//
// Row interleave: MFMA tile i of group p holds tile rows 128p + 4t + i (t = 0..31, the MFMA
// row) and MFMA tile j of wave i holds columns 64i + 2t + j.  The DMA places those rows at
// LDS rows 128p + 32i + t (resp. 64i + 32j + t), so fragment reads keep the bank-conflict-free
// swizzle, while a lane's four A scales (rows 4t..4t+3) and two B scales (columns 2t, 2t+1)
// are adjacent bytes: one LDS read each, the byte picked by the MFMA's scale selector.  In
// the epilogue a lane then holds 2 adjacent columns of 4 adjacent rows, and writes pairs.
//
// LDS reads are inline assembly with immediate offsets from a few per-lane base registers:
// the compiler neither tracks them (it cannot tell that they never touch a stage with loads
// in flight, and would wait for every outstanding load) nor needs registers per address.

// MFMAs of a compute phase issued before its loads of the next B fragments
constexpr int kPPLead = 2;
// memory phase: fragment reads before the stage refill's loads
constexpr bool kPPReadsFirst = true;
// buffer resource word 3 for raw byte-addressed buffers on gfx9 (32-bit data format, no swizzle)
constexpr int kBufferFlags = 0x00020000;

template <int OFF>
__device__ __forceinline__ u32x4 ds_read16(uint32_t vaddr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field is 16 bits");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(vaddr), "i"(OFF) : "memory");
  return v;
}
template <int OFF>
__device__ __forceinline__ uint32_t ds_read4(uint32_t vaddr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field is 16 bits");
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(vaddr), "i"(OFF) : "memory");
  return v;
}
template <int OFF>
__device__ __forceinline__ uint32_t ds_read2(uint32_t vaddr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field is 16 bits");
  uint32_t v;
  asm volatile("ds_read_u16 %0, %1 offset:%2" : "=v"(v) : "v"(vaddr), "i"(OFF) : "memory");
  return v;
}

// compile-time unrolling: f(integral_constant<int, I>) for I = 0 .. N-1
template <typename F, int... Is>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}

// NST: LDS ring depth (stages in flight NST - 1 ahead); 4 x 34 KB for MX, 5 x 32 KB per tensor
template <int MODE, int FA, int FB, int OUT, bool FUSED, int NST>
__global__ void __launch_bounds__(512, 1) gemm_pp_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                         const void* __restrict__ sa_p, const void* __restrict__ sb_p,
                                                         const EpiParams ep, int M, int N, int K, int tiles_m,
                                                         int tiles_n) {
  constexpr bool MX = MODE == MODE_MX;
  // MX: each group loads its own copy of the stage's scale rows, so that every wave issues the
  // same loads and the steady-state loop has no group-dependent branch
  constexpr int STAGE = BIG_TILE_BYTES + (MX ? 2 * BIG_SCALE_BYTES : 0);
  constexpr int B_OFF = BIG_BM * BIG_BK, S_OFF = BIG_TILE_BYTES;
  constexpr int D = NST - 1;                  // stages issued ahead
  constexpr int U = NST % 2 == 0 ? NST : 2 * NST;  // unroll: stage buffer and B set both repeat
  static_assert(NST >= 4 && NST * STAGE <= 160 * 1024, "LDS ring must fit the 160 KB of a CU");
  static_assert(STAGE + B_OFF + 2048 + 16 < 65536, "odd stages' offsets must fit the LDS offset field");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wi = wave & 3;
  const int g = lane >> 5, r = lane & 31;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BIG_BM, n0 = tn * BIG_BN;
  const int nk = K / BIG_BK;

  // ---- this group's half of each stage: group 0 the A rows, group 1 the B rows, through a
  //      buffer resource (uniform base, 32-bit lane offsets, range = the rows present); rows
  //      past the matrix edge re-read its last row
  const int lim = grp == 0 ? M - m0 : N - n0;
  const uint8_t* d_base = grp == 0 ? A + (size_t)m0 * K : B + (size_t)n0 * K;
  const uint64_t d_bytes = (uint64_t)lim * (uint64_t)K;
  const __amdgpu_buffer_rsrc_t d_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(d_base), (short)0, (int)(d_bytes < 0xFFFFFFFFull ? d_bytes : 0xFFFFFFFFull), kBufferFlags);
  const int d_lds = grp * B_OFF;
  uint32_t od[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = (wi * 4 + i) * 64 + lane;
    const int q = slot >> 2, c = (slot & 3) ^ bswz_pos(q);  // LDS row q, global 16-byte chunk c
    const int row = grp == 0 ? (q & ~127) + 4 * (q & 31) + ((q >> 5) & 3)   // A: 128p + 4t + i
                             : (q & ~63) + 2 * (q & 31) + ((q >> 5) & 1);   // B: 64w + 2t + j
    const int rr = row < lim ? row : lim - 1;
    od[i] = (uint32_t)rr * (uint32_t)K + c * 16;
  }
  // MX scales: wave i of each group loads scale row i of the stage (A K-blocks 2s, 2s+1, then
  // B's) into its group's copy
  __amdgpu_buffer_rsrc_t s_rsrc = d_rsrc;  // replaced below (MX)
  uint32_t os = 0;
  int s_lim = 0;
  if constexpr (MX) {
    const bool isb = wi >= 2;
    s_lim = isb ? N : M;
    const int base_row = isb ? n0 : m0;
    const uint8_t* s_base = static_cast<const uint8_t*>(isb ? sb_p : sa_p) + (size_t)(wi & 1) * s_lim + base_row;
    const uint64_t s_bytes = (uint64_t)(K / 32) * s_lim - ((uint64_t)(wi & 1) * s_lim + base_row);
    s_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(s_base), (short)0,
                                               (int)(s_bytes < 0xFFFFFFFFull ? s_bytes : 0xFFFFFFFFull), kBufferFlags);
    const int rel = lane * 4, room = s_lim - 4 - base_row;  // M, N multiples of 4 here
    os = (uint32_t)(rel < room ? rel : room);
  }
  auto issue = [&](int ks, int st) {
    uint8_t* buf = smem + st * STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(d_rsrc, (lds_ptr_t)(buf + d_lds + (wi * 4 + i) * 1024), 16, od[i],
                                               ks * BIG_BK, 0, 0);
    if constexpr (MX)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_ptr_t)(buf + S_OFF + grp * BIG_SCALE_BYTES + wi * 256), 4,
                                               os, 2 * ks * s_lim, 0, 0);
  };
  // wait until at most `later` stages of this wave's loads are in flight (they retire in order)
  auto wait_stage = [&](int later) {
    if (later >= 3) {
      if constexpr (MX) asm volatile("s_waitcnt vmcnt(15)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    } else if (later == 2) {
      if constexpr (MX) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    } else if (later == 1) {
      if constexpr (MX) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };

  // ---- per-lane LDS base addresses; stage s, tile i adds the immediate (s%2)*STAGE + i*2048
  //      to the base set of stage pair s/2, keeping offsets within 16 bits
  constexpr int NH = (NST + 1) / 2;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const uint32_t row_lo = r * 64 + ((g ^ bswz_pos(r)) << 4), row_hi = r * 64 + (((g + 2) ^ bswz_pos(r)) << 4);
  uint32_t a_lo[NH], a_hi[NH], b_lo[NH], b_hi[NH], s_a[NH], s_b[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const uint32_t base = lds0 + h * 2 * STAGE;
    a_lo[h] = base + grp * 128 * 64 + row_lo;
    a_hi[h] = base + grp * 128 * 64 + row_hi;
    b_lo[h] = base + B_OFF + wi * 64 * 64 + row_lo;
    b_hi[h] = base + B_OFF + wi * 64 * 64 + row_hi;
    s_a[h] = base + S_OFF + grp * BIG_SCALE_BYTES + g * 256 + grp * 128 + 4 * r;
    s_b[h] = base + S_OFF + grp * BIG_SCALE_BYTES + 512 + g * 256 + wi * 64 + 2 * r;
  }

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragments: A of the current stage, B of the current and the next stage (two sets);
  // fsa / fsb pack the e8m0 bytes of tiles i = 0..3 / j = 0..1
  v8i fa[4], fb[2][2];
  int fsa = 0, fsb[2] = {0, 0};
  auto pack = [](const u32x4& lo, const u32x4& hi) -> v8i {
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  // ST: stage buffer 0 .. NST-1 (compile time); SET: B register set
  auto read_a = [&](auto st_c) {
    constexpr int ST = decltype(st_c)::value, H = ST >> 1, O = (ST & 1) * STAGE;
    fa[0] = pack(ds_read16<O + 0 * 2048>(a_lo[H]), ds_read16<O + 0 * 2048>(a_hi[H]));
    fa[1] = pack(ds_read16<O + 1 * 2048>(a_lo[H]), ds_read16<O + 1 * 2048>(a_hi[H]));
    fa[2] = pack(ds_read16<O + 2 * 2048>(a_lo[H]), ds_read16<O + 2 * 2048>(a_hi[H]));
    fa[3] = pack(ds_read16<O + 3 * 2048>(a_lo[H]), ds_read16<O + 3 * 2048>(a_hi[H]));
    if constexpr (MX) fsa = (int)ds_read4<O>(s_a[H]);
  };
  auto read_b = [&](auto st_c, auto set_c) {
    constexpr int ST = decltype(st_c)::value, H = ST >> 1, O = (ST & 1) * STAGE;
    constexpr int SET = decltype(set_c)::value;
    fb[SET][0] = pack(ds_read16<O + 0 * 2048>(b_lo[H]), ds_read16<O + 0 * 2048>(b_hi[H]));
    fb[SET][1] = pack(ds_read16<O + 1 * 2048>(b_lo[H]), ds_read16<O + 1 * 2048>(b_hi[H]));
    if constexpr (MX) fsb[SET] = (int)ds_read2<O>(s_b[H]);
  };
  // MFMA n of a stage: tile (n / 2, n % 2)
  auto mfma = [&](auto n_c, auto set_c) {
    constexpr int n = decltype(n_c)::value, I = n / 2, J = n % 2, SET = decltype(set_c)::value;
    acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[I], fb[SET][J], acc[I][J], FA, FB, MX ? I : 0, fsa,
                                                                 MX ? J : 0, fsb[SET]);
  };
  // the stage's 8 MFMAs with `between` issued after the first kPPLead of them; the fragments
  // stay live to the end, so that loads issued in `between` never target registers an
  // earlier MFMA of this run reads
  auto compute = [&](auto set_c, auto&& between) {
    constexpr int SET = decltype(set_c)::value;
    auto at = [&](auto n_c) {
      constexpr int n = decltype(n_c)::value;
      if constexpr (n == kPPLead) {
        __builtin_amdgcn_sched_barrier(0);
        between();
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma(n_c, set_c);
    };
    at(std::integral_constant<int, 0>{});
    at(std::integral_constant<int, 1>{});
    at(std::integral_constant<int, 2>{});
    at(std::integral_constant<int, 3>{});
    at(std::integral_constant<int, 4>{});
    at(std::integral_constant<int, 5>{});
    at(std::integral_constant<int, 6>{});
    at(std::integral_constant<int, 7>{});
    __builtin_amdgcn_sched_barrier(0);
    const v8i a0 = fa[0], a1 = fa[1], a2 = fa[2], a3 = fa[3], b0 = fb[SET][0], b1 = fb[SET][1];
    asm volatile("" ::"v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b0), "v"(b1));
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;

  // M_k then C_k for stage k in buffer ST (= k % NST), B set SET (= k % 2).  STEADY steps
  // (stage k+D exists) contain no branch, so the compiler keeps each phase's MFMAs between its
  // two barriers.  The barrier closing slot 2nk-1 (group 0 after C_{nk-1}, group 1 after
  // M_{nk-1}) and group 1's last one are dropped: no LDS is written or read after them.
  auto step = [&](auto steady, auto st_c, auto set_c, int k) {
    constexpr bool STEADY = decltype(steady)::value;
    constexpr int ST = decltype(st_c)::value, SET = decltype(set_c)::value;
    using NextSt = std::integral_constant<int, (ST + 1) % NST>;
    using NextSet = std::integral_constant<int, SET ^ 1>;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPPReadsFirst) {
      read_a(st_c);
      __builtin_amdgcn_sched_barrier(0);
      if (STEADY || k + D < nk) issue(k + D, (ST + D) % NST);
    } else {
      if (STEADY || k + D < nk) issue(k + D, (ST + D) % NST);
      __builtin_amdgcn_sched_barrier(0);
      read_a(st_c);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // A (and the previous C's B) in registers
    if (STEADY || !(grp == 1 && k + 1 == nk)) barrier();
    compute(set_c, [&]() {
      if (STEADY || k + 1 < nk) read_b(NextSt{}, NextSet{});
    });
    __builtin_amdgcn_sched_barrier(0);  // the wait below must not split the MFMA run
    if constexpr (STEADY) {
      wait_stage(D - 2);  // this wave's part of stage k+2
    } else {
      if (k + 2 < nk) wait_stage(nk - k - 3 < D - 2 ? nk - k - 3 : D - 2);
    }
    if (STEADY || k + 1 < nk) barrier();
  };
  using steady_t = std::integral_constant<bool, true>;
  using tail_t = std::integral_constant<bool, false>;

  if (nk > 0) {
    unroll_seq([&](auto s_c) {
      constexpr int S = decltype(s_c)::value;
      if (S < nk) issue(S, S);
    }, std::make_integer_sequence<int, D>{});
    // this wave's parts of stages 0 and 1 landed: of the first min(D, nk) stages, the later
    // ones may stay in flight
    const int issued = nk < D ? nk : D, need = nk > 1 ? 2 : 1;
    wait_stage(issued - need);
    barrier();                  // stages 0 and 1 visible
    read_b(I0{}, I0{});         // stage 0's B set
    if (grp == 1) barrier();    // group 1 sits out slot 0
    int k = 0;
    for (; k + U + D <= nk; k += U)  // every step of the block has a stage D ahead to issue
      unroll_seq([&](auto i_c) {
        constexpr int I = decltype(i_c)::value;
        step(steady_t{}, std::integral_constant<int, I % NST>{}, std::integral_constant<int, I % 2>{}, k + I);
      }, std::make_integer_sequence<int, U>{});
    for (; k < nk; k += U)
      unroll_seq([&](auto i_c) {
        constexpr int I = decltype(i_c)::value;
        if (k + I < nk)
          step(tail_t{}, std::integral_constant<int, I % NST>{}, std::integral_constant<int, I % 2>{}, k + I);
      }, std::make_integer_sequence<int, U>{});
  }

  // ---- epilogue: result register e of tile (i, j) is tile row 128p + 4(8(e/4) + 4g + e%4) + i,
  //      column 64w + 2r + j: each lane writes column pairs (2r, 2r+1).  The stores are
  //      nontemporal: C goes on to HBM while other tiles still compute, instead of staying
  //      dirty in the caches for whatever kernel runs next to write back.
  Epilogue<OUT, FUSED> epi(ep);
  float scale = 1.0f;
  if constexpr (MODE == MODE_TENSOR) scale = *static_cast<const float*>(sa_p) * *static_cast<const float*>(sb_p);
  const int gn = n0 + wi * 64 + 2 * r;
  const bool pair = (N & 1) == 0 && gn + 1 < N;  // both columns present, pair store aligned
  float b[2];
  epi.template bias<2>(gn, N, b);
  epi.with_act([&](auto act_c) {
    constexpr int ACT = decltype(act_c)::value;
#pragma unroll
    for (int e = 0; e < 16; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gm = m0 + grp * 128 + 4 * (8 * (e >> 2) + 4 * g + (e & 3)) + i;
        if (gm >= M) continue;
        float v[2] = {acc[i][0][e], acc[i][1][e]};
        if constexpr (MODE == MODE_TENSOR) {
          v[0] *= scale;
          v[1] *= scale;
        }
        epi.pre(v, b);
        epi.aux(v, gm, gn, N, pair);
        epi.template out<ACT>(v, gm, gn, N, pair);
      }
  });
  epi.finish(lane, reinterpret_cast<uint32_t*>(smem));
}

// ------------------------------------------------------------------ blockwise large-tile kernel
//
// 1x128 activation tiles x 128x128 weight blocks (DeepSeek-V3 style scaling, per the course
// page's absmax bullet): every 128-K block's partial product is scaled by
// sa[kb][m] * sb[n/128][kb] and added into an fp32 accumulator.  The K step is one scale
// block (128), so each 16x16x128 MFMA computes a whole block's partial for a 16 x 16 tile
// from zero, and the partial goes straight into the accumulator with one fma: no second set
// of accumulators is needed.
//
// Block tile 256 x 128 (one weight block column), 3-stage LDS ring of 50 KB (A 256 x 128 B,
// B 128 x 128 B, the stage's 256 row scales, copies of its weight-block scale), filled by
// direct-to-LDS loads 2 stages ahead.  8 waves: group p = wave / 4 holds tile rows
// 128p .. 128p+127; wave i of a group takes the 64 x 64 slab at rows 64 (i / 2), columns
// 64 (i % 2): 4 x 4 tiles of 16x16, 64 fp32 accumulators per lane.  Same ping-pong as the
// kernel above (memory phase: this wave's loads of stage k+2, all of stage k's fragments and
// scales; compute phase: 16 MFMAs and 64 fmas), with group 1 one barrier behind.
//
// 16x16x128 operand layout: lane l = 16 g + r supplies row r; its 32 bytes are K = 16g..16g+15
// and K = 64+16g..64+16g+15; result register jj of lane l is C[4g + jj][r].
// Row interleave: tile i's MFMA row t is slab row 4t + i, tile j's column t is slab column
// 4t + j (the DMA places them at LDS rows 16i + t / 16j + t).  A lane's 16 accumulator rows
// (16g + 4jj + i) are then 16 consecutive rows, whose scales are one 64-byte LDS read, and its
// 4 columns per row (4r + j) leave as one 8-byte (bf16) or 16-byte (fp32) store.

constexpr int BLK_BM = 256, BLK_BN = 128, BLK_BK = 128;
constexpr int BLK_B_OFF = BLK_BM * BLK_BK;               // 32 KB of A
constexpr int BLK_SA_OFF = BLK_B_OFF + BLK_BN * BLK_BK;  // 16 KB of B
constexpr int BLK_SB_OFF = BLK_SA_OFF + 1024;            // 256 row scales
constexpr int BLK_STAGE = BLK_SB_OFF + 1024;             // 4 copies x 64 of the block scale
constexpr int BLK_NST = 3;

// the tile row held at LDS row q of a 64-row slab layout (tile i's MFMA row t at 16i + t is
// slab row 4t + i)
__device__ __forceinline__ int blk_row_of(int q) { return (q & ~63) + 4 * (q & 15) + ((q >> 4) & 3); }
// the B row (output column) held at LDS row q of a slab of 16 NT columns: MFMA tile j's
// column t at LDS row 16j + t is slab column NT t + j (NT = 4: the same map as the rows)
__device__ __forceinline__ int blk_col_of(int q, int nt) {
  return (q & ~(16 * nt - 1)) + nt * (q & 15) + ((q >> 4) & (nt - 1));
}
// position of 16-byte chunk c in 128-byte LDS row q (the small-tile kernel's swizzle)
__device__ __forceinline__ int blk_pos(int q, int c) { return c ^ (((q >> 1) ^ ((q & 1) << 2)) & 7); }

// MODE: MODE_BLOCK (B scales per 128x128 block: one value per stage), MODE_TILE2 (B scales
// per 1x128 run along K: one per column per stage, [K/128][N]) or MODE_TENSOR (no scale loads;
// the MFMAs accumulate straight into acc and the epilogue multiplies by sa * sb: the 256 x 128
// tile gives small per-tensor problems twice the tiles of the 256 x 256 kernel)
// the tile-width-dependent shape of the kernel below: NT MFMA column tiles per wave slab of SW
// columns; the B rows of a stage are BN x 128 B, loaded as NB of the stage's NOPS 1 KB
// operations (OPW per wave).
template <int BN>
struct BlkShape {
  static constexpr int NT = BN / 32, SW = BN / 2, NB = BN / 8, NOPS = 32 + NB, OPW = NOPS / 8;
  static constexpr int SA_OFF = BLK_B_OFF + BN * BLK_BK, SB_OFF = SA_OFF + 1024, STAGE = SB_OFF + 1024;
};

template <int MODE, int FA, int FB, int OUT, bool FUSED, int BN>
__global__ void __launch_bounds__(512, 1) gemm_blk_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                          const float* __restrict__ sa_p,
                                                          const float* __restrict__ sb_p, const EpiParams ep, int M,
                                                          int N, int K, int tiles_m, int tiles_n) {
  constexpr bool TENSOR = MODE == MODE_TENSOR;
  static_assert(BN == BLK_BN || (BN == 64 && TENSOR), "256 x 64 tiles serve per-tensor scaling only");
  using Shape = BlkShape<BN>;
  constexpr int NT = Shape::NT, SW = Shape::SW, NOPS = Shape::NOPS, OPW = Shape::OPW;
  constexpr int SA_OFF = Shape::SA_OFF, SB_OFF = Shape::SB_OFF, STAGE = Shape::STAGE;
  constexpr int NST = BLK_NST, D = NST - 1, U = NST;
  static_assert(NOPS % 8 == 0, "every wave issues the same number of loads");
  static_assert(NST * STAGE <= 160 * 1024, "LDS ring must fit the 160 KB of a CU");
  __shared__ __attribute__((aligned(16))) uint8_t smem[BLK_NST * Shape::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wi = wave & 3, wr = wi >> 1, wc = wi & 1;
  const int g = lane >> 4, r = lane & 15;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BLK_BM, n0 = tn * BN;
  const int nk = K / BLK_BK;

  // ---- loads: NOPS x 1 KB of tile data per stage, OPW per wave (ops 0..31 are A, then B), and
  //      one scale load per wave (waves 0-3: 64 row scales each; 4-7: a copy of the block scale)
  const int lim_a = M - m0, lim_b = N - n0;
  const uint64_t a_bytes = (uint64_t)lim_a * K, b_bytes = (uint64_t)lim_b * K;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(A + (size_t)m0 * K), (short)0, (int)(a_bytes < 0xFFFFFFFFull ? a_bytes : 0xFFFFFFFFull),
      kBufferFlags);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(B + (size_t)n0 * K), (short)0, (int)(b_bytes < 0xFFFFFFFFull ? b_bytes : 0xFFFFFFFFull),
      kBufferFlags);
  // fixed size, OPW <= 6 of them used: sized by OPW, the array made the host compiler drop
  // this kernel's launch stubs (every instantiation, with no diagnostic)
  static_assert(OPW <= 6, "load offsets per wave");
  uint32_t od[6];
#pragma unroll
  for (int i = 0; i < OPW; ++i) {
    const int o = wave * OPW + i, local = o < 32 ? o : o - 32;
    const int slot = local * 64 + lane, q = slot >> 3, c = blk_pos(q, slot & 7);
    const int row = o < 32 ? blk_row_of(q) : blk_col_of(q, NT), lim = o < 32 ? lim_a : lim_b;
    od[i] = (uint32_t)(row < lim ? row : lim - 1) * (uint32_t)K + c * 16;
  }
  const int nkb = nk;
  const bool s_is_a = wave < 4;
  __amdgpu_buffer_rsrc_t rs = ra;
  uint32_t s_voff = 0;
  if constexpr (TENSOR) {
  } else if (s_is_a) {
    const uint64_t bytes = ((uint64_t)nkb * M - m0) * 4;
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sa_p + m0), (short)0,
                                           (int)(bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull), kBufferFlags);
    const int row = wave * 64 + lane;
    s_voff = (uint32_t)(row < lim_a ? row : lim_a - 1) * 4;
  } else if constexpr (MODE == MODE_BLOCK) {
    const uint64_t bytes = ((uint64_t)tiles_n * nkb - (uint64_t)tn * nkb) * 4;
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sb_p + (size_t)tn * nkb), (short)0,
                                           (int)(bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull), kBufferFlags);
    s_voff = 0;
  } else {
    // waves 4 and 5 load the tile's 128 column scales; 6 and 7 repeat them into unused slots
    const uint64_t bytes = ((uint64_t)nkb * N - n0) * 4;
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sb_p + n0), (short)0,
                                           (int)(bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull), kBufferFlags);
    const int col = (wave & 1) * 64 + lane;
    s_voff = (uint32_t)(col < lim_b ? col : lim_b - 1) * 4;
  }
  const int s_lds = s_is_a ? SA_OFF + wave * 256 : SB_OFF + (wave - 4) * 256;
  const uint32_t s_step = s_is_a ? (uint32_t)M * 4 : (MODE == MODE_BLOCK ? 4u : (uint32_t)N * 4);
  auto issue = [&](int ks, int st) {
    uint8_t* buf = smem + st * STAGE;
#pragma unroll
    for (int i = 0; i < OPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wave * OPW + i < 32 ? ra : rb, (lds_ptr_t)(buf + (wave * OPW + i) * 1024),
                                               16, od[i], ks * BLK_BK, 0, 0);
    if constexpr (!TENSOR)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(buf + s_lds), 4, s_voff, ks * s_step, 0, 0);
  };
  // wait until at most `later` stages of this wave's loads (OPW per stage, + 1 scale load
  // unless per tensor) are in flight
  auto wait_stage = [&](int later) {
    if (later >= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"i"(TENSOR ? OPW : OPW + 1) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // ---- per-lane LDS bases per stage (immediates add the tile offsets)
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int slab_a = grp * 128 + wr * 64, slab_b = wc * SW;
  uint32_t a_lo[NST], a_hi[NST], b_lo[NST], b_hi[NST], s_a[NST], s_b[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const uint32_t base = lds0 + st * STAGE;
    const int qa = slab_a + r, qb = slab_b + r;  // tile 0's rows; tile i adds 16 rows = 2048 B
    a_lo[st] = base + qa * 128 + (blk_pos(qa, g) << 4);
    a_hi[st] = base + qa * 128 + (blk_pos(qa, g + 4) << 4);
    b_lo[st] = base + BLK_B_OFF + qb * 128 + (blk_pos(qb, g) << 4);
    b_hi[st] = base + BLK_B_OFF + qb * 128 + (blk_pos(qb, g + 4) << 4);
    s_a[st] = base + SA_OFF + (slab_a + 16 * g) * 4;
    s_b[st] = base + SB_OFF + (MODE == MODE_TILE2 ? (slab_b + 4 * r) * 4 : 0);
  }

  v4f acc[4][Shape::NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  v8i fa[4], fb[Shape::NT];
  float fsa[16], fsb[4] = {0.f, 0.f, 0.f, 0.f};
  // the fold's scale factors for this K step: sa[row] * sb (block) in sc[0..15], or
  // sa[row] * sb[column j] in sc[16 j + e] for two 1x128 operands
  float sc[64];
  auto pack = [](const u32x4& lo, const u32x4& hi) -> v8i {
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto read_all = [&](auto st_c) {
    constexpr int ST = decltype(st_c)::value;
    // rows 16i + r of the slab: blk_pos depends on bits 0-3 of the row only, so tile i is the
    // same lane address + 16 rows of 128 B
    fa[0] = pack(ds_read16<0 * 2048>(a_lo[ST]), ds_read16<0 * 2048>(a_hi[ST]));
    fa[1] = pack(ds_read16<1 * 2048>(a_lo[ST]), ds_read16<1 * 2048>(a_hi[ST]));
    fa[2] = pack(ds_read16<2 * 2048>(a_lo[ST]), ds_read16<2 * 2048>(a_hi[ST]));
    fa[3] = pack(ds_read16<3 * 2048>(a_lo[ST]), ds_read16<3 * 2048>(a_hi[ST]));
    fb[0] = pack(ds_read16<0 * 2048>(b_lo[ST]), ds_read16<0 * 2048>(b_hi[ST]));
    fb[1] = pack(ds_read16<1 * 2048>(b_lo[ST]), ds_read16<1 * 2048>(b_hi[ST]));
    if constexpr (NT == 4) {
      fb[NT > 2 ? 2 : 0] = pack(ds_read16<2 * 2048>(b_lo[ST]), ds_read16<2 * 2048>(b_hi[ST]));
      fb[NT > 3 ? 3 : 0] = pack(ds_read16<3 * 2048>(b_lo[ST]), ds_read16<3 * 2048>(b_hi[ST]));
    }
    if constexpr (TENSOR) return;
    const u32x4 s0 = ds_read16<0>(s_a[ST]), s1 = ds_read16<16>(s_a[ST]), s2 = ds_read16<32>(s_a[ST]),
                s3 = ds_read16<48>(s_a[ST]);
    const u32x4 sv[4] = {s0, s1, s2, s3};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      fsa[4 * h + 0] = __uint_as_float(sv[h].x);
      fsa[4 * h + 1] = __uint_as_float(sv[h].y);
      fsa[4 * h + 2] = __uint_as_float(sv[h].z);
      fsa[4 * h + 3] = __uint_as_float(sv[h].w);
    }
    if constexpr (MODE == MODE_BLOCK) {
      fsb[0] = __uint_as_float(ds_read4<0>(s_b[ST]));
    } else {
      const u32x4 sbv = ds_read16<0>(s_b[ST]);  // columns 4r .. 4r+3 of the slab
      fsb[0] = __uint_as_float(sbv.x);
      fsb[1] = __uint_as_float(sbv.y);
      fsb[2] = __uint_as_float(sbv.z);
      fsb[3] = __uint_as_float(sbv.w);
    }
  };
  // 16 MFMAs, each partial folded into its accumulators four MFMAs later (at 4096 x 7168 x
  // 7168, folding one MFMA later was 25% slower and two MFMAs later 1.5%):
  // acc[i][j][jj] += p * (sa[row 16g + 4jj + i] * sb[block] or sb[column 4r + j])
  auto compute = [&]() {
    if constexpr (TENSOR) {
#pragma unroll
      for (int t = 0; t < 4 * NT; ++t) {
        acc[t / NT][t % NT] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[t / NT], fb[t % NT],
                                                                                acc[t / NT][t % NT], FA, FB, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    } else {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    constexpr int kFoldLag = 4;
    v4f p[16];
    auto fold = [&](int t) {
      const int i = t >> 2, j = t & 3;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        acc[i][j][jj] = fmaf(p[t][jj], sc[(MODE == MODE_BLOCK ? 0 : 16 * j) + 4 * jj + i], acc[i][j][jj]);
    };
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      p[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[t >> 2], fb[t & 3], zero, FA, FB, 0, 0, 0, 0);
      if (t >= kFoldLag) fold(t - kFoldLag);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 16 - kFoldLag; t < 16; ++t) fold(t);
    }
  };
  // the scale products, formed while the other wave group runs its MFMAs, so that the fold
  // in compute() is one FMA per accumulator
  auto prep = [&]() {
    if constexpr (MODE == MODE_BLOCK) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = fsa[e] * fsb[0];
    } else if constexpr (MODE == MODE_TILE2) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[16 * j + e] = fsa[e] * fsb[j];
    }
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // M_k then C_k for stage k in buffer ST = k % 3; the last barriers are dropped as in the
  // kernel above
  auto step = [&](auto steady, auto st_c, int k) {
    constexpr bool STEADY = decltype(steady)::value;
    constexpr int ST = decltype(st_c)::value;
    __builtin_amdgcn_sched_barrier(0);
    read_all(st_c);
    __builtin_amdgcn_sched_barrier(0);
    if (STEADY || k + D < nk) issue(k + D, (ST + D) % NST);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if constexpr (!TENSOR) {
      __builtin_amdgcn_sched_barrier(0);
      prep();
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (STEADY) {
      wait_stage(1);  // this wave's part of stage k+1
    } else {
      if (k + 1 < nk) wait_stage(nk - k - 2 < 1 ? nk - k - 2 : 1);
    }
    if (STEADY || !(grp == 1 && k + 1 == nk)) barrier();
    compute();
    __builtin_amdgcn_sched_barrier(0);
    if (STEADY || k + 1 < nk) barrier();
  };
  using steady_t = std::integral_constant<bool, true>;
  using tail_t = std::integral_constant<bool, false>;

  if (nk > 0) {
    issue(0, 0);
    if (nk > 1) issue(1, 1);
    wait_stage(nk > 1 ? 1 : 0);  // this wave's part of stage 0
    barrier();                   // stage 0 visible
    if (grp == 1) barrier();     // group 1 sits out slot 0
    int k = 0;
    for (; k + U + D <= nk; k += U)
      unroll_seq([&](auto i_c) {
        constexpr int I = decltype(i_c)::value;
        step(steady_t{}, std::integral_constant<int, I>{}, k + I);
      }, std::make_integer_sequence<int, U>{});
    for (; k < nk; k += U)
      unroll_seq([&](auto i_c) {
        constexpr int I = decltype(i_c)::value;
        if (k + I < nk) step(tail_t{}, std::integral_constant<int, I>{}, k + I);
      }, std::make_integer_sequence<int, U>{});
  }

  // ---- epilogue: acc[i][j][jj] is tile row slab + 16g + 4jj + i, column slab + NT r + j
  Epilogue<OUT, FUSED> epi(ep);
  float scale = 1.0f;
  if constexpr (TENSOR) scale = sa_p[0] * sb_p[0];
  const int gn = n0 + slab_b + NT * r;
  const bool quad = N % NT == 0 && gn + NT - 1 < N;  // all NT columns present, store aligned
  float b[Shape::NT];
  epi.template bias<Shape::NT>(gn, N, b);
  epi.with_act([&](auto act_c) {
    constexpr int ACT = decltype(act_c)::value;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gm = m0 + slab_a + 16 * g + 4 * jj + i;
        if (gm >= M) continue;
        float v[Shape::NT];
#pragma unroll
        for (int c = 0; c < NT; ++c) v[c] = acc[i][c][jj];
        if constexpr (TENSOR) {
#pragma unroll
          for (int c = 0; c < NT; ++c) v[c] *= scale;
        }
        epi.pre(v, b);
        epi.aux(v, gm, gn, N, quad);
        epi.template out<ACT>(v, gm, gn, N, quad);
      }
  });
  epi.finish(lane, reinterpret_cast<uint32_t*>(smem));
}

// per-tensor problems with fewer 256 x 128 tiles than this run on 256 x 64 tiles (at 200, the
// 144- and 192-tile GEMMs of the MiniGPT layer set moved too and its step got 5-7% slower)
constexpr int64_t kNarrowTiles = 128;

template <int MODE, int FA, int FB, int OUT, bool FUSED>
static int launch_gemm(const uint8_t* A, const uint8_t* B, const void* sa, const void* sb, const EpiParams& ep, int M,
                       int N, int K, hipStream_t st, const char* what) {
  if constexpr (MODE == MODE_TENSOR) {
    // fewer 256 x 256 tiles than CUs: the 256 x 128 tiles of the blockwise kernel keep twice
    // as many CUs busy (workload 2's per-tensor GEMMs 1.5x faster); from one full wave of
    // tiles on, the 256 x 256 kernel reads less per FLOP and wins
    const int64_t big_tiles = (int64_t)((M + BIG_BM - 1) / BIG_BM) * ((N + BIG_BN - 1) / BIG_BN);
    if (big_tiles < 256 && 256ll * K < (1ll << 32)) {
      const int tiles_m = (M + BLK_BM - 1) / BLK_BM, tiles_n = (N + BLK_BN - 1) / BLK_BN;
      if ((int64_t)tiles_m * tiles_n < kNarrowTiles) {
        // still a fraction of the CUs: 256 x 64 tiles double the count
        const int tiles_n64 = (N + 63) / 64;
        hipLaunchKernelGGL((gemm_blk_kernel<MODE, FA, FB, OUT, FUSED, 64>), dim3(tiles_m * tiles_n64), dim3(512), 0, st,
                           A, B, static_cast<const float*>(sa), static_cast<const float*>(sb), ep, M, N, K, tiles_m,
                           tiles_n64);
        return check_launch(what);
      }
      hipLaunchKernelGGL((gemm_blk_kernel<MODE, FA, FB, OUT, FUSED, BLK_BN>), dim3(tiles_m * tiles_n), dim3(512), 0, st, A, B,
                         static_cast<const float*>(sa), static_cast<const float*>(sb), ep, M, N, K, tiles_m, tiles_n);
      return check_launch(what);
    }
  }
  if constexpr (MODE == MODE_TENSOR || MODE == MODE_MX) {
    const int tiles_m = (M + BIG_BM - 1) / BIG_BM, tiles_n = (N + BIG_BN - 1) / BIG_BN;
    // every size it supports: even with a few tiles (e.g. 2048 x 2304 x 768, 72 tiles) it beats
    // the 128 x 128 kernel by 1.2-1.9x; MX scale rows are read as 4-byte runs, so M and N must be
    // multiples of 4 there
    if (M >= 4 && N >= 4 && (MODE != MODE_MX || (M % 4 == 0 && N % 4 == 0))) {
      // the large-tile kernel addresses a tile's rows and a stage's scale rows with 32-bit
      // offsets; beyond that the 128 x 128 kernel (64-bit addressing) takes the problem
      const int64_t mn = M > N ? M : N;
      const bool offsets32 = 256ll * K < (1ll << 32) && (MODE != MODE_MX || (int64_t)(K / 32) * mn < (1ll << 32));
      if (offsets32) {
        constexpr int NST = 4;  // 5 stages (per tensor, 160 KB) measured no faster
        hipLaunchKernelGGL((gemm_pp_kernel<MODE, FA, FB, OUT, FUSED, NST>), dim3(tiles_m * tiles_n), dim3(512), 0, st, A, B,
                           sa, sb, ep, M, N, K, tiles_m, tiles_n);
        return check_launch(what);
      }
    }
  }
  if constexpr (MODE == MODE_BLOCK || MODE == MODE_TILE2) {
    const int tiles_m = (M + BLK_BM - 1) / BLK_BM, tiles_n = (N + BLK_BN - 1) / BLK_BN;
    // every size (1.4-3.1x over the 128 x 128 kernel at workload 2's shapes); 32-bit offsets for
    // a tile's rows and a stage's scales
    const int64_t mn = M > N ? M : N;
    const bool offsets32 = 256ll * K < (1ll << 32) && (int64_t)(K / 128) * mn * 4 < (1ll << 32);
    if (offsets32) {
      hipLaunchKernelGGL((gemm_blk_kernel<MODE, FA, FB, OUT, FUSED, BLK_BN>), dim3(tiles_m * tiles_n), dim3(512), 0, st, A, B,
                         static_cast<const float*>(sa), static_cast<const float*>(sb), ep, M, N, K, tiles_m, tiles_n);
      return check_launch(what);
    }
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
