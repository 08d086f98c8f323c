// The 256 x 256 FP8 GEMM kernel with one wave per SIMD (per-tensor and MX scaling) and its
// launch.
#pragma once

#include "gemm_common.h"

namespace sfp8 {

// 256 x 256 block tile, 4 waves, one per SIMD.  Wave w computes the 128 x 128 quarter
// (w / 2, w % 2) of the tile: 4 x 4 MFMAs of 32x32x64 per 64-deep K step into 256 fp32
// accumulators per lane, which live in the accumulation registers.
//
// Why this shape, on gfx950:
//  - the operand bytes a wave reads from LDS per MFMA shrink as its tile grows: a 128 x 128
//    wave tile reads 16 KB per 16 MFMAs (a 128 x 64 one, two waves per SIMD, 12 KB per 8);
//  - a direct-to-LDS load that takes 64 bytes from each of 16 rows moves half as many bytes
//    per cycle as one that takes whole 128-byte rows from 8 (29 vs 58 B/clk per CU,
//    measured), so a stage holds K = 128: whole cache lines;
//  - two such stages (128 KB of the 160 KB LDS) are the ring.  A stage is read into
//    registers in a single step (three register sets of fragments), which frees its buffer a
//    step early: the loads of a stage then have about three steps to land.
//
// Stage j (K = 128j .. 128j+127, buffer j % 2) feeds MFMA steps 2j and 2j+1; step s uses
// fragment set s % 3.
//   even step 2j: its first kW4Lead MFMAs; wait for this wave's reads of stage j, then a
//     barrier (every wave has read stage j into registers, so its buffer is free); the
//     remaining MFMAs with the first half of stage j+2's loads between them;
//   odd step 2j+1: its first kW4Lead MFMAs; wait for this wave's loads of stage j+1, then a
//     barrier (stage j+1 complete for every wave); the remaining MFMAs with stage j+1's
//     fragment reads (for steps 2j+2, then 2j+3) and the second half of stage j+2's loads
//     between them; wait for the reads of step 2j+2's fragments (those of step 2j+3 issued
//     last may stay in flight into the next step).
// The MFMAs queued before a barrier keep the matrix core busy while the waves meet there.
//
// LDS: A of stages 0 and 1 at 0 and 32 KB, B's at 64 and 96 KB (so that one base register
// reaches both stages of an operand through the 16-bit offset field), then (MX) each stage's
// e8m0 scales: A's 4 K-blocks x 256 rows, then B's.  A row holds 128 bytes; its 16-byte chunk
// c sits at position c ^ f(row), f(row) = ((row >> 1) ^ ((row & 1) << 2)) & 7, so that the 16
// rows one 128-bit read phase touches (and any 8 consecutive ones) cover distinct banks.
// Row interleave: MFMA tile i of a wave holds tile rows 128p + 4t + i (t = 0..31, the MFMA
// row) and sits at LDS rows 128p + 32i + t, so that a lane's four A scales (rows 4t..4t+3)
// are adjacent bytes, read at once, the byte picked by the MFMA's scale selector; B's columns
// likewise.  In the epilogue a lane then holds 4 adjacent columns of a row and writes them
// with one store.

constexpr int W4_BM = 256, W4_BN = 256, W4_BK = 128;
constexpr int W4_A = 0, W4_B = 65536, W4_S = 131072;  // LDS regions
constexpr int W4_OPER_STAGE = 32768;                   // one operand's stage
constexpr int W4_SCALE_STAGE = 2048;                   // MX: A, B x 4 K-blocks x 256 rows
// MFMAs of a step issued before its barrier
constexpr int kW4Lead = 2;
// an even step's loads go between MFMAs kW4Lead .. kW4Last; an odd step's reads and loads
// between MFMAs kW4Lead .. 15, the reads for the next step first, so that the wait closing the
// step leaves the reads issued after MFMA kW4Last (for the step after next) in flight
constexpr int kW4Last = 13;

__device__ __forceinline__ int w4_swz(int row) { return ((row >> 1) ^ ((row & 1) << 2)) & 7; }

template <int MODE, int FA, int FB, int OUT, bool FUSED>
__global__ void __launch_bounds__(256, 1) gemm_w4_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                         const void* __restrict__ sa_p, const void* __restrict__ sb_p,
                                                         const EpiParams ep, int M, int N, int K, int tiles_m,
                                                         int tiles_n) {
  constexpr bool MX = MODE == MODE_MX;
  constexpr int HALF = MX ? 9 : 8;     // loads per wave per step: half a stage
  constexpr int NREAD = MX ? 36 : 32;  // LDS reads per wave per stage
  constexpr int SMEM = W4_S + (MX ? 2 * W4_SCALE_STAGE : 0);
  static_assert(SMEM <= 160 * 1024, "LDS must fit the 160 KB of a CU");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5, r = lane & 31;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * W4_BM, n0 = tn * W4_BN;
  const int ns = K / W4_BK;  // stages; MFMA steps 2 ns

  // ---- loads: waves 0, 1 fill A's rows 0-127 / 128-255, waves 2, 3 B's; load u (0..15) of a
  //      stage covers LDS rows 8u .. 8u+7 of the wave's 128 (lane L: row 8u + L/8, position
  //      L%8), through a buffer resource (uniform base, 32-bit lane offsets, range = the rows
  //      present); rows past the matrix edge re-read its last row
  const bool isb = wave >= 2;
  const int half = wave & 1;
  const int lim = isb ? N - n0 : M - m0;
  const uint8_t* d_base = isb ? B + (size_t)n0 * K : A + (size_t)m0 * K;
  const uint64_t d_bytes = (uint64_t)lim * (uint64_t)K;
  const __amdgpu_buffer_rsrc_t d_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(d_base), (short)0, (int)(d_bytes < 0xFFFFFFFFull ? d_bytes : 0xFFFFFFFFull), kBufferFlags);
  const int d_lds = (isb ? W4_B : W4_A) + half * 128 * W4_BK;
  // LDS row q = 128 half + 8u + L/8 holds tile row 128 half + 32 (u % 4) + 4 (L/8) + u/4; the
  // swizzle depends on q % 16 = 8 (u % 2) + L/8
  const int lrow = 4 * (lane >> 3);
  const uint32_t c_even = ((lane & 7) ^ w4_swz(lane >> 3)) * 16, c_odd = ((lane & 7) ^ w4_swz(8 + (lane >> 3))) * 16;
  // MX scales: wave w loads K-blocks 2 (w%2) and 2 (w%2) + 1 of each stage for A (w < 2) or B
  __amdgpu_buffer_rsrc_t s_rsrc = d_rsrc;  // replaced below (MX)
  uint32_t os = 0;
  int s_lim = 0;
  if constexpr (MX) {
    s_lim = isb ? N : M;
    const int base_row = isb ? n0 : m0;
    const uint8_t* s_base = static_cast<const uint8_t*>(isb ? sb_p : sa_p) + base_row;
    const uint64_t s_bytes = (uint64_t)(K / 32) * s_lim - base_row;
    s_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(s_base), (short)0,
                                               (int)(s_bytes < 0xFFFFFFFFull ? s_bytes : 0xFFFFFFFFull), kBufferFlags);
    const int rel = lane * 4, room = s_lim - 4 - base_row;  // M, N multiples of 4 here
    os = (uint32_t)(2 * half * s_lim + (rel < room ? rel : room));
  }
  // load u (0 .. 2 HALF - 1) of stage js into buffer BUF: data loads 0..15, then (MX) 2 scale loads
  auto load = [&](auto u_c, auto buf_c, int js) {
    constexpr int U = decltype(u_c)::value, BUF = decltype(buf_c)::value;
    if constexpr (U < 16) {
      const int row = half * 128 + 32 * (U & 3) + (U >> 2) + lrow;
      const int rr = row < lim ? row : lim - 1;
      const uint32_t off = (uint32_t)rr * (uint32_t)K + ((U & 1) ? c_odd : c_even);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          d_rsrc, (lds_ptr_t)(smem + d_lds + BUF * W4_OPER_STAGE + U * 1024), 16, off, js * W4_BK, 0, 0);
    } else {
      constexpr int T = U - 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          s_rsrc, (lds_ptr_t)(smem + W4_S + BUF * W4_SCALE_STAGE + ((isb ? 4 : 0) + 2 * half + T) * 256), 4,
          os + T * s_lim, 4 * js * s_lim, 0, 0);
    }
  };
  // the first or second half of a stage's loads: data loads 0..7 (+ scale load 0), or 8..15 (+ 1)
  auto load_half = [&](auto h_c, auto x_c, auto buf_c, int js) {
    constexpr int H = decltype(h_c)::value, X = decltype(x_c)::value;
    if constexpr (X < 8) load(std::integral_constant<int, 8 * H + X>{}, buf_c, js);
    else load(std::integral_constant<int, 16 + H>{}, buf_c, js);
  };
  // wait until at most `halves` half-stages of this wave's loads are in flight (they retire in order)
  auto wait_loads = [&](int halves) {
    if (halves >= 2) {
      if constexpr (MX) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    } else if (halves == 1) {
      if constexpr (MX) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };

  // ---- per-lane LDS read addresses: fragment half d (K bytes 16g.. / 32+16g..) of MFMA step h
  //      of a stage reads chunk 4h + 2d + g of row 32i + r; stage, tile and step-in-stage
  //      offsets go in the offset field
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  uint32_t ad[2][2], bd[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t lp = r * W4_BK + (((4 * h + 2 * d + g) ^ w4_swz(r)) << 4);
      ad[h][d] = lds0 + W4_A + wm * 128 * W4_BK + lp;
      bd[h][d] = lds0 + W4_B + wn * 128 * W4_BK + lp;
    }
  const uint32_t sad = lds0 + W4_S + g * 256 + wm * 128 + 4 * r;
  const uint32_t sbd = lds0 + W4_S + 1024 + g * 256 + wn * 128 + 4 * r;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // three fragment sets; fsa / fsb pack the e8m0 bytes of tiles i = 0..3 / j = 0..3
  u32x4 ra[3][8], rb[3][8];
  int fsa[3] = {0, 0, 0}, fsb[3] = {0, 0, 0};
  // read n (0 .. NREAD-1) of the stage in buffer BUF: for MFMA step h = n / (NREAD/2) of the
  // stage into set SET0 (h = 0) or SET1: A's 8 halves, B's 8, then (MX) A's and B's scales
  auto read = [&](auto n_c, auto buf_c, auto set0_c, auto set1_c) {
    constexpr int n = decltype(n_c)::value, BUF = decltype(buf_c)::value;
    constexpr int H = n / (NREAD / 2), m = n % (NREAD / 2);
    constexpr int SET = H == 0 ? decltype(set0_c)::value : decltype(set1_c)::value;
    if constexpr (m < 8) {
      constexpr int O = BUF * W4_OPER_STAGE + (m / 2) * 32 * W4_BK;
      ra[SET][m] = ds_read16<O>(ad[H][m & 1]);
    } else if constexpr (m < 16) {
      constexpr int O = BUF * W4_OPER_STAGE + ((m - 8) / 2) * 32 * W4_BK;
      rb[SET][m - 8] = ds_read16<O>(bd[H][m & 1]);
    } else if constexpr (m == 16) {
      fsa[SET] = (int)ds_read4<BUF * W4_SCALE_STAGE + H * 512>(sad);
    } else {
      fsb[SET] = (int)ds_read4<BUF * W4_SCALE_STAGE + H * 512>(sbd);
    }
  };
  auto frag = [](const u32x4& lo, const u32x4& hi) -> v8i {
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto mfma = [&](auto n_c, auto set_c) {
    constexpr int n = decltype(n_c)::value, I = n / 4, J = n % 4, SET = decltype(set_c)::value;
    acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        frag(ra[SET][2 * I], ra[SET][2 * I + 1]), frag(rb[SET][2 * J], rb[SET][2 * J + 1]), acc[I][J], FA, FB,
        MX ? I : 0, fsa[SET], MX ? J : 0, fsb[SET]);
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // MFMA step s = 2j + PAR (stage j in buffer BUF = j % 2, fragment set SET = s % 3).  STEADY
  // steps (stage j+2 exists) test nothing at run time.
  auto step = [&](auto steady, auto par_c, auto buf_c, auto set_c, int j) {
    constexpr bool STEADY = decltype(steady)::value;
    constexpr int PAR = decltype(par_c)::value, BUF = decltype(buf_c)::value, SET = decltype(set_c)::value;
    using OtherBuf = std::integral_constant<int, BUF ^ 1>;
    using Set1 = std::integral_constant<int, (SET + 1) % 3>;
    using Set2 = std::integral_constant<int, (SET + 2) % 3>;
    const bool ahead = STEADY || j + 2 < ns;           // stage j+2 exists: load its half
    const bool more = PAR == 1 && (STEADY || j + 1 < ns);  // odd step: stage j+1 exists, read it
    // ops between MFMAs: the even step's HALF loads; the odd step's NREAD reads with a load
    // after every fourth read
    constexpr int NOPS = PAR == 0 ? HALF : NREAD + HALF;
    constexpr int LAST = PAR == 0 ? kW4Last : 15;
    constexpr int SPAN = LAST - kW4Lead + 1;
    // reads issued after MFMA kW4Last (odd steps): left in flight by the closing wait
    constexpr int TAIL_FIRST = (kW4Last + 1 - kW4Lead) * NOPS / SPAN;
    constexpr int TAIL_READS = PAR == 0 ? 0 : (NOPS - TAIL_FIRST) - (NOPS / 5 - TAIL_FIRST / 5);
    static_assert(PAR == 0 || TAIL_FIRST - TAIL_FIRST / 5 >= NREAD / 2,
                  "the next step's reads must all precede the ones left in flight");
    static_assert(TAIL_READS <= 15, "lgkmcnt counts at most 15");
    auto op = [&](auto o_c) {
      constexpr int o = decltype(o_c)::value;
      if constexpr (PAR == 0) {
        if (ahead) load_half(std::integral_constant<int, 0>{}, o_c, buf_c, j + 2);
      } else if constexpr (o % 5 == 4) {
        if (ahead) load_half(std::integral_constant<int, 1>{}, std::integral_constant<int, o / 5>{}, buf_c, j + 2);
      } else {
        if (more) read(std::integral_constant<int, o - o / 5>{}, OtherBuf{}, Set1{}, Set2{});
      }
    };
    unroll_seq([&](auto n_c) {
      constexpr int n = decltype(n_c)::value;
      __builtin_amdgcn_sched_barrier(0);
      mfma(n_c, set_c);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (n == kW4Lead - 1) {
        if constexpr (PAR == 0) {
          if (ahead) {
            // the reads of stage j the previous step left in flight are done (in every wave,
            // by the barrier) before its buffer is refilled
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            barrier();
          }
        } else {
          if (more) {
            if constexpr (STEADY) wait_loads(1);
            else wait_loads(ahead ? 1 : 0);
            barrier();
          }
        }
      }
      if constexpr (n >= kW4Lead && n <= LAST) {
        constexpr int lo = (n - kW4Lead) * NOPS / SPAN, hi = (n - kW4Lead + 1) * NOPS / SPAN;
        unroll_seq([&](auto x_c) { op(std::integral_constant<int, lo + decltype(x_c)::value>{}); },
                   std::make_integer_sequence<int, hi - lo>{});
      }
    }, std::make_integer_sequence<int, 16>{});
    __builtin_amdgcn_sched_barrier(0);
    // odd step: the next step's fragments in registers; even step: the current step's reads
    // of the fragments for the next one (issued in the previous step) too
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(TAIL_READS) : "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  using steady_t = std::integral_constant<bool, true>;
  using tail_t = std::integral_constant<bool, false>;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  constexpr int U = 12;  // unroll in steps: parity, buffer (s/2 % 2) and set (s % 3) all repeat

  if (ns > 0) {
    unroll_seq([&](auto u_c) { load(u_c, I0{}, 0); }, std::make_integer_sequence<int, 2 * HALF>{});
    if (ns > 1) unroll_seq([&](auto u_c) { load(u_c, I1{}, 1); }, std::make_integer_sequence<int, 2 * HALF>{});
    wait_loads(ns > 1 ? 2 : 0);  // this wave's part of stage 0
    barrier();                   // stage 0 complete
    unroll_seq([&](auto n_c) { read(n_c, I0{}, I0{}, I1{}); }, std::make_integer_sequence<int, NREAD>{});
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int nk = 2 * ns;
    int s = 0;
    for (; s + U + 4 <= nk; s += U)  // every step of the block has stage j+2 to load
      unroll_seq([&](auto i_c) {
        constexpr int I = decltype(i_c)::value;
        step(steady_t{}, std::integral_constant<int, I % 2>{}, std::integral_constant<int, (I / 2) % 2>{},
             std::integral_constant<int, I % 3>{}, (s + I) / 2);
      }, std::make_integer_sequence<int, U>{});
    for (; s < nk; s += U)
      unroll_seq([&](auto i_c) {
        constexpr int I = decltype(i_c)::value;
        if (s + I < nk)
          step(tail_t{}, std::integral_constant<int, I % 2>{}, std::integral_constant<int, (I / 2) % 2>{},
               std::integral_constant<int, I % 3>{}, (s + I) / 2);
      }, std::make_integer_sequence<int, U>{});
  }

  // ---- epilogue: result register e of tile (i, j) is tile row 128 wm + 4(8(e/4) + 4g + e%4) + i,
  //      column 128 wn + 4r + j: each lane writes runs of 4 columns.  The stores are
  //      nontemporal: C goes on to HBM while other tiles still compute, instead of staying
  //      dirty in the caches for whatever kernel runs next to write back.
  Epilogue<OUT, FUSED> epi(ep);
  float scale = 1.0f;
  if constexpr (MODE == MODE_TENSOR) scale = *static_cast<const float*>(sa_p) * *static_cast<const float*>(sb_p);
  const int gn = n0 + wn * 128 + 4 * r;
  float b[4];
  epi.template bias<4>(gn, N, b);
  // one wave per SIMD leaves no other wave to hide the epilogue's latencies, so a tile that
  // lies wholly inside C (all but the edge tiles) stores every run without the per-row and
  // per-column tests (the branch is uniform; the 4 values are read before it)
  const bool interior = m0 + W4_BM <= M && n0 + W4_BN <= N && (N & 3) == 0;
  const bool full = (N & 3) == 0 && gn + 3 < N;  // all 4 columns present, the run's store aligned
  epi.with_act([&](auto act_c) {
    constexpr int ACT = decltype(act_c)::value;
#pragma unroll
    for (int e = 0; e < 16; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gm = m0 + wm * 128 + 4 * (8 * (e >> 2) + 4 * g + (e & 3)) + i;
        float v[4] = {acc[i][0][e], acc[i][1][e], acc[i][2][e], acc[i][3][e]};
        if constexpr (MODE == MODE_TENSOR) {
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] *= scale;
        }
        epi.pre(v, b);
        if (interior) {
          epi.aux(v, gm, gn, N, true);
          epi.template out<ACT>(v, gm, gn, N, true);
        } else if (gm < M && gn < N) {
          epi.aux(v, gm, gn, N, full);
          epi.template out<ACT>(v, gm, gn, N, full);
        }
      }
  });
  epi.finish(lane, reinterpret_cast<uint32_t*>(smem));
}

// launch over the tiles of C (per-tensor or MX); the caller has checked that the kernel
// applies (M, N >= 4; MX: multiples of 4; 32-bit row and scale offsets)
template <int MODE, int FA, int FB, int OUT, bool FUSED>
static int launch_w4(const uint8_t* A, const uint8_t* B, const void* sa, const void* sb, const EpiParams& ep, int M,
                     int N, int K, hipStream_t st, const char* what) {
  const int tiles_m = (M + W4_BM - 1) / W4_BM, tiles_n = (N + W4_BN - 1) / W4_BN;
  hipLaunchKernelGGL((gemm_w4_kernel<MODE, FA, FB, OUT, FUSED>), dim3(tiles_m * tiles_n), dim3(256), 0, st, A, B, sa,
                     sb, ep, M, N, K, tiles_m, tiles_n);
  return check_launch(what);
}

}  // namespace sfp8
