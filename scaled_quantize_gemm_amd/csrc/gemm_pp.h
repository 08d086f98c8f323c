// The 256 x 256 ping-pong FP8 GEMM kernel (per-tensor and MX scaling) and its launch.
#pragma once

#include "gemm_common.h"

namespace sfp8 {

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

constexpr int BIG_BM = 256, BIG_BN = 256, BIG_BK = 64;
constexpr int BIG_TILE_BYTES = (BIG_BM + BIG_BN) * BIG_BK;  // 32 KB
constexpr int BIG_SCALE_BYTES = 2 * (BIG_BM + BIG_BN);      // 1 KB (MX only)

__device__ __forceinline__ int bswz_pos(int row) { return ((row >> 2) ^ (row >> 1)) & 3; }
__device__ __forceinline__ int bswz(int row, int c) { return row * 64 + ((c ^ bswz_pos(row)) << 4); }

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

// launch over the tiles of C (per-tensor or MX); the caller has checked that the kernel
// applies (M, N >= 4; MX: multiples of 4; 32-bit row and scale offsets)
template <int MODE, int FA, int FB, int OUT, bool FUSED>
static int launch_pp(const uint8_t* A, const uint8_t* B, const void* sa, const void* sb, const EpiParams& ep, int M,
                     int N, int K, hipStream_t st, const char* what) {
  const int tiles_m = (M + BIG_BM - 1) / BIG_BM, tiles_n = (N + BIG_BN - 1) / BIG_BN;
  constexpr int NST = 4;  // 5 stages (per tensor, 160 KB) measured no faster
  hipLaunchKernelGGL((gemm_pp_kernel<MODE, FA, FB, OUT, FUSED, NST>), dim3(tiles_m * tiles_n), dim3(512), 0, st, A, B, sa,
                     sb, ep, M, N, K, tiles_m, tiles_n);
  return check_launch(what);
}

}  // namespace sfp8
