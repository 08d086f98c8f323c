// The 256 x 128 (and 256 x 64) ping-pong FP8 GEMM kernel (blockwise, 1x128 x 1x128 and small
// per-tensor problems) and its launch.
#pragma once

#include "gemm_common.h"

namespace sfp8 {

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
constexpr int BLK_NST = 3;

// the tile row (A) or output column (B) held at LDS row q of a slab of 16 nt rows or columns:
// MFMA tile j's row / column t at LDS row 16j + t is slab row / column nt t + j
__device__ __forceinline__ int blk_col_of(int q, int nt) {
  return (q & ~(16 * nt - 1)) + nt * (q & 15) + ((q >> 4) & (nt - 1));
}
// position of 16-byte chunk c in 128-byte LDS row q (the small-tile kernel's swizzle)
__device__ __forceinline__ int blk_pos(int q, int c) { return c ^ (((q >> 1) ^ ((q & 1) << 2)) & 7); }

// MODE: MODE_BLOCK (B scales per 128x128 block: one value per stage), MODE_TILE2 (B scales
// per 1x128 run along K: one per column per stage, [K/128][N]) or MODE_TENSOR (no scale loads;
// the MFMAs accumulate straight into acc and the epilogue multiplies by sa * sb: the 256 x 128
// tile gives small per-tensor problems twice the tiles of the 256 x 256 kernel)
// the tile-shape-dependent layout of the kernel below: TI MFMA row tiles and NT column tiles per
// wave slab of SH x SW; the A rows of a stage are BM x 128 B and the B rows BN x 128 B, loaded as
// NA + NB = NOPS 1 KB operations (OPW per wave).  BM = 128 (per-tensor only) halves the slab
// height: twice the tiles again for problems that leave most CUs idle.
template <int BM, int BN>
struct BlkShape {
  static constexpr int TI = BM / 64, SH = BM / 4, NT = BN / 32, SW = BN / 2;
  static constexpr int NA = BM / 8, NB = BN / 8, NOPS = NA + NB, OPW = NOPS / 8;
  static constexpr int B_OFF = BM * BLK_BK, SA_OFF = B_OFF + BN * BLK_BK, SB_OFF = SA_OFF + 1024,
                       STAGE = SB_OFF + 1024;
};

// Block b of a launch over the tiles of a tiles_m x tiles_n tiling in tile_of's order: on XCD
// b % 8, that XCD's tiles from index idx0 on, `sub` blocks per tile (part = which 1/sub of the
// tile's columns the block takes).  False where the XCD has no such tile.
__device__ __forceinline__ bool tile_part_of(int b, int tiles_m, int tiles_n, int idx0, int sub, int& tm, int& tn,
                                             int& part) {
  const int T = tiles_m * tiles_n, xcd = b & 7, j = b >> 3, idx = idx0 + j / sub;
  part = j - (j / sub) * sub;
  if (idx >= (T >> 3) + (xcd < (T & 7) ? 1 : 0)) return false;
  tile_of(8 * idx + xcd, tiles_m, tiles_n, tm, tn);
  return true;
}

template <int MODE, int FA, int FB, int OUT, bool FUSED, int BN, int BM>
__global__ void __launch_bounds__(512, 1) gemm_blk_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                          const float* __restrict__ sa_p,
                                                          const float* __restrict__ sb_p, const EpiParams ep, int M,
                                                          int N, int K, int tiles_m, int tiles_n, int idx0, int sub) {
  constexpr bool TENSOR = MODE == MODE_TENSOR;
  static_assert(BN == BLK_BN || BN == 64, "256 x 128 or 256 x 64 tiles");
  static_assert(BM == BLK_BM || (BM == 128 && TENSOR), "128-row tiles serve per-tensor scaling only");
  using Shape = BlkShape<BM, BN>;
  constexpr int TI = Shape::TI, SH = Shape::SH, NT = Shape::NT, SW = Shape::SW, NA = Shape::NA;
  constexpr int NOPS = Shape::NOPS, OPW = Shape::OPW;
  constexpr int B_OFF = Shape::B_OFF, SA_OFF = Shape::SA_OFF, SB_OFF = Shape::SB_OFF, STAGE = Shape::STAGE;
  constexpr int NST = BLK_NST, D = NST - 1, U = NST;
  static_assert(NOPS % 8 == 0, "every wave issues the same number of loads");
  static_assert(NST * STAGE <= 160 * 1024, "LDS ring must fit the 160 KB of a CU");
  __shared__ __attribute__((aligned(16))) uint8_t smem[BLK_NST * Shape::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wi = wave & 3, wr = wi >> 1, wc = wi & 1;
  const int g = lane >> 4, r = lane & 15;
  int tm, tn, part;
  if (!tile_part_of(blockIdx.x, tiles_m, tiles_n, idx0, sub, tm, tn, part)) return;
  const int m0 = tm * BM, n0 = (tn * sub + part) * BN;
  if (n0 >= N) return;  // the second half of a last tile column at most 64 wide
  const int nk = K / BLK_BK;

  // ---- loads: NOPS x 1 KB of tile data per stage, OPW per wave (ops 0..NA-1 are A, then B), and
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
    const int o = wave * OPW + i, local = o < NA ? o : o - NA;
    const int slot = local * 64 + lane, q = slot >> 3, c = blk_pos(q, slot & 7);
    const int row = o < NA ? blk_col_of(q, TI) : blk_col_of(q, NT), lim = o < NA ? lim_a : lim_b;
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
    // the tile lies in weight-block column n0 / 128 (its [K/128] scales are contiguous)
    const int bc = n0 >> 7, nbc = (N + 127) >> 7;
    const uint64_t bytes = (uint64_t)(nbc - bc) * nkb * 4;
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sb_p + (size_t)bc * nkb), (short)0,
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
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wave * OPW + i < NA ? ra : rb, (lds_ptr_t)(buf + (wave * OPW + i) * 1024),
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
  const int slab_a = grp * (2 * SH) + wr * SH, slab_b = wc * SW;
  uint32_t a_lo[NST], a_hi[NST], b_lo[NST], b_hi[NST], s_a[NST], s_b[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const uint32_t base = lds0 + st * STAGE;
    const int qa = slab_a + r, qb = slab_b + r;  // tile 0's rows; tile i adds 16 rows = 2048 B
    a_lo[st] = base + qa * 128 + (blk_pos(qa, g) << 4);
    a_hi[st] = base + qa * 128 + (blk_pos(qa, g + 4) << 4);
    b_lo[st] = base + B_OFF + qb * 128 + (blk_pos(qb, g) << 4);
    b_hi[st] = base + B_OFF + qb * 128 + (blk_pos(qb, g + 4) << 4);
    s_a[st] = base + SA_OFF + (slab_a + 16 * g) * 4;
    s_b[st] = base + SB_OFF + (MODE == MODE_TILE2 ? (slab_b + NT * r) * 4 : 0);
  }

  v4f acc[Shape::TI][Shape::NT];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  v8i fa[Shape::TI], fb[Shape::NT];
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
    if constexpr (TI == 4) {
      fa[TI > 2 ? 2 : 0] = pack(ds_read16<2 * 2048>(a_lo[ST]), ds_read16<2 * 2048>(a_hi[ST]));
      fa[TI > 3 ? 3 : 0] = pack(ds_read16<3 * 2048>(a_lo[ST]), ds_read16<3 * 2048>(a_hi[ST]));
    }
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
      // columns NT r .. NT r + NT - 1 of the slab (NT = 2: the first two of the four read)
      const u32x4 sbv = ds_read16<0>(s_b[ST]);
      fsb[0] = __uint_as_float(sbv.x);
      fsb[1] = __uint_as_float(sbv.y);
      fsb[2] = __uint_as_float(sbv.z);
      fsb[3] = __uint_as_float(sbv.w);
    }
  };
  // TI x NT MFMAs (16, or 8 on 64-wide tiles), each partial folded into its accumulators four
  // MFMAs later (at 4096 x 7168 x 7168, folding one MFMA later was 25% slower and two MFMAs
  // later 1.5%): acc[i][j][jj] += p * (sa[row 16g + 4jj + i] * sb[block] or sb[column NT r + j])
  auto compute = [&]() {
    if constexpr (TENSOR) {
#pragma unroll
      for (int t = 0; t < TI * NT; ++t) {
        acc[t / NT][t % NT] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[t / NT], fb[t % NT],
                                                                                acc[t / NT][t % NT], FA, FB, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    } else {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    constexpr int kFoldLag = 4, NM = TI * NT;
    v4f p[NM];
    auto fold = [&](int t) {
      const int i = t / NT, j = t % NT;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        acc[i][j][jj] = fmaf(p[t][jj], sc[(MODE == MODE_BLOCK ? 0 : 16 * j) + 4 * jj + i], acc[i][j][jj]);
    };
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      p[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[t / NT], fb[t % NT], zero, FA, FB, 0, 0, 0, 0);
      if (t >= kFoldLag) fold(t - kFoldLag);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = NM - kFoldLag; t < NM; ++t) fold(t);
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
      for (int j = 0; j < NT; ++j)
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

  // ---- epilogue: acc[i][j][jj] is tile row slab + TI (4g + jj) + i, column slab + NT r + j
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
      for (int i = 0; i < TI; ++i) {
        const int gm = m0 + slab_a + TI * (4 * g + jj) + i;
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

// launch over BM x BN tiles of C; the caller has checked the 32-bit offsets.
// A 256 x 128 tiling whose last round of tiles would leave at least three quarters of an XCD's
// 32 CUs idle (tile_of gives each XCD a contiguous run of tiles, which its CUs take 32 at a
// time, one block per CU) runs as two launches: the whole rounds, then what is left of each
// XCD's run as twice as many 256 x 64 tiles, which take less than a whole tile's time each
// (workload 3's wgrad, 7168 x 7168 x 4096 with 4 tiles per XCD left: 256 -> 243 us).  With
// half the CUs left busy the halves gained nothing (its forward, 16 tiles per XCD left:
// 215 -> 220 us), so that case keeps the 256 x 128 tiles.
template <int MODE, int FA, int FB, int OUT, bool FUSED, int BN, int BM = BLK_BM>
static int launch_blk(const uint8_t* A, const uint8_t* B, const void* sa, const void* sb, const EpiParams& ep, int M,
                      int N, int K, hipStream_t st, const char* what) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const float* fa = static_cast<const float*>(sa);
  const float* fb = static_cast<const float*>(sb);
  if constexpr (BN == BLK_BN && BM == BLK_BM) {
    constexpr int kXcdCus = 32;
    const int T = tiles_m * tiles_n, per = T >> 3;
    const int whole = per / kXcdCus * kXcdCus;                // tile indices every XCD runs in whole rounds
    const int left = per - whole + ((T & 7) != 0 ? 1 : 0);  // at most this many tiles per XCD after them
    if (whole > 0 && left > 0 && 4 * left <= kXcdCus) {
      hipLaunchKernelGGL((gemm_blk_kernel<MODE, FA, FB, OUT, FUSED, BN, BM>), dim3(8 * whole), dim3(512), 0, st, A, B,
                         fa, fb, ep, M, N, K, tiles_m, tiles_n, 0, 1);
      const int rc = check_launch(what);
      if (rc != FP8_OK) return rc;
      hipLaunchKernelGGL((gemm_blk_kernel<MODE, FA, FB, OUT, FUSED, 64, BM>), dim3(8 * 2 * left), dim3(512), 0, st, A,
                         B, fa, fb, ep, M, N, K, tiles_m, tiles_n, whole, 2);
      return check_launch(what);
    }
  }
  hipLaunchKernelGGL((gemm_blk_kernel<MODE, FA, FB, OUT, FUSED, BN, BM>), dim3(tiles_m * tiles_n), dim3(512), 0, st, A, B,
                     fa, fb, ep, M, N, K, tiles_m, tiles_n, 0, 1);
  return check_launch(what);
}

}  // namespace sfp8
