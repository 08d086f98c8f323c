// Per-tensor FP8 cast and its transpose in one pass (+ amax).
//
// The hybrid recipe's backward pass ("Transformer Scaling" lesson, Part 01: E4M3 forward,
// wider-range E5M2 gradients; "Week 14" course page, FP8 bullet) multiplies by transposed
// operands.  Writing the transposed FP8 copy during the cast keeps every GEMM in the
// K-contiguous form without a second read of the high-precision tensor.
//
// Shapes whose sides are multiples of 128 take the 128 x 128 kernel below (its per-tensor mode);
// the others this one.  Tile 64 x 64, 256 threads, one block per tile (the loop below also
// serves a capped grid):
//   phase 1: thread (row r, 8-column chunk) loads 8 elements of rows r and r+32, casts them,
//            stores the 8 codes to q and to an LDS tile (dword pitch 17 to spread banks);
//   phase 2: thread (4-column group, 4-row group) reads 4 dwords (4 rows x 4 columns),
//            transposes the 4x4 bytes in registers with v_perm_b32 and stores one dword
//            (4 consecutive source rows) to each of 4 rows of qT; 16 lanes cover 64
//            contiguous bytes of a qT row.
// Tiles that are partial or whose rows are not 16-byte aligned take an element-wise path.
#include <algorithm>

#include "quant_rules.h"

namespace sfp8 {

constexpr int kCtTile = 64;
constexpr int kCtPitch = 17;  // dwords per LDS row (16 + 1 pad)

template <bool BF16>
__device__ __forceinline__ float ld1(const void* __restrict__ base, int64_t i) {
  if constexpr (BF16) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[i] << 16);
  else return static_cast<const float*>(base)[i];
}

template <int FMT, bool BF16>
__global__ void __launch_bounds__(256) cast_transpose_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                             const float* __restrict__ scale_p,
                                                             uint32_t* __restrict__ amax_slot, uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ qT) {
  __shared__ uint32_t lds[kCtTile * kCtPitch];
  __shared__ uint32_t red[4];
  const float s = *scale_p;
  const int t = threadIdx.x;
  const int64_t tiles_c = (cols + kCtTile - 1) / kCtTile;
  const int64_t ntiles = ((rows + kCtTile - 1) / kCtTile) * tiles_c;
  const bool aligned_rows = (cols % 8 == 0) && (rows % 4 == 0);
  uint32_t mx = 0;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t r0 = (tile / tiles_c) * kCtTile, c0 = (tile % tiles_c) * kCtTile;
    const bool full = aligned_rows && r0 + kCtTile <= rows && c0 + kCtTile <= cols;
    if (full) {
      const int cg = t & 7, rr = t >> 3;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = rr + 32 * h;
        const int64_t e0 = (r0 + r) * cols + c0 + cg * 8;
        float v[8];
        load8<BF16>(x, e0, v);
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t a = abs_bits(v[i]);
          m = m > a ? m : a;
        }
        uint32_t w0 = cvt4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
        uint32_t w1 = cvt4<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
        if (m > 0x7F800000u) {
          w0 = patch_nan4(w0, &v[0]);
          w1 = patch_nan4(w1, &v[4]);
        }
        mx = mx > m ? mx : m;
        *reinterpret_cast<uint2*>(q + e0) = make_uint2(w0, w1);
        lds[r * kCtPitch + cg * 2] = w0;
        lds[r * kCtPitch + cg * 2 + 1] = w1;
      }
      __syncthreads();
      const int g4 = t >> 4, rc = t & 15;  // 4-column group, 4-row group
      uint32_t d0 = lds[(4 * rc + 0) * kCtPitch + g4];
      uint32_t d1 = lds[(4 * rc + 1) * kCtPitch + g4];
      uint32_t d2 = lds[(4 * rc + 2) * kCtPitch + g4];
      uint32_t d3 = lds[(4 * rc + 3) * kCtPitch + g4];
      // 4x4 byte transpose: out_j byte i = d_i byte j
      uint32_t lo01 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);
      uint32_t hi01 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);
      uint32_t lo23 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
      uint32_t hi23 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
      uint32_t o[4];
      o[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
      o[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
      o[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
      o[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(qT + (c0 + 4 * g4 + j) * rows + r0 + 4 * rc) = o[j];
      __syncthreads();  // the LDS tile is rewritten by the next tile
    } else {
      for (int e = t; e < kCtTile * kCtTile; e += 256) {
        const int64_t r = r0 + (e >> 6), c = c0 + (e & 63);
        if (r < rows && c < cols) {
          float xv = ld1<BF16>(x, r * cols + c);
          uint32_t w = cvt_pair<FMT, false>(xv * s, 0.0f, 0u) & 0xFFu;
          uint32_t b = __float_as_uint(xv);
          uint32_t a = b & 0x7FFFFFFFu;
          if (a > 0x7F800000u) w = nan_code(b);
          mx = mx > a ? mx : a;
          q[r * cols + c] = (uint8_t)w;
          qT[c * rows + r] = (uint8_t)w;
        }
      }
    }
  }
  uint32_t r = wave_max_u32(mx);
  if ((t & 63) == 0) red[t >> 6] = r;
  __syncthreads();
  if (t == 0 && amax_slot != nullptr) {
    uint32_t b = red[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) b = b > red[i] ? b : red[i];
    if (b > __hip_atomic_load(amax_slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(amax_slot, b);
  }
}


// ------------------------------------------------------------------ blockwise cast-transpose
//
// The blockwise recipe's backward pass needs the transposed operands with their own scales
// (DeepSeek-V3's blocks, per the course page's absmax bullet): for dgrad, W^T with the same
// 128x128 blocks (transposed); for wgrad, X^T and dY^T with 1x128 runs along the new K (the
// source's rows).  One 512-thread block per 128 x 128 source tile reads it once and writes
// both copies:
//   TILE:  q  uses one scale per source row run of 128 (scale_inv [cols/128][rows]),
//          qT uses one scale per source column run of 128 (its rows; [rows/128][cols]);
//   BLOCK: one scale for the tile in both (scale_inv [rows/128][cols/128] and, for qT, the
//          transposed [cols/128][rows/128]).
// Thread t holds source rows t/16 + 32p (p = 0..3), columns 8(t%16)..+8: row amaxes reduce
// over 16 lanes, column amaxes over the wave's four 16-lane groups and then the 8 waves in
// LDS.  The qT codes go through an LDS tile (dword pitch 33) and leave with 4x4 byte
// transposes, 128 contiguous bytes of a qT row per 32 lanes.

constexpr int kBwPitch = 33;

// KIND: kBwTile (1x128 runs), kBwBlock (128x128 blocks) or kBwTensor (the caller's per-tensor
// scale for both copies, the tensor's amax max-reduced into amax_slot: the per-tensor
// cast-transpose of 128-aligned shapes, whose 128-byte row pieces of q and qT are whole cache
// lines where the 64 x 64 kernel writes half lines)
constexpr int kBwTile = 1, kBwBlock = 2, kBwTensor = 0;
// the kernel's static LDS (qT code tile, column-amax partials, column scales) and the dynamic
// padding that holds the per-tensor launch at 3 resident blocks of the CU's 160 KB
constexpr size_t kBwStaticLds = 128 * kBwPitch * 4 + 8 * 128 * 4 + 128 * 4;
constexpr size_t kCtTensorLdsPad = 20 * 1024;
static_assert(3 * (kBwStaticLds + kCtTensorLdsPad) <= 160 * 1024 && 4 * (kBwStaticLds + kCtTensorLdsPad) > 160 * 1024,
              "the LDS padding must leave room for exactly 3 blocks per CU");

template <int FMT, bool BF16, int KIND>
__global__ void __launch_bounds__(512) cast_transpose_bw_kernel(const void* __restrict__ x, int64_t rows,
                                                                int64_t cols, uint8_t* __restrict__ q,
                                                                float* __restrict__ q_sinv, uint8_t* __restrict__ qT,
                                                                float* __restrict__ qT_sinv,
                                                                const float* __restrict__ scale_p,
                                                                uint32_t* __restrict__ amax_slot) {
  constexpr bool TILE = KIND == kBwTile;
  __shared__ uint32_t lds[128 * kBwPitch];
  __shared__ uint32_t cred[8][128];
  __shared__ float cscale[128];
  const int64_t nkb = cols >> 7, nrb = rows >> 7, ntiles = nkb * nrb;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r16 = t >> 4, cg = t & 15;
  uint32_t amax_acc = 0;  // per tensor: this thread's |x| bits max over its tiles
  // tile order.  Blockwise modes: row-band major (a band's blocks read whole source rows).
  // Per tensor: bands of 8 tile rows walked column by column, so that the blocks in flight
  // together write 1 KB runs of each qT row instead of 128-byte pieces spread over all of
  // them (workload 4's dY 8192 x 14336: 99 -> 91 us, the rate of a device-to-device copy with
  // the same read:write mix; 64-row bands helped dY more and X, W less)
  auto tile_rc = [&](int64_t ix, int64_t& rb, int64_t& kb) {
    if constexpr (KIND == kBwTensor) {
      constexpr int64_t SR = 8;
      const int64_t band = ix / (SR * nkb), first = band * SR;
      const int64_t h = nrb - first < SR ? nrb - first : SR;
      const int64_t in = ix - band * SR * nkb;
      rb = first + in % h;
      kb = in / h;
    } else {
      rb = ix / nkb;
      kb = ix - rb * nkb;
    }
  };
  // the tile stays as loaded (packed bf16: 16 VGPRs) until the cast widens it: widened at the
  // load, the 1x128 mode held 110 VGPRs (2 blocks per CU) and the others ~70 (3); now 56-60 (4)
  Raw8<BF16> raw[4];
  auto load_tile = [&](int64_t ix) {
    int64_t rb, kb;
    tile_rc(ix, rb, kb);
    const int64_t base = rb * 128 * cols + kb * 128 + cg * 8;
#pragma unroll
    for (int p = 0; p < 4; ++p) raw[p] = load_raw8<BF16>(x, base + (int64_t)(r16 + 32 * p) * cols);
  };
  // tile ix = blockIdx.x, + gridDim.x, ... (the blockwise launches have one block per tile; the
  // per-tensor launch is capped at the blocks resident at once, see launch_ct); each tile's
  // loads are issued before the previous tile's transpose
  auto tile = [&](int64_t ix) {
  int64_t rb, kb;
  tile_rc(ix, rb, kb);
  const int64_t base = rb * 128 * cols + kb * 128 + cg * 8;
  if constexpr (KIND != kBwTensor) {
#pragma unroll
    for (int p = 0; p < 4; ++p) raw[p] = load_raw8<BF16>(x, base + (int64_t)(r16 + 32 * p) * cols);
  }
  uint32_t m[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) m[p] = raw_amax_bits<BF16>(raw[p]);
  float srow[4], scol[8];
  if constexpr (KIND == kBwTensor) {
    const float sc = *scale_p;
#pragma unroll
    for (int p = 0; p < 4; ++p) srow[p] = sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) scol[e] = sc;
#pragma unroll
    for (int p = 0; p < 4; ++p) amax_acc = amax_acc > m[p] ? amax_acc : m[p];
  } else if constexpr (TILE) {
    // row runs: the 16 lanes sharing r16
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float si;
      current_scale<FMT>(group_max_u32<16>(m[p]), srow[p], si);
      if (cg == 0) q_sinv[kb * rows + rb * 128 + r16 + 32 * p] = si;  // [cols/128][rows]
    }
    // column runs: this thread's 4 rows, then the wave's 4 lane groups, then the 8 waves
    uint32_t cm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t c = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = raw_abs_bits<BF16>(raw[p], e);
        c = c > a ? c : a;
      }
      uint32_t o = (uint32_t)__shfl_xor((int)c, 16, 64);
      c = c > o ? c : o;
      o = (uint32_t)__shfl_xor((int)c, 32, 64);
      cm[e] = c > o ? c : o;
    }
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) cred[wave][cg * 8 + e] = cm[e];
    }
    __syncthreads();
    if (t < 128) {
      uint32_t c = cred[0][t];
#pragma unroll
      for (int w = 1; w < 8; ++w) c = c > cred[w][t] ? c : cred[w][t];
      float sc, si;
      current_scale<FMT>(c, sc, si);
      cscale[t] = sc;
      qT_sinv[rb * cols + kb * 128 + t] = si;  // [rows/128][cols]
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) scol[e] = cscale[cg * 8 + e];
  } else {
    uint32_t mx = m[0];
#pragma unroll
    for (int p = 1; p < 4; ++p) mx = mx > m[p] ? mx : m[p];
    mx = wave_max_u32(mx);
    if (lane == 0) cred[wave][0] = mx;
    __syncthreads();
    uint32_t bm = cred[0][0];
#pragma unroll
    for (int w = 1; w < 8; ++w) bm = bm > cred[w][0] ? bm : cred[w][0];
    float sc, si;
    current_scale<FMT>(bm, sc, si);
#pragma unroll
    for (int p = 0; p < 4; ++p) srow[p] = sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) scol[e] = sc;
    if (t == 0) {
      q_sinv[rb * nkb + kb] = si;   // [rows/128][cols/128]
      qT_sinv[kb * nrb + rb] = si;  // [cols/128][rows/128]
    }
  }
  // q with the row scales; the qT codes (column scales) into the LDS tile
#pragma unroll
  for (int p = 0; p < 4; ++p) opaque_raw8<BF16>(raw[p]);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float sr = srow[p];
    float v[8];
    widen8<BF16>(raw[p], v);
    uint32_t w0 = cvt4<FMT>(v[0] * sr, v[1] * sr, v[2] * sr, v[3] * sr);
    uint32_t w1 = cvt4<FMT>(v[4] * sr, v[5] * sr, v[6] * sr, v[7] * sr);
    uint32_t c0 = cvt4<FMT>(v[0] * scol[0], v[1] * scol[1], v[2] * scol[2], v[3] * scol[3]);
    uint32_t c1 = cvt4<FMT>(v[4] * scol[4], v[5] * scol[5], v[6] * scol[6], v[7] * scol[7]);
    if (m[p] > 0x7F800000u) {
      w0 = patch_nan4(w0, &v[0]);
      w1 = patch_nan4(w1, &v[4]);
      c0 = patch_nan4(c0, &v[0]);
      c1 = patch_nan4(c1, &v[4]);
    }
    const u32x2 w = {w0, w1};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(q + base + (int64_t)(r16 + 32 * p) * cols));
    lds[(r16 + 32 * p) * kBwPitch + cg * 2] = c0;
    lds[(r16 + 32 * p) * kBwPitch + cg * 2 + 1] = c1;
  }
  // the next tile's loads (per tensor: the blockwise launches run one tile per block)
  if constexpr (KIND == kBwTensor)
    if (ix + gridDim.x < ntiles) load_tile(ix + gridDim.x);  // this tile's codes are out of raw
  __syncthreads();
  // transpose: 4 source rows x 4 source columns per dword quad
  const int rg = t & 31, cgt = t >> 5;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cq = cgt + 16 * h;  // source columns 4cq .. 4cq+3
    const uint32_t d0 = lds[(4 * rg + 0) * kBwPitch + cq];
    const uint32_t d1 = lds[(4 * rg + 1) * kBwPitch + cq];
    const uint32_t d2 = lds[(4 * rg + 2) * kBwPitch + cq];
    const uint32_t d3 = lds[(4 * rg + 3) * kBwPitch + cq];
    const uint32_t lo01 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);
    const uint32_t hi01 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);
    const uint32_t lo23 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
    uint32_t o[4];
    o[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_nontemporal_store(o[j],
                                  reinterpret_cast<uint32_t*>(qT + (kb * 128 + 4 * cq + j) * rows + rb * 128 + 4 * rg));
  }
  };
  if constexpr (KIND == kBwTensor) {
    load_tile(blockIdx.x);
    for (int64_t ix = blockIdx.x; ix < ntiles; ix += gridDim.x) {
      if (ix != (int64_t)blockIdx.x) __syncthreads();  // the previous tile's transpose is done with lds
      tile(ix);
    }
  } else {
    tile(blockIdx.x);
  }
  // per tensor: the block's amax into the slot with one atomic.  One atomic per 128 x 128 tile
  // (a block per tile) cost workload 4's dY 16 us of 87 when the slot starts each call at zero,
  // as it does in a training step: while atomics queue at the slot, the plain reads that should
  // filter them return stale values.
  if constexpr (KIND == kBwTensor) {
    if (amax_slot != nullptr) {
      const uint32_t mx = wave_max_u32(amax_acc);
      __syncthreads();
      if (lane == 0) cred[wave][0] = mx;
      __syncthreads();
      if (t == 0) {
        uint32_t bm = cred[0][0];
#pragma unroll
        for (int w = 1; w < 8; ++w) bm = bm > cred[w][0] ? bm : cred[w][0];
        if (bm > __hip_atomic_load(amax_slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(amax_slot, bm);
      }
    }
  }
}

template <int FMT, bool BF16>
static int launch_ct(const void* x, int64_t rows, int64_t cols, const float* scale, float* amax_slot, uint8_t* q,
                     uint8_t* qT, hipStream_t st) {
  const int64_t ntiles = ((rows + kCtTile - 1) / kCtTile) * ((cols + kCtTile - 1) / kCtTile);
  // 64 x 64 tiles: the grid is capped at 8 blocks per CU (those resident at once), which loop
  // over the tiles, so that the amax takes one atomic per block, not per tile (see the per-tensor
  // launch below; in the slot's first use of a step atomics queue and the reads that filter them
  // go stale)
  const int64_t cap = 8ll * device_cus();
  const int64_t blocks = ntiles < cap ? ntiles : cap;
  if (rows % 128 == 0 && cols % 128 == 0 && (rows >> 7) * (cols >> 7) < 0x7FFFFFFF) {
    // 128 x 128 tiles, the blockwise kernel with the per-tensor scale: whole 128-byte lines of q
    // and qT (8192 x 14336 bf16: 88-91 us against 132 us on 64 x 64 tiles, inputs and outputs
    // beyond the last-level cache)
    // 20 KB of unused dynamic LDS hold residency at 3 blocks per CU (41 KB each of 160 KB): at
    // the 4 its registers allow, this launch measured 2-5% slower at workload 4's shapes.
    // The grid is capped so that the blocks loop over tiles and fewer atomics carry the amax:
    // up to 16 tiles per CU, at the resident blocks (fp32 input: 2 per CU, its registers allow
    // no more); above, at 6/7 of the tiles and at most 24 blocks per CU, so that the first
    // blocks take two tiles.  Slot cleared / kept, bf16, us: workload 4's X (2048 tiles) 28-31 /
    // 27 (one block per tile: 42 / 26), W (3584) 46 / 45 (56 / 42; 4096 blocks or more: 54 / 43),
    // dY (7168) 90 / 88 (105 / 87; resident blocks only: 96 / 96; 4096-6144 blocks: 90-92 /
    // 89-90)
    const int64_t t128 = (rows >> 7) * (cols >> 7), cus = device_cus();
    const int64_t cap = t128 <= 16 * cus ? (BF16 ? 3 : 2) * cus : std::min<int64_t>(24 * cus, t128 * 6 / 7);
    hipLaunchKernelGGL((cast_transpose_bw_kernel<FMT, BF16, kBwTensor>), dim3((unsigned)(t128 < cap ? t128 : cap)),
                       dim3(512), kCtTensorLdsPad, st, x, rows, cols, q, nullptr, qT, nullptr, scale,
                       reinterpret_cast<uint32_t*>(amax_slot));
    return check_launch("fp8_cast_transpose");
  }
  hipLaunchKernelGGL((cast_transpose_kernel<FMT, BF16>), dim3((unsigned)blocks), dim3(256), 0, st, x, rows, cols,
                     scale, reinterpret_cast<uint32_t*>(amax_slot), q, qT);
  return check_launch("fp8_cast_transpose");
}

template <int FMT, bool BF16>
static int launch_ct_bw(const void* x, int64_t rows, int64_t cols, int gran, uint8_t* q, float* q_sinv, uint8_t* qT,
                        float* qT_sinv, hipStream_t st) {
  const int64_t blocks = (rows >> 7) * (cols >> 7);
  if (gran == FP8_SCALE_TILE_1x128)
    hipLaunchKernelGGL((cast_transpose_bw_kernel<FMT, BF16, kBwTile>), dim3((unsigned)blocks), dim3(512), 0, st, x,
                       rows, cols, q, q_sinv, qT, qT_sinv, nullptr, nullptr);
  else
    hipLaunchKernelGGL((cast_transpose_bw_kernel<FMT, BF16, kBwBlock>), dim3((unsigned)blocks), dim3(512), 0, st, x,
                       rows, cols, q, q_sinv, qT, qT_sinv, nullptr, nullptr);
  return check_launch("fp8_cast_transpose_blockwise");
}

}  // namespace sfp8

using namespace sfp8;

extern "C" int fp8_cast_transpose(const void* x, int x_dtype, int64_t rows, int64_t cols, int fmt, const float* scale,
                                  float* amax_slot, uint8_t* q, uint8_t* qT, void* stream) {
  SFP8_REQUIRE(rows >= 0 && cols >= 0, FP8_ERR_SHAPE, "fp8_cast_transpose: negative shape (%lld, %lld)",
               (long long)rows, (long long)cols);
  SFP8_REQUIRE(x_dtype == HP_F32 || x_dtype == HP_BF16, FP8_ERR_DTYPE, "fp8_cast_transpose: x_dtype %d", x_dtype);
  SFP8_REQUIRE(fmt == FP8_E4M3 || fmt == FP8_E5M2, FP8_ERR_ARG, "fp8_cast_transpose: fmt %d", fmt);
  SFP8_REQUIRE(scale != nullptr, FP8_ERR_ARG, "fp8_cast_transpose: null scale");
  SFP8_REQUIRE(aligned4(scale) && (amax_slot == nullptr || aligned4(amax_slot)), FP8_ERR_ARG,
               "fp8_cast_transpose: scale / amax_slot must be 4-byte aligned");
  if (rows * cols == 0) return FP8_OK;
  SFP8_REQUIRE(x != nullptr && q != nullptr && qT != nullptr, FP8_ERR_ARG, "fp8_cast_transpose: null x, q or qT");
  SFP8_REQUIRE(aligned16(x) && aligned16(q) && aligned16(qT), FP8_ERR_ARG,
               "fp8_cast_transpose: x, q and qT must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const bool bf = x_dtype == HP_BF16;
  if (fmt == FP8_E4M3)
    return bf ? launch_ct<FP8_E4M3, true>(x, rows, cols, scale, amax_slot, q, qT, st)
              : launch_ct<FP8_E4M3, false>(x, rows, cols, scale, amax_slot, q, qT, st);
  return bf ? launch_ct<FP8_E5M2, true>(x, rows, cols, scale, amax_slot, q, qT, st)
            : launch_ct<FP8_E5M2, false>(x, rows, cols, scale, amax_slot, q, qT, st);
}

extern "C" int fp8_cast_transpose_blockwise(const void* x, int x_dtype, int64_t rows, int64_t cols, int fmt,
                                            int granularity, uint8_t* q, float* q_scale_inv, uint8_t* qT,
                                            float* qT_scale_inv, void* stream) {
  SFP8_REQUIRE(rows >= 0 && cols >= 0, FP8_ERR_SHAPE, "fp8_cast_transpose_blockwise: negative shape (%lld, %lld)",
               (long long)rows, (long long)cols);
  SFP8_REQUIRE(x_dtype == HP_F32 || x_dtype == HP_BF16, FP8_ERR_DTYPE, "fp8_cast_transpose_blockwise: x_dtype %d",
               x_dtype);
  SFP8_REQUIRE(fmt == FP8_E4M3 || fmt == FP8_E5M2, FP8_ERR_ARG, "fp8_cast_transpose_blockwise: fmt %d", fmt);
  SFP8_REQUIRE(granularity == FP8_SCALE_TILE_1x128 || granularity == FP8_SCALE_BLOCK_128x128, FP8_ERR_ARG,
               "fp8_cast_transpose_blockwise: granularity %d (TILE_1x128 or BLOCK_128x128)", granularity);
  SFP8_REQUIRE(rows % 128 == 0 && cols % 128 == 0, FP8_ERR_SHAPE,
               "fp8_cast_transpose_blockwise: rows=%lld and cols=%lld must be multiples of 128", (long long)rows,
               (long long)cols);
  if (rows * cols == 0) return FP8_OK;
  SFP8_REQUIRE(x != nullptr && q != nullptr && qT != nullptr && q_scale_inv != nullptr && qT_scale_inv != nullptr,
               FP8_ERR_ARG, "fp8_cast_transpose_blockwise: null pointer");
  SFP8_REQUIRE(aligned16(x) && aligned16(q) && aligned16(qT), FP8_ERR_ARG,
               "fp8_cast_transpose_blockwise: x, q and qT must be 16-byte aligned");
  SFP8_REQUIRE(aligned4(q_scale_inv) && aligned4(qT_scale_inv), FP8_ERR_ARG,
               "fp8_cast_transpose_blockwise: scale_inv arrays must be 4-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const bool bf = x_dtype == HP_BF16;
  if (fmt == FP8_E4M3)
    return bf ? launch_ct_bw<FP8_E4M3, true>(x, rows, cols, granularity, q, q_scale_inv, qT, qT_scale_inv, st)
              : launch_ct_bw<FP8_E4M3, false>(x, rows, cols, granularity, q, q_scale_inv, qT, qT_scale_inv, st);
  return bf ? launch_ct_bw<FP8_E5M2, true>(x, rows, cols, granularity, q, q_scale_inv, qT, qT_scale_inv, st)
            : launch_ct_bw<FP8_E5M2, false>(x, rows, cols, granularity, q, q_scale_inv, qT, qT_scale_inv, st);
}
