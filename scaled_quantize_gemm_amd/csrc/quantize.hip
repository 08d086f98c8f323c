// Fused amax + scale + saturating RNE cast to FP8, at four scale granularities.
//
// "Transformer Scaling" lesson, Part 01 (a scale maps values into the FP8 range, often via
// amax) and Core vocabulary (delayed scaling avoids a second, pre-quantisation read);
// "Week 14" course page, absmax bullet (per-tensor and per-block scales; MX: a shared
// scale per 32 numbers; DeepSeek-V3: per 128 activation values and per 128x128 weight block,
// computed online from the current block).
//
// Every kernel reads its input once from HBM and writes the codes once: amax is computed
// from the same registers the cast reads (delayed scaling records it for the next step;
// the blockwise and MX kernels hold the whole block in registers, reduce, then cast).
#include "quant_rules.h"

namespace sfp8 {

template <bool BF16>
__device__ __forceinline__ float load_one(const void* __restrict__ base, int64_t i) {
  if constexpr (BF16) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[i] << 16);
  else return static_cast<const float*>(base)[i];
}

template <int FMT>
__device__ __forceinline__ uint8_t cast_one(float x, float s) {
  uint32_t w = cvt_pair<FMT, false>(x * s, 0.0f, 0u) & 0xFFu;
  uint32_t b = __float_as_uint(x);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) w = nan_code(b);
  return (uint8_t)w;
}

// Block-wide unsigned max (NW waves) -> returned to every thread.
template <int NW>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = r > red[i] ? r : red[i];
  return r;
}

// ------------------------------------------------------------------ per-tensor (delayed)
//
// Flat stream over n elements in pieces of 8 (16 bytes of bf16).  A block takes 2 x 1024
// pieces per pass of a grid-stride loop; the pieces of one load instruction are consecutive
// across the wave's lanes, so every instruction reads 1 KB (bf16) contiguous.  amax is
// reduced per block and max-ed into *amax_slot with one unsigned atomic per block (|x| bits
// of non-negative floats order like the floats; NaN wins).
// The grid is capped at 4 blocks of 1024 threads per CU (two rounds of the resident ones).  The
// atomics decide it: in a training step the slot starts each call at zero, and with a block
// per 4096 elements (32768 blocks of 256 threads on 2^28) the 2^28-element cast took 156 us
// instead of the 126 it takes when the slot already holds the maximum (the plain reads that
// filter the atomics return stale values while atomics queue at the slot); 1024 blocks of
// 1024 threads take 131 / 128 us.

constexpr int kTensorThreads = 1024;
constexpr int kTensorPieces = 2;
constexpr int kTensorBlocksPerCu = 4;

// Cast diagnostics (DIAG): per element, saturated = |fp32(x s)| > fmax (so the code was
// clipped), underflowed = x finite and non-zero but its code is +-0, nan = x is NaN; block
// sums are added to counts[0..2] with one 64-bit atomic each.
template <int FMT>
__device__ __forceinline__ void diag8(const float (&v)[8], float s, u32x2 codes, uint32_t (&cnt)[3]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float y = v[i] * s;
    const uint32_t a = abs_bits(v[i]);
    const uint32_t code = ((i < 4 ? codes.x : codes.y) >> (8 * (i & 3))) & 0x7Fu;
    cnt[0] += fabsf(y) > Fp8Traits<FMT>::fmax ? 1u : 0u;
    cnt[1] += (a != 0 && a < 0x7F800000u && code == 0) ? 1u : 0u;
    cnt[2] += a > 0x7F800000u ? 1u : 0u;
  }
}

template <int FMT, bool BF16, bool DIAG>
__global__ void __launch_bounds__(kTensorThreads) quant_tensor_kernel(const void* __restrict__ x, int64_t n,
                                                                      const float* __restrict__ scale_p,
                                                                      uint32_t* __restrict__ amax_slot,
                                                                      uint8_t* __restrict__ q,
                                                                      unsigned long long* __restrict__ counts) {
  constexpr int NW = kTensorThreads / 64;
  __shared__ uint32_t red[NW];
  __shared__ uint32_t cred[DIAG ? 3 : 1][NW];
  uint32_t cnt[3] = {0, 0, 0};
  const float s = *scale_p;
  const int64_t npieces = n >> 3;
  const int64_t step = (int64_t)gridDim.x * kTensorThreads * kTensorPieces;
  uint32_t mxf = 0;
  for (int64_t b = (int64_t)blockIdx.x * kTensorThreads * kTensorPieces; b < npieces; b += step) {
    float v[kTensorPieces][8];
#pragma unroll
    for (int j = 0; j < kTensorPieces; ++j) {
      const int64_t pc = b + j * kTensorThreads + threadIdx.x;
      if (pc < npieces) load8<BF16>(x, pc << 3, v[j]);
    }
#pragma unroll
    for (int j = 0; j < kTensorPieces; ++j) {
      const int64_t pc = b + j * kTensorThreads + threadIdx.x;
      if (pc < npieces) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t a = abs_bits(v[j][i]);
          m = m > a ? m : a;
        }
        const u32x2 codes = cast8<FMT>(v[j], s, m);
        __builtin_nontemporal_store(codes, reinterpret_cast<u32x2*>(q + (pc << 3)));
        mxf = mxf > m ? mxf : m;
        if constexpr (DIAG) diag8<FMT>(v[j], s, codes, cnt);
      }
    }
  }
  // tail (n % 8 elements): block 0
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t i = (npieces << 3) + threadIdx.x;
    float xv = load_one<BF16>(x, i);
    const uint8_t c = cast_one<FMT>(xv, s);
    q[i] = c;
    uint32_t a = abs_bits(xv);
    mxf = mxf > a ? mxf : a;
    if constexpr (DIAG) {
      cnt[0] += fabsf(xv * s) > Fp8Traits<FMT>::fmax ? 1u : 0u;
      cnt[1] += (a != 0 && a < 0x7F800000u && (c & 0x7Fu) == 0) ? 1u : 0u;
      cnt[2] += a > 0x7F800000u ? 1u : 0u;
    }
  }
  if constexpr (DIAG) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      uint32_t v = cnt[k];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
      if ((threadIdx.x & 63) == 0) cred[k][threadIdx.x >> 6] = v;
    }
  }
  uint32_t r = block_max_u32<NW>(mxf, red);  // (its barrier also publishes cred)
  if constexpr (DIAG) {
    if (threadIdx.x < 3) {
      uint32_t tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += cred[threadIdx.x][w];
      if (tot != 0) atomicAdd(counts + threadIdx.x, (unsigned long long)tot);
    }
  }
  // a plain read first: most blocks do not raise the running maximum
  if (threadIdx.x == 0 && amax_slot != nullptr &&
      r > __hip_atomic_load(amax_slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    atomicMax(amax_slot, r);
}

// ------------------------------------------------------------------ 1x128 tiles
//
// One 16-lane group per 1x128 run (8 elements per lane): amax over the group, s = fmax/amax,
// cast.  A block covers 8 rows x 4 runs (512 columns); wave w takes rows 2w, 2w+1 of it, so
// each lane has two rows' loads in flight and each wave reads 1 KB row segments (4096 x 7168
// bf16: 17.3 us with 2 rows per wave, 18.5 with 4, 20.8 with 8, 19.5 with 1).
// Consecutive blocks walk the input in address order.  scale_inv is [kb][row] (kb-major, so
// one K step of the GEMM reads a contiguous vector of rows); the block's 4 x 16 values are
// staged in LDS and leave as 32-byte rows of that layout.

constexpr int kTileRowsPerWave = 2;
constexpr int kTileRows = 4 * kTileRowsPerWave;

template <int FMT, bool BF16>
__global__ void __launch_bounds__(256) quant_tile_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                         uint8_t* __restrict__ q, float* __restrict__ sinv_out) {
  __shared__ float sinv_s[4][kTileRows];
  const int64_t nkb = cols >> 7;
  const int64_t ncb = (nkb + 3) >> 2;
  const int64_t rb = blockIdx.x / ncb, cb = blockIdx.x - rb * ncb;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lrun = lane >> 4, lane16 = lane & 15;
  const int64_t kb = cb * 4 + lrun;
  const int64_t row0 = rb * kTileRows + wave * kTileRowsPerWave;
  if (kb < nkb) {  // whole 16-lane groups take the same branch
    const int64_t c0 = kb * 128 + lane16 * 8;
    float v[kTileRowsPerWave][8];
#pragma unroll
    for (int j = 0; j < kTileRowsPerWave; ++j)
      if (row0 + j < rows) load8<BF16>(x, (row0 + j) * cols + c0, v[j]);
#pragma unroll
    for (int j = 0; j < kTileRowsPerWave; ++j) {
      if (row0 + j >= rows) break;
      uint32_t mx = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t a = abs_bits(v[j][i]);
        mx = mx > a ? mx : a;
      }
      const bool nan_here = mx > 0x7F800000u;
      mx = group_max_u32<16>(mx);
      float s, s_inv;
      current_scale<FMT>(mx, s, s_inv);
      uint32_t w0 = cvt4<FMT>(v[j][0] * s, v[j][1] * s, v[j][2] * s, v[j][3] * s);
      uint32_t w1 = cvt4<FMT>(v[j][4] * s, v[j][5] * s, v[j][6] * s, v[j][7] * s);
      if (nan_here) {
        w0 = patch_nan4(w0, &v[j][0]);
        w1 = patch_nan4(w1, &v[j][4]);
      }
      const u32x2 o = {w0, w1};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(q + (row0 + j) * cols + c0));
      if (lane16 == 0) sinv_s[lrun][wave * kTileRowsPerWave + j] = s_inv;
    }
  }
  __syncthreads();
  if (threadIdx.x < 4 * kTileRows) {
    const int lr = threadIdx.x / kTileRows, rr = threadIdx.x - lr * kTileRows;
    const int64_t kbx = cb * 4 + lr, row = rb * kTileRows + rr;
    if (kbx < nkb && row < rows) sinv_out[kbx * rows + row] = sinv_s[lr][rr];
  }
}

// ------------------------------------------------------------------ 128x128 blocks
//
// One 512-thread block per 128x128 block (blocks in address order): thread t covers rows
// t/16 + 32p (p = 0..3), columns 8(t%16)..+8, so each load instruction reads 4 whole
// 256-byte block rows; the 32 values stay in registers through the block reduction (wave
// shuffles, then the 8 waves in LDS).  A partial last row block uses the rows present
// (absent rows contribute nothing).

constexpr int kBlockThreads = 512;

// the block's amax from each thread's partial maximum `mx` (fp32 bits of |x|): the scale for
// the cast, with its scale_inv stored by thread 0 at sinv_out[at]
template <int FMT>
__device__ __forceinline__ float block_scale(uint32_t mx, int t, float* __restrict__ sinv_out, int64_t at) {
  __shared__ uint32_t red[8];
  mx = wave_max_u32(mx);
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  uint32_t bm = red[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) bm = bm > red[i] ? bm : red[i];
  float s, s_inv;
  current_scale<FMT>(bm, s, s_inv);
  if (t == 0) sinv_out[at] = s_inv;
  return s;
}

template <int FMT, bool BF16>
__global__ void __launch_bounds__(kBlockThreads) quant_block_kernel(const void* __restrict__ x, int64_t rows,
                                                                   int64_t cols, uint8_t* __restrict__ q,
                                                                   float* __restrict__ sinv_out) {
  const int64_t nkb = cols >> 7;
  const int64_t rb = blockIdx.x / nkb, kb = blockIdx.x - rb * nkb;
  const int t = threadIdx.x, r16 = t >> 4, cg = t & 15;
  const int64_t base = rb * 128 * cols + kb * 128 + cg * 8;
  // the 32 values stay as loaded (packed bf16: 16 VGPRs) across the barrier and widen at the
  // cast: widened at the load, the bf16 kernel held 86 VGPRs (2 blocks per CU, 64 KB of loads
  // in flight per CU); now 40 (4 blocks)
  Raw8<BF16> raw[4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
    raw[p] = rb * 128 + r16 + 32 * p < rows ? load_raw8<BF16>(x, base + (int64_t)(r16 + 32 * p) * cols)
                                            : zero_raw8<BF16>();
  uint32_t m[4], mx = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    m[p] = raw_amax_bits<BF16>(raw[p]);
    mx = mx > m[p] ? mx : m[p];
  }
  const float s = block_scale<FMT>(mx, t, sinv_out, rb * nkb + kb);
#pragma unroll
  for (int p = 0; p < 4; ++p)
    if (rb * 128 + r16 + 32 * p < rows) {
      float v[8];
      widen8<BF16>(raw[p], v);
      __builtin_nontemporal_store(cast8<FMT>(v, s, m[p]),
                                  reinterpret_cast<u32x2*>(q + base + (int64_t)(r16 + 32 * p) * cols));
    }
}


// ------------------------------------------------------------------ MX 1x32
//
// One 4-lane group per 1x32 run (8 elements per lane).  E = smallest integer with
// amax <= fmax * 2^E, from amax's exponent e and mantissa: E = e - bias when the mantissa
// is <= 1.75 (bits <= 0x600000), else e - bias + 1 (bias 8 for E4M3, 15 for E5M2); clamped
// to [-127, 127]; zero amax -> -127; non-finite amax -> code 255 and multiplier 1.  The
// multiplier 2^-E is exact, so the product is rounded only once, by the cast.

// A block covers 4*kMxRowsPerWave rows x 16 runs (512 columns).  Wave w takes rows
// w*kMxRowsPerWave.. of the block; on each row its 64 lanes read 512 consecutive elements
// (4 lanes per run), so every load and code store is a contiguous row segment.  The e8m0
// codes collect in LDS as [run][row] and leave as contiguous pieces of the [cols/32][rows]
// layout.  Consecutive blocks walk the input in address order (all column blocks of one
// row group, then the next group): on 8192 x 8192 bf16 that order measured 32 us against
// 43 us for the column-block-major order, whose 16 KB row stride crowds few HBM channels.
constexpr int kMxRowsPerWave = 2;
constexpr int kMxRows = 4 * kMxRowsPerWave;
constexpr int kMxRuns = 16;


template <int FMT, bool BF16>
__global__ void __launch_bounds__(256) quant_mx_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                       uint8_t* __restrict__ q, uint8_t* __restrict__ e8) {
  __shared__ uint8_t codes[kMxRuns][kMxRows];
  const int64_t nrun = cols >> 5;
  const int64_t ncb = (nrun + kMxRuns - 1) / kMxRuns;
  const int64_t rb = blockIdx.x / ncb, cb = blockIdx.x - rb * ncb;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lrun = lane >> 2, lane4 = lane & 3;
  const int64_t run = cb * kMxRuns + lrun;
  const int64_t row0 = rb * kMxRows + wave * kMxRowsPerWave;
  if (run < nrun) {  // whole 4-lane groups take the same branch
    const int64_t c0 = run * 32 + lane4 * 8;
    float v[kMxRowsPerWave][8];
#pragma unroll
    for (int j = 0; j < kMxRowsPerWave; ++j)
      if (row0 + j < rows) load8<BF16>(x, (row0 + j) * cols + c0, v[j]);
#pragma unroll
    for (int j = 0; j < kMxRowsPerWave; ++j) {
      if (row0 + j >= rows) break;
      uint32_t mx = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t a = abs_bits(v[j][i]);
        mx = mx > a ? mx : a;
      }
      const bool nan_here = mx > 0x7F800000u;
      mx = group_max_u32<4>(mx);
      uint32_t code;
      float mult;
      mx_rule<FMT>(mx, code, mult);
      uint32_t w0 = cvt4<FMT>(v[j][0] * mult, v[j][1] * mult, v[j][2] * mult, v[j][3] * mult);
      uint32_t w1 = cvt4<FMT>(v[j][4] * mult, v[j][5] * mult, v[j][6] * mult, v[j][7] * mult);
      if (nan_here) {
        w0 = patch_nan4(w0, &v[j][0]);
        w1 = patch_nan4(w1, &v[j][4]);
      }
      u32x2 o = {w0, w1};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(q + (row0 + j) * cols + c0));
      if (lane4 == 0) codes[lrun][wave * kMxRowsPerWave + j] = (uint8_t)code;
    }
  }
  __syncthreads();
  const int64_t rbase = rb * kMxRows;
  for (int i = threadIdx.x; i < kMxRuns * kMxRows; i += 256) {
    const int lr = i / kMxRows, rr = i - lr * kMxRows;
    const int64_t rn = cb * kMxRuns + lr;
    if (rn < nrun && rbase + rr < rows) e8[rn * rows + rbase + rr] = codes[lr][rr];
  }
}

// ------------------------------------------------------------------ launchers

template <int FMT, bool BF16>
static int launch_quant(const void* x, int64_t rows, int64_t cols, int gran, const float* scale, float* amax_slot,
                        uint8_t* q, void* sinv, hipStream_t st) {
  const int64_t n = rows * cols;
  if (gran == FP8_SCALE_TENSOR) {
    const int64_t per_block = (int64_t)kTensorThreads * kTensorPieces * 8;
    int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks < 1) blocks = 1;
    if (blocks > (int64_t)kTensorBlocksPerCu * device_cus()) blocks = (int64_t)kTensorBlocksPerCu * device_cus();
    hipLaunchKernelGGL((quant_tensor_kernel<FMT, BF16, false>), dim3((unsigned)blocks), dim3(kTensorThreads), 0, st,
                       x, n, scale, reinterpret_cast<uint32_t*>(amax_slot), q, nullptr);
  } else if (gran == FP8_SCALE_TILE_1x128) {
    const int64_t blocks = ((rows + kTileRows - 1) / kTileRows) * (((cols >> 7) + 3) / 4);
    hipLaunchKernelGGL((quant_tile_kernel<FMT, BF16>), dim3((unsigned)blocks), dim3(256), 0, st, x, rows, cols, q,
                       static_cast<float*>(sinv));
  } else if (gran == FP8_SCALE_BLOCK_128x128) {
    const int64_t blocks = ((rows + 127) / 128) * (cols >> 7);
    hipLaunchKernelGGL((quant_block_kernel<FMT, BF16>), dim3((unsigned)blocks), dim3(kBlockThreads), 0, st, x, rows,
                       cols, q, static_cast<float*>(sinv));
  } else {
    const int64_t blocks = ((rows + kMxRows - 1) / kMxRows) * (((cols >> 5) + kMxRuns - 1) / kMxRuns);
    hipLaunchKernelGGL((quant_mx_kernel<FMT, BF16>), dim3((unsigned)blocks), dim3(256), 0, st, x, rows, cols, q,
                       static_cast<uint8_t*>(sinv));
  }
  return check_launch("fp8_quantize");
}

}  // namespace sfp8

using namespace sfp8;

extern "C" int fp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int fmt, int granularity,
                            const float* scale, float* amax_slot, uint8_t* q, void* scale_inv_out, void* stream) {
  SFP8_REQUIRE(rows >= 0 && cols >= 0, FP8_ERR_SHAPE, "fp8_quantize: negative shape (%lld, %lld)", (long long)rows,
               (long long)cols);
  SFP8_REQUIRE(x_dtype == HP_F32 || x_dtype == HP_BF16, FP8_ERR_DTYPE, "fp8_quantize: x_dtype %d", x_dtype);
  SFP8_REQUIRE(fmt == FP8_E4M3 || fmt == FP8_E5M2, FP8_ERR_ARG, "fp8_quantize: fmt %d", fmt);
  SFP8_REQUIRE(granularity >= FP8_SCALE_TENSOR && granularity <= FP8_SCALE_MX_1x32, FP8_ERR_ARG,
               "fp8_quantize: granularity %d", granularity);
  if (granularity == FP8_SCALE_TENSOR) {
    SFP8_REQUIRE(scale != nullptr, FP8_ERR_ARG, "fp8_quantize: per-tensor scaling needs the device scale");
    SFP8_REQUIRE(scale_inv_out == nullptr, FP8_ERR_ARG, "fp8_quantize: per-tensor scaling writes no scale_inv");
    SFP8_REQUIRE(aligned4(scale) && (amax_slot == nullptr || aligned4(amax_slot)), FP8_ERR_ARG,
                 "fp8_quantize: scale / amax_slot must be 4-byte aligned");
  } else {
    SFP8_REQUIRE(scale == nullptr && amax_slot == nullptr, FP8_ERR_ARG,
                 "fp8_quantize: current-scaling granularities take no scale / amax_slot");
    const int64_t run = granularity == FP8_SCALE_MX_1x32 ? 32 : 128;
    SFP8_REQUIRE(cols % run == 0, FP8_ERR_SHAPE, "fp8_quantize: cols=%lld must be a multiple of %lld",
                 (long long)cols, (long long)run);
    SFP8_REQUIRE(rows * cols == 0 || scale_inv_out != nullptr, FP8_ERR_ARG, "fp8_quantize: scale_inv_out is null");
    SFP8_REQUIRE(granularity == FP8_SCALE_MX_1x32 || scale_inv_out == nullptr || aligned4(scale_inv_out), FP8_ERR_ARG,
                 "fp8_quantize: scale_inv_out must be 4-byte aligned");
  }
  if (rows * cols == 0) return FP8_OK;
  SFP8_REQUIRE(x != nullptr && q != nullptr, FP8_ERR_ARG, "fp8_quantize: null x or q");
  SFP8_REQUIRE(aligned16(x) && aligned16(q), FP8_ERR_ARG, "fp8_quantize: x and q must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const bool bf = x_dtype == HP_BF16;
  if (fmt == FP8_E4M3)
    return bf ? launch_quant<FP8_E4M3, true>(x, rows, cols, granularity, scale, amax_slot, q, scale_inv_out, st)
              : launch_quant<FP8_E4M3, false>(x, rows, cols, granularity, scale, amax_slot, q, scale_inv_out, st);
  return bf ? launch_quant<FP8_E5M2, true>(x, rows, cols, granularity, scale, amax_slot, q, scale_inv_out, st)
            : launch_quant<FP8_E5M2, false>(x, rows, cols, granularity, scale, amax_slot, q, scale_inv_out, st);
}

extern "C" int fp8_quantize_diag(const void* x, int x_dtype, int64_t rows, int64_t cols, int fmt, const float* scale,
                                 float* amax_slot, uint8_t* q, unsigned long long* counts, void* stream) {
  SFP8_REQUIRE(rows >= 0 && cols >= 0, FP8_ERR_SHAPE, "fp8_quantize_diag: negative shape (%lld, %lld)",
               (long long)rows, (long long)cols);
  SFP8_REQUIRE(x_dtype == HP_F32 || x_dtype == HP_BF16, FP8_ERR_DTYPE, "fp8_quantize_diag: x_dtype %d", x_dtype);
  SFP8_REQUIRE(fmt == FP8_E4M3 || fmt == FP8_E5M2, FP8_ERR_ARG, "fp8_quantize_diag: fmt %d", fmt);
  SFP8_REQUIRE(scale != nullptr && counts != nullptr, FP8_ERR_ARG, "fp8_quantize_diag: null scale or counts");
  SFP8_REQUIRE(aligned4(scale) && (amax_slot == nullptr || aligned4(amax_slot)) &&
                   (reinterpret_cast<uintptr_t>(counts) & 7) == 0,
               FP8_ERR_ARG, "fp8_quantize_diag: scale / amax_slot must be 4-byte and counts 8-byte aligned");
  const int64_t n = rows * cols;
  if (n == 0) return FP8_OK;
  SFP8_REQUIRE(x != nullptr && q != nullptr, FP8_ERR_ARG, "fp8_quantize_diag: null x or q");
  SFP8_REQUIRE(aligned16(x) && aligned16(q), FP8_ERR_ARG, "fp8_quantize_diag: x and q must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const int64_t per_block = (int64_t)kTensorThreads * kTensorPieces * 8;
  int64_t blocks = (n + per_block - 1) / per_block;
  if (blocks < 1) blocks = 1;
  if (blocks > (int64_t)kTensorBlocksPerCu * device_cus()) blocks = (int64_t)kTensorBlocksPerCu * device_cus();
  const dim3 grid((unsigned)blocks), block(kTensorThreads);
  uint32_t* slot = reinterpret_cast<uint32_t*>(amax_slot);
  const bool bf = x_dtype == HP_BF16;
  if (fmt == FP8_E4M3) {
    if (bf) hipLaunchKernelGGL((quant_tensor_kernel<FP8_E4M3, true, true>), grid, block, 0, st, x, n, scale, slot, q, counts);
    else hipLaunchKernelGGL((quant_tensor_kernel<FP8_E4M3, false, true>), grid, block, 0, st, x, n, scale, slot, q, counts);
  } else {
    if (bf) hipLaunchKernelGGL((quant_tensor_kernel<FP8_E5M2, true, true>), grid, block, 0, st, x, n, scale, slot, q, counts);
    else hipLaunchKernelGGL((quant_tensor_kernel<FP8_E5M2, false, true>), grid, block, 0, st, x, n, scale, slot, q, counts);
  }
  return check_launch("fp8_quantize_diag");
}
