// Matrix-core ceiling on given FP8 data, for the GEMM's roofline: every wave issues scaled
// 32x32x64 FP8 MFMAs back to back (the large-tile GEMM kernel's instruction, with 8 independent
// accumulators per wave), alternating between two operand sets read once from the caller's
// FP8 codes and e8m0 bytes, so that the data toggles the multipliers as the GEMM's does.  Wave
// 0 of each block records the core cycle counter and the constant-rate counter around its
// loop: their ratio is the clock the chip ran at.  Measurement only; no part of the FP8 path.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "../../include/fp8_calib.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;

__global__ void __launch_bounds__(512) mfma_ceiling_kernel(const uint8_t* __restrict__ A, uint64_t a_chunks,
                                                           const uint32_t* __restrict__ E, uint64_t e_words,
                                                           int iters, float* __restrict__ sink,
                                                           long long* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const uint64_t gw = (uint64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  // 2 sets x (4 A + 2 B) fragments of 32 bytes per lane, at 32-byte chunks inside A
  v8i f[12];
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const uint64_t chunk = ((gw * 12 + i) * 64 + lane) % a_chunks;
    const uint4* p = reinterpret_cast<const uint4*>(A + chunk * 32);
    const uint4 lo = p[0], hi = p[1];
    f[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  int sa[2], sb[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    sa[s] = (int)E[((gw * 4 + 2 * s) * 64 + lane) % e_words];
    sb[s] = (int)E[((gw * 4 + 2 * s + 1) * 64 + lane) % e_words];
  }
  v16f acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  const long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f[6 * s + t / 2], f[6 * s + 4 + t % 2], acc[t], 0, 0, 0,
                                                                 sa[s], 0, sb[s]);
  }
  const long long c1 = clock64(), w1 = wall_clock64();
  float v = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) v += acc[t][e];
  sink[gw * 64 + lane] = v;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = w1 - w0;
  }
}

}  // namespace

extern "C" int fp8_calib_mfma(const uint8_t* A, size_t a_bytes, const uint8_t* e8m0, size_t e_bytes, int blocks,
                              int iters, float* sink, long long* clocks, void* stream) {
  if (A == nullptr || e8m0 == nullptr || sink == nullptr || clocks == nullptr) return -1;
  if (a_bytes < 32 * 64 || e_bytes < 4 * 64 || blocks <= 0 || iters <= 0) return -2;
  if ((reinterpret_cast<uintptr_t>(A) & 15) || (reinterpret_cast<uintptr_t>(e8m0) & 3)) return -1;
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(blocks), dim3(64 * kWaves), 0, (hipStream_t)stream, A,
                     (uint64_t)(a_bytes / 32), reinterpret_cast<const uint32_t*>(e8m0), (uint64_t)(e_bytes / 4), iters,
                     sink, clocks);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" double fp8_calib_mfma_flops(int blocks, int iters) {
  return (double)blocks * kWaves * iters * 16 * (2.0 * 32 * 32 * 64);
}

extern "C" int fp8_calib_wall_clock_khz(int device) {
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) != hipSuccess) return -4;
  return khz;
}
