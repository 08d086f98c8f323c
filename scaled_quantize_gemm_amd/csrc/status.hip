// Error text, device check and the delayed-scaling recipe update.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace sfp8 {

static thread_local char g_last_error[512] = "";

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(FP8_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return FP8_OK;
}

// ------------------------------------------------------------------ recipe update
//
// "Transformer Scaling" lesson (Part 01; Core vocabulary): delayed scaling takes the
// scale from the amax history; Worked example 01: scale = fmax / amax.  Transformer Engine
// tutorial: DelayedScaling(amax_history_len, amax_compute_algo="max"), history read back
// as amax_history[0, :4] (history-major).  One thread per slot; the history column is
// read once, its max taken as unsigned bits (entries are >= 0 or NaN, so NaN wins),
// the scale updated, and the column rolled: row i <- row i+1, last <- old row 0, row 0 <- 0.

struct FmtBits {
  uint32_t w[128];  // bit j set: slot j is E5M2 (4096 slots per launch)
};
constexpr int kSlotsPerLaunch = 4096;

__global__ void __launch_bounds__(256) recipe_update_kernel(float* __restrict__ hist, float* __restrict__ scale,
                                                             float* __restrict__ scale_inv, int n, int slot0,
                                                             int nslots, int H, float two_pow_neg_margin,
                                                             FmtBits fb) {
  int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= nslots) return;
  const int col = slot0 + j;
  const float fm = ((fb.w[j >> 5] >> (j & 31)) & 1u) ? 57344.0f : 448.0f;
  float* h = hist + col;
  const uint32_t first = __float_as_uint(h[0]);
  uint32_t m = first;
  // 16 rows at a time: their 17 loads (the 17th for the shift) in flight together, then the
  // shifted stores (row i <- row i + 1); the rows of a chunk are stored only after all its loads,
  // and a later chunk loads rows no earlier chunk stores.  One row per round trip measured
  // 4.7 us per call at H = 16.
  for (int i0 = 0; i0 < H; i0 += 16) {
    float v[17];
#pragma unroll
    for (int k = 0; k < 17; ++k) v[k] = i0 + k < H ? h[(size_t)(i0 + k) * n] : 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t b = __float_as_uint(v[k]);
      if (i0 + k < H) m = b > m ? b : m;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (i0 + k + 1 < H) h[(size_t)(i0 + k) * n] = v[k + 1];
  }
  if (m > 0u && m < 0x7F800000u) {
    float r = fm / __uint_as_float(m);
    r = fminf(r, 3.40282346638528859812e+38f);
    float s = r * two_pow_neg_margin;
    scale[col] = s;
    scale_inv[col] = 1.0f / s;
  }
  h[(size_t)(H - 1) * n] = __uint_as_float(first);
  h[0] = 0.0f;
}

}  // namespace sfp8

using namespace sfp8;

extern "C" int fp8_device_check(int device, char* reason, size_t reason_len) {
  char buf[256];
  int rc = FP8_OK;
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count == 0) {
    snprintf(buf, sizeof buf, "no HIP device available (%s)", e != hipSuccess ? hipGetErrorString(e) : "count = 0");
    rc = FP8_ERR_DEVICE;
  } else if (device < 0 || device >= count) {
    snprintf(buf, sizeof buf, "device %d out of range (%d devices)", device, count);
    rc = FP8_ERR_DEVICE;
  } else {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, device);
    if (e != hipSuccess) {
      snprintf(buf, sizeof buf, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
      rc = FP8_ERR_DEVICE;
    } else if (strncmp(p.gcnArchName, "gfx950", 6) != 0) {
      snprintf(buf, sizeof buf, "device %d is %s; this library is built for gfx950 (MI350 series) only", device,
               p.gcnArchName);
      rc = FP8_ERR_DEVICE;
    } else {
      snprintf(buf, sizeof buf, "ok: %s (%s), %d compute units", p.name, p.gcnArchName, p.multiProcessorCount);
    }
  }
  if (reason && reason_len) {
    strncpy(reason, buf, reason_len - 1);
    reason[reason_len - 1] = '\0';
  }
  if (rc != FP8_OK) set_error(rc, "%s", buf);
  return rc;
}

extern "C" const char* fp8_last_error(void) { return g_last_error; }

extern "C" int fp8_recipe_update(float* amax_history, float* scale, float* scale_inv, const int* fmts, int n,
                                 int history_len, int algo, int margin, void* stream) {
  SFP8_REQUIRE(amax_history && scale && scale_inv && fmts, FP8_ERR_ARG, "fp8_recipe_update: null pointer");
  SFP8_REQUIRE(n >= 1 && history_len >= 1, FP8_ERR_ARG, "fp8_recipe_update: n=%d history_len=%d must be >= 1", n,
               history_len);
  SFP8_REQUIRE(algo == FP8_AMAX_ALGO_MAX, FP8_ERR_ARG, "fp8_recipe_update: unknown amax algorithm %d", algo);
  SFP8_REQUIRE(margin >= 0 && margin <= 64, FP8_ERR_ARG, "fp8_recipe_update: margin %d out of [0, 64]", margin);
  SFP8_REQUIRE(aligned4(amax_history) && aligned4(scale) && aligned4(scale_inv), FP8_ERR_ARG,
               "fp8_recipe_update: fp32 buffers must be 4-byte aligned");
  for (int j = 0; j < n; ++j)
    SFP8_REQUIRE(fmts[j] == FP8_E4M3 || fmts[j] == FP8_E5M2, FP8_ERR_ARG, "fp8_recipe_update: fmts[%d]=%d", j,
                 fmts[j]);
  // 2^-margin as float32: exact for margin <= 126
  const float tpm = ldexpf(1.0f, -margin);
  hipStream_t st = (hipStream_t)stream;
  for (int slot0 = 0; slot0 < n; slot0 += kSlotsPerLaunch) {
    const int ns = (n - slot0) < kSlotsPerLaunch ? (n - slot0) : kSlotsPerLaunch;
    FmtBits fb;
    memset(&fb, 0, sizeof fb);
    for (int j = 0; j < ns; ++j)
      if (fmts[slot0 + j] == FP8_E5M2) fb.w[j >> 5] |= 1u << (j & 31);
    hipLaunchKernelGGL(recipe_update_kernel, dim3((ns + 255) / 256), dim3(256), 0, st, amax_history, scale, scale_inv,
                       n, slot0, ns, history_len, tpm, fb);
    int rc = check_launch("fp8_recipe_update");
    if (rc != FP8_OK) return rc;
  }
  return FP8_OK;
}
