// Element rules shared by the quantizers (quantize.hip) and the fused LayerNorm + cast
// (layernorm.hip): 8-element loads, the scaled saturating cast of 8 values, and the MX
// (e8m0) scale rule.
#pragma once

#include "common.h"

namespace sfp8 {

// ------------------------------------------------------------------ element loaders
//
// 8 consecutive elements: one 16-byte load for bf16, two for fp32 (nontemporal: each input
// is read once).
template <bool BF16>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t e0, float (&v)[8]) {
  if constexpr (BF16) {
    u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + e0));
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + e0);
    u32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
  }
}

// 8 values * s -> 8 codes (NaN inputs patched)
template <int FMT>
__device__ __forceinline__ u32x2 cast8(const float (&v)[8], float s, uint32_t amax_bits) {
  uint32_t w0 = cvt4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
  uint32_t w1 = cvt4<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
  if (amax_bits > 0x7F800000u) {
    w0 = patch_nan4(w0, &v[0]);
    w1 = patch_nan4(w1, &v[4]);
  }
  return u32x2{w0, w1};
}

// MX 1x32 scale rule: E = the smallest integer with amax <= fmax * 2^E (from amax's exponent
// and mantissa), clamped to [-127, 127]; zero amax -> -127; non-finite amax -> code 255 and
// multiplier 1.  code = E + 127 (e8m0), mult = 2^-E (exact).
template <int FMT>
__device__ __forceinline__ void mx_rule(uint32_t amax_bits, uint32_t& code, float& mult) {
  if (amax_bits >= 0x7F800000u) {
    code = 255u;
    mult = 1.0f;
    return;
  }
  int E;
  const int ef = (int)(amax_bits >> 23);
  if (ef == 0) {
    E = -127;  // zero or subnormal amax: the smallest E already exceeds it
  } else {
    const int e = ef - 127;
    E = e - Fp8Traits<FMT>::mx_bias + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    E = E < -127 ? -127 : (E > 127 ? 127 : E);
  }
  code = (uint32_t)(E + 127);
  // E <= 120 for every finite amax, so 2^-E is a normal float: exponent field 127 - E
  mult = __uint_as_float((uint32_t)(127 - E) << 23);
}

}  // namespace sfp8
