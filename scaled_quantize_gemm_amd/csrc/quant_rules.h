// Element rules shared by the quantizers (quantize.hip), the cast-transposes
// (cast_transpose.hip) and the fused LayerNorm + cast (layernorm.hip): 8-element loads, packed
// 8-element runs, the scaled saturating cast of 8 values, and the MX (e8m0) scale rule.
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

// ------------------------------------------------------------------ packed 8-element runs
//
// 8 consecutive elements kept as loaded (bf16: one 16-byte word quad; fp32: two), widened to
// fp32 only where arithmetic needs them.  A kernel that holds its tile in registers across a
// barrier needs half the registers for bf16 this way.  The amax works on the bit patterns:
// |x| as an unsigned integer orders like the value, and NaN sorts above every finite value.
template <bool BF16>
struct Raw8 {
  u32x4 w[BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ Raw8<BF16> load_raw8(const void* __restrict__ x, int64_t e0) {
  Raw8<BF16> r;
  if constexpr (BF16) {
    r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + e0));
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + e0);
    r.w[0] = __builtin_nontemporal_load(p);
    r.w[1] = __builtin_nontemporal_load(p + 1);
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ Raw8<BF16> zero_raw8() {
  Raw8<BF16> r;
#pragma unroll
  for (int i = 0; i < (BF16 ? 1 : 2); ++i) r.w[i] = u32x4{0u, 0u, 0u, 0u};
  return r;
}

// word i: bf16 elements 2i and 2i+1 (i < 4), or fp32 element i (i < 8)
template <bool BF16>
__device__ __forceinline__ uint32_t raw_word(const Raw8<BF16>& r, int i) {
  const u32x4& q = r.w[i >> 2];
  const int j = i & 3;
  return j == 0 ? q.x : (j == 1 ? q.y : (j == 2 ? q.z : q.w));
}

// fp32 bits of |element e|
template <bool BF16>
__device__ __forceinline__ uint32_t raw_abs_bits(const Raw8<BF16>& r, int e) {
  if constexpr (BF16) {
    const uint32_t w = raw_word<BF16>(r, e >> 1);
    return (((e & 1) ? (w >> 16) : w) & 0x7FFFu) << 16;
  } else {
    return raw_word<BF16>(r, e) & 0x7FFFFFFFu;
  }
}

// fp32 bits of the largest |element|
template <bool BF16>
__device__ __forceinline__ uint32_t raw_amax_bits(const Raw8<BF16>& r) {
  uint32_t m = 0;
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a = raw_word<BF16>(r, i) & 0x7FFF7FFFu;
      const uint32_t lo = a & 0xFFFFu, hi = a >> 16;
      m = m > lo ? m : lo;
      m = m > hi ? m : hi;
    }
    return m << 16;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = raw_word<BF16>(r, i) & 0x7FFFFFFFu;
      m = m > a ? m : a;
    }
    return m;
  }
}

// the words pass through an empty asm: nothing computed from them before this point (the
// amax's masked halves equal the widened values' bits) is reused after it, so the compiler
// cannot keep a widened copy of the tile live across a barrier
template <bool BF16>
__device__ __forceinline__ void opaque_raw8(Raw8<BF16>& r) {
#pragma unroll
  for (int i = 0; i < (BF16 ? 1 : 2); ++i) asm volatile("" : "+v"(r.w[i]));
}

template <bool BF16>
__device__ __forceinline__ void widen8(const Raw8<BF16>& r, float (&v)[8]) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = raw_word<BF16>(r, i);
      v[2 * i] = bf16_lo(w);
      v[2 * i + 1] = bf16_hi(w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(raw_word<BF16>(r, i));
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
