// Shared device helpers and host error plumbing for the FP8 scaled-linear library (gfx950).
//
// FP8 encode on gfx950: v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 round to nearest even, keep
// subnormals and the sign of zero -- the encode the pages call for ("Week 14" course page,
// FP8 bullet and accumulation-precision bullet: ties go to even) -- for every input up to
// fmax in magnitude.  They do not saturate (E4M3 overflow gives NaN, E5M2 gives inf) and
// write NaN without its sign, so the cast is: clamp to [-fmax, fmax] with v_med3_f32
// (which also sends +-inf to +-fmax, the "clips at 448" rule of the "Transformer Scaling"
// lesson, Worked example 02), convert, and rewrite the byte of any NaN input as
// sign | 0x7F.  NaN inputs are rare; they are detected from the amax bits the kernels
// compute anyway, and patched on a per-lane slow path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/scaled_fp8.h"

namespace sfp8 {

// ------------------------------------------------------------------ host-side errors

int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int check_launch(const char* what);

#define SFP8_REQUIRE(cond, code, ...)        \
  do {                                       \
    if (!(cond)) return set_error((code), __VA_ARGS__); \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// compute units of the current device (256 on MI355X), asked once per device: for grids sized to
// the blocks that are resident at once
inline int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

// ------------------------------------------------------------------ device helpers

// 16-byte vector usable with the nontemporal (streaming) load/store builtins
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 u32x4_make(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return v;
}

template <int FMT>
struct Fp8Traits;
template <>
struct Fp8Traits<FP8_E4M3> {
  static constexpr float fmax = 448.0f;
  // amax <= 1.75 * 2^e  <=>  E = e - 8 (smallest E with amax <= 448 * 2^E)
  static constexpr int mx_bias = 8;
};
template <>
struct Fp8Traits<FP8_E5M2> {
  static constexpr float fmax = 57344.0f;
  static constexpr int mx_bias = 15;
};

// Two float32 values -> two FP8 codes in bytes (2*hi, 2*hi+1) of `old` (saturating).
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt_pair(float a, float b, uint32_t old) {
  constexpr float fm = Fp8Traits<FMT>::fmax;
  a = __builtin_amdgcn_fmed3f(a, -fm, fm);
  b = __builtin_amdgcn_fmed3f(b, -fm, fm);
  if constexpr (FMT == FP8_E4M3)
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
  else
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}

// Four float32 values -> one dword of four FP8 codes (byte i = value i).
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  uint32_t w = cvt_pair<FMT, false>(a, b, 0u);
  return cvt_pair<FMT, true>(c, d, w);
}

// NaN input bits -> its FP8 code (sign | 0x7F in both formats).
__device__ __forceinline__ uint32_t nan_code(uint32_t f32bits) { return ((f32bits >> 24) & 0x80u) | 0x7Fu; }

// Replace byte i of `w` by the NaN code of x_i wherever x_i is NaN.
__device__ __forceinline__ uint32_t patch_nan4(uint32_t w, const float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t b = __float_as_uint(x[i]);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) w = (w & ~(0xFFu << (8 * i))) | (nan_code(b) << (8 * i));
  }
  return w;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// |x| bits of a float: unsigned order of these bits is the order of |x|, and every NaN
// compares above +inf, so an unsigned max propagates NaN.
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// Lane exchanges on the DPP path (a VALU operand modifier, no LDS round trip): each lane reads
// its partner's value under a quad swap (lane ^ 1, lane ^ 2), a reversal of its 8-lane half-row
// or a reversal of its 16-lane row.  Every step of the reductions below combines a lane with a
// partner that in turn reads it, so all lanes of a group end with the same result.
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_partner(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Unsigned max over aligned groups of W lanes (W = 2, 4, 8, 16, 32, 64; result in every lane):
// DPP within a row of 16, lane shuffles across rows.
template <int W>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group of 2^k lanes");
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, dpp_partner<kDppQuadXor1>(v));
  if constexpr (W >= 4) v = mx(v, dpp_partner<kDppQuadXor2>(v));
  if constexpr (W >= 8) v = mx(v, dpp_partner<kDppHalfMirror>(v));
  if constexpr (W >= 16) v = mx(v, dpp_partner<kDppMirror>(v));
  if constexpr (W >= 32) v = mx(v, (uint32_t)__shfl_xor((int)v, 16, 64));
  if constexpr (W >= 64) v = mx(v, (uint32_t)__shfl_xor((int)v, 32, 64));
  return v;
}

// Unsigned max over the 64 lanes of a wave (result in every lane).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return group_max_u32<64>(v); }

// Current-scaling rule: s = fmax / amax (correctly rounded), overflow clamped to FLT_MAX;
// amax zero or not finite -> s = 1.  s_inv = 1 / s.
template <int FMT>
__device__ __forceinline__ void current_scale(uint32_t amax_bits, float& s, float& s_inv) {
  if (amax_bits == 0u || amax_bits >= 0x7F800000u) {
    s = 1.0f;
    s_inv = 1.0f;
    return;
  }
  float r = Fp8Traits<FMT>::fmax / __uint_as_float(amax_bits);
  s = fminf(r, 3.40282346638528859812e+38f);
  s_inv = 1.0f / s;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// two fp32 -> packed bf16 (a in the low half), round to nearest even, by gfx950's packed
// conversion instruction: the same finite results as f32_to_bf16_bits, NaN stays NaN (quiet)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const bf16x2_t h = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

}  // namespace sfp8
