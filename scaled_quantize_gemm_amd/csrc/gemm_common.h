// Definitions shared by the GEMM kernels (gemm_small.h, gemm_w4.h, gemm_blk.h): operand vector
// types, the scaling modes, inline LDS reads with immediate offsets, compile-time unrolling, and
// the XCD-aware order in which the large-tile kernels walk their tiles.
#pragma once

#include <type_traits>
#include <utility>

#include "common.h"
#include "gemm_epilogue.h"

namespace sfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum { MODE_TENSOR = 0, MODE_BLOCK = 1, MODE_MX = 2, MODE_TILE2 = 3 };
typedef float v16f __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// buffer resource word 3 for raw byte-addressed buffers on gfx9 (32-bit data format, no swizzle)
constexpr int kBufferFlags = 0x00020000;

// Tile order: workgroups are dealt round-robin to the 8 XCDs (each with its own L2), so
// block b runs on XCD b % 8; each XCD gets a contiguous range of tiles, walked in groups of
// 4 tile-rows so that the tiles resident on one XCD share A rows and B columns.
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int xcd = b & 7, idx = b >> 3;
  const int per = T >> 3, rem = T & 7;
  const int t = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  constexpr int GM = 4;
  const int group = t / (GM * tiles_n);
  const int first = group * GM;
  const int gsz = (tiles_m - first) < GM ? (tiles_m - first) : GM;
  const int in = t - group * GM * tiles_n;
  tm = first + in % gsz;
  tn = in / gsz;
}

template <int OFF>
__device__ __forceinline__ u32x4 ds_read16(uint32_t vaddr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field is 16 bits");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(vaddr), "i"(OFF) : "memory");
  return v;
}
template <int OFF>
__device__ __forceinline__ uint32_t ds_read4(uint32_t vaddr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field is 16 bits");
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(vaddr), "i"(OFF) : "memory");
  return v;
}
template <int OFF>
__device__ __forceinline__ uint32_t ds_read2(uint32_t vaddr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field is 16 bits");
  uint32_t v;
  asm volatile("ds_read_u16 %0, %1 offset:%2" : "=v"(v) : "v"(vaddr), "i"(OFF) : "memory");
  return v;
}

// compile-time unrolling: f(integral_constant<int, I>) for I = 0 .. N-1
template <typename F, int... Is>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}


}  // namespace sfp8
