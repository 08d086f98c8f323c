// GEMM epilogues: what a tile's dequantised fp32 results go through on their way to memory.
//
// Plain (fp8_gemm): C = the result, stored as fp32 or bf16 (round to nearest even; "Week 14"
// course page, precision paragraph).
//
// Fused (fp8_gemm_fused), in this order per element, all in fp32:
//   1. + bias[n]  (a Linear with a bias: the Transformer Engine tutorial's te.Linear(bias=True)
//      in its module tour cell);
//   2. optional copy of the pre-activation value to `aux` as bf16 (what an activation's
//      backward needs);
//   3. activation: GELU in its exact form x * Phi(x) (the tutorial's plain-PyTorch block puts
//      nn.GELU between the MLP's two linears), or SwiGLU silu(g) * u (the course page's MoE
//      exercise sizes a SwiGLU expert at 3 D F parameters: gate, up and down projections),
//      with the gate and up rows of B interleaved (B row 2f is gate unit f, row 2f+1 its up
//      unit), so that both halves of an output land in the same lane;
//   4. output as fp32, bf16, or FP8 for the next layer's input: code = enc(fp32(y * scale))
//      with the saturating round-to-nearest-even cast of the quantizers, and the output's amax
//      max-reduced into an amax slot for the delayed recipe ("Transformer Scaling" lesson,
//      Part 01: each tensor's amax is recorded every step).
//
// The kernels run their store loop inside with_act(), which calls it with the activation as a
// compile-time constant (a runtime test inside the unrolled loop let the compiler evaluate
// the GELU of every element whatever the activation, and select), and call, per lane, for
// runs of W adjacent columns gn .. gn+W-1 (gn % W == 0) of one row gm:  pre() (bias), aux(),
// out<ACT>();  and finish() once at the end (amax reduction).  `full` means all W columns
// exist and a W-wide vector store is aligned (N % W == 0).
#pragma once

#include <type_traits>

#include "common.h"

namespace sfp8 {

// output element types of the GEMM kernels (the public OUT_* values)
enum { EPI_F32 = OUT_F32, EPI_BF16 = OUT_BF16, EPI_E4M3 = OUT_E4M3, EPI_E5M2 = OUT_E5M2 };

struct EpiParams {
  void* C;               // [M][ldc] output, ldc = N (N / 2 for SwiGLU)
  const void* bias;      // fused: [N] fp32 or bf16, or null
  void* aux;             // fused: bf16 [M][N] pre-activation copy, or null
  const float* c_scale;  // FP8 output: the scale (device scalar)
  float* c_amax;         // FP8 output: amax slot (max-reduced into)
  int bias_bf16;         // bias element type is bf16
  int act;               // FP8_ACT_*
};

// GELU, exact form x Phi(x), with erfc from Abramowitz & Stegun 7.1.26 (Hastings' rational
// approximation): for z >= 0, erfc(z) = (a1 t + a2 t^2 + ... + a5 t^5) e^(-z^2) with
// t = 1 / (1 + p z) and |error| <= 1.5e-7.  Phi(x) = erfc(|x| / sqrt 2) / 2 for x < 0 (no
// cancellation) and 1 - that for x >= 0, so |gelu error| <= ~1e-7 |x| beyond the fp32
// rounding of the ~16 operations; the library erfcf costs several times more, and the
// epilogue runs while the matrix cores idle.
__device__ __forceinline__ float gelu_exact(float x) {
  constexpr float p = 0.3275911f, a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f,
                  a4 = -1.453152027f, a5 = 1.061405429f;
  const float z = fabsf(x) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(fmaf(p, z, 1.0f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  // e^(-z^2) = 2^(-z^2 log2 e); v_exp_f32 underflows to 0 for z > ~9.3, where Phi is 0 or 1
  const float tail = 0.5f * poly * __builtin_amdgcn_exp2f(-z * z * 1.44269504088896341f);
  return x * (x < 0.0f ? tail : 1.0f - tail);
}

// silu(g) u = g sigmoid(g) u with sigmoid = 1 / (1 + 2^(-g log2 e)) (hardware exp2 and
// reciprocal, a few ulp); g -> -inf gives 2^inf = inf and sigmoid 0
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896341f)) * u;
}

template <int OUT, bool FUSED>
struct Epilogue {
  static constexpr bool kFp8 = OUT == EPI_E4M3 || OUT == EPI_E5M2;
  static constexpr int kFmt = OUT == EPI_E5M2 ? FP8_E5M2 : FP8_E4M3;
  const EpiParams p;
  float cs;            // output scale (FP8)
  uint32_t amax_bits;  // running max of |output| bits (FP8)

  __device__ explicit Epilogue(const EpiParams& params) : p(params), cs(1.0f), amax_bits(0u) {
    if constexpr (kFp8) cs = *p.c_scale;
  }

  // f(integral_constant<int, ACT>) with the launch's activation
  template <class F>
  __device__ __forceinline__ void with_act(F&& f) const {
    if constexpr (FUSED) {
      if (p.act == FP8_ACT_GELU) {
        f(std::integral_constant<int, FP8_ACT_GELU>{});
        return;
      }
      if (p.act == FP8_ACT_SWIGLU) {
        f(std::integral_constant<int, FP8_ACT_SWIGLU>{});
        return;
      }
    }
    f(std::integral_constant<int, FP8_ACT_NONE>{});
  }

  // bias[gn + i] for i < W (0 where absent)
  template <int W>
  __device__ __forceinline__ void bias(int gn, int N, float (&b)[W]) const {
#pragma unroll
    for (int i = 0; i < W; ++i) b[i] = 0.0f;
    if constexpr (FUSED) {
      if (p.bias == nullptr) return;
#pragma unroll
      for (int i = 0; i < W; ++i)
        if (gn + i < N)
          b[i] = p.bias_bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(p.bias)[gn + i] << 16)
                             : static_cast<const float*>(p.bias)[gn + i];
    }
  }

  template <int W>
  __device__ __forceinline__ void pre(float (&v)[W], const float (&b)[W]) const {
    if constexpr (FUSED) {
      if (p.bias == nullptr) return;  // no +0 added: -0 results stay -0
#pragma unroll
      for (int i = 0; i < W; ++i) v[i] += b[i];
    }
  }

  // bf16 copy of the pre-activation values, row pitch N
  template <int W>
  __device__ __forceinline__ void aux(const float (&v)[W], int gm, int gn, int N, bool full) const {
    if constexpr (FUSED) {
      if (p.aux == nullptr) return;
      store_run<EPI_BF16, W>(p.aux, (size_t)gm * N + gn, v, full, N - gn);
    }
  }

  // activation and the output store
  template <int ACT, int W>
  __device__ __forceinline__ void out(float (&v)[W], int gm, int gn, int N, bool full) {
    if constexpr (ACT == FP8_ACT_SWIGLU) {
      static_assert(W % 2 == 0, "SwiGLU needs column pairs");
      float o[W / 2];
#pragma unroll
      for (int i = 0; i < W / 2; ++i) o[i] = swiglu(v[2 * i], v[2 * i + 1]);
      // output column gn/2 + i exists iff its up column gn + 2i + 1 does
      emit<W / 2>(o, (size_t)gm * (N / 2) + gn / 2, full, (N - gn) / 2);
    } else {
      if constexpr (ACT == FP8_ACT_GELU) {
#pragma unroll
        for (int i = 0; i < W; ++i) v[i] = gelu_exact(v[i]);
      }
      emit<W>(v, (size_t)gm * N + gn, full, N - gn);
    }
  }

  // every thread of the block, after its stores: fold the block's amax into the slot with one
  // atomic (one per wave measured ~8% of a 8192 x 14336 x 4096 GEMM: same-address atomics
  // from every CU serialise).  `red` = LDS for one word per wave; the first barrier makes
  // sure no wave still reads the tile stages there.
  __device__ __forceinline__ void finish(int lane, uint32_t* red) const {
    if constexpr (kFp8) {
      const uint32_t m = wave_max_u32(amax_bits);
      const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
      __syncthreads();
      if (lane == 0) red[wave] = m;
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t r = red[0];
        for (int i = 1; i < nw; ++i) r = r > red[i] ? r : red[i];
        unsigned int* slot = reinterpret_cast<unsigned int*>(p.c_amax);
        // a plain read first: most blocks do not raise the running maximum
        if (r > __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(slot, r);
      }
    }
  }

 private:
  // W values to element offset `at` of the output; `avail` = how many of them exist
  template <int W>
  __device__ __forceinline__ void emit(const float (&v)[W], size_t at, bool full, int avail) {
    bool nan_here = false;
    if constexpr (kFp8) {
      uint32_t m = 0u;
#pragma unroll
      for (int i = 0; i < W; ++i)
        if (full || i < avail) m = m > abs_bits(v[i]) ? m : abs_bits(v[i]);
      amax_bits = amax_bits > m ? amax_bits : m;
      nan_here = m > 0x7F800000u;
    }
    store_run<OUT, W>(p.C, at, v, full, avail, nan_here);
  }

  template <int T, int W>
  __device__ __forceinline__ void store_run(void* base, size_t at, const float (&v)[W], bool full, int avail,
                                            bool nan_here = false) const {
    if constexpr (T == EPI_F32) {
      float* c = static_cast<float*>(base) + at;
      if (full && W == 4) {
        const u32x4 w = u32x4_make(__float_as_uint(v[0]), __float_as_uint(v[W > 1 ? 1 : 0]),
                                   __float_as_uint(v[W > 2 ? 2 : 0]), __float_as_uint(v[W > 3 ? 3 : 0]));
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(c));
      } else if (full && W == 2) {
        const u32x2 w = {__float_as_uint(v[0]), __float_as_uint(v[W > 1 ? 1 : 0])};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(c));
      } else {
#pragma unroll
        for (int i = 0; i < W; ++i)
          if (full || i < avail) c[i] = v[i];
      }
    } else if constexpr (T == EPI_BF16) {
      uint16_t* c = static_cast<uint16_t*>(base) + at;
      if (full && W == 4) {
        const u32x2 w = {f32x2_to_bf16x2(v[0], v[W > 1 ? 1 : 0]), f32x2_to_bf16x2(v[W > 2 ? 2 : 0], v[W > 3 ? 3 : 0])};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(c));
      } else if (full && W == 2) {
        __builtin_nontemporal_store(f32x2_to_bf16x2(v[0], v[W > 1 ? 1 : 0]), reinterpret_cast<uint32_t*>(c));
      } else {
        uint32_t b[W];
#pragma unroll
        for (int i = 0; i < W; ++i) b[i] = f32_to_bf16_bits(v[i]);
#pragma unroll
        for (int i = 0; i < W; ++i)
          if (full || i < avail) c[i] = (uint16_t)b[i];
      }
    } else {
      uint8_t* c = static_cast<uint8_t*>(base) + at;
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = i < W ? v[i < W ? i : 0] * cs : 0.0f;
      uint32_t w;
      if constexpr (W == 4) w = cvt4<kFmt>(x[0], x[1], x[2], x[3]);
      else w = cvt_pair<kFmt, false>(x[0], x[1], 0u);
      if (nan_here) w = patch_nan4(w, x);  // rare: NaN results
      if (full && W == 4) {
        __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(c));
      } else if (full && W == 2) {
        __builtin_nontemporal_store((uint16_t)w, reinterpret_cast<uint16_t*>(c));
      } else {
#pragma unroll
        for (int i = 0; i < W; ++i)
          if (full || i < avail) c[i] = (uint8_t)(w >> (8 * i));
      }
    }
  }
};

}  // namespace sfp8
