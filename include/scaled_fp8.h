/*
 * scaled_fp8.h -- C ABI of the FP8 scaled linear layer hot path for AMD Instinct MI355X (gfx950).
 *
 * The path: amax -> scale derivation -> saturating round-to-nearest-even cast to FP8
 * (plus cast-transpose) -> FP8 x FP8 GEMM with fp32 promotion -> dequantising epilogue.
 *
 * Sources (web pages; cited by title and section):
 *   [L]  "Transformer Scaling" lesson reading, lab.mindcaptain.ai/reading/06
 *        (Concept deep dive 01; Part 01; Core vocabulary; Worked example 01-02).
 *   [W]  "Week 14. Scaling laws, precision, parallelism", snula.amonoc.com/course/en/week-14.html
 *        (precision paragraph; absmax paragraph and bullet; FP8 bullet; accumulation-precision bullet).
 *   [T]  Transformer Engine fused-kernels tutorial, juicytalk.now (DelayedScaling recipe cell;
 *        FP8 metadata readback cell; capability check cell).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is DEVICE memory owned by the caller (e.g. a torch tensor's
 *    data_ptr()).  The library allocates nothing, frees nothing and keeps no state
 *    between calls apart from the thread-local error text.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls validate
 *    their arguments on the host, enqueue kernels on `stream` and return without
 *    synchronising.  Buffers must stay valid until the stream has passed this work.
 *  - All matrices are row-major and contiguous.  Data pointers must be 16-byte aligned;
 *    scale / amax pointers 4-byte aligned.
 *  - Return value: FP8_OK, or a negative FP8_ERR_* code with nothing enqueued (argument
 *    errors) or with the launch error recorded (FP8_ERR_LAUNCH).  fp8_last_error()
 *    returns the text for the calling thread's last non-OK status.  Device faults
 *    surface at the caller's next synchronisation, as for any HIP work.
 *  - Empty inputs (rows * cols == 0, or M * N == 0) are valid and enqueue nothing.
 */
#ifndef SCALED_FP8_H
#define SCALED_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* FP8 formats ([L] Concept deep dive 01; [W] FP8 bullet): OCP E4M3 (4 exponent, 3 mantissa
 * bits, max 448, no infinity, S.1111.111 = NaN) and OCP E5M2 (5 + 2 bits, max 57344). */
enum { FP8_E4M3 = 0, FP8_E5M2 = 1 };

/* High-precision input element types. */
enum { HP_F32 = 0, HP_BF16 = 1 };

/* GEMM output element types ([W] precision paragraph: bf16 rounds to nearest even).
 * OUT_E4M3 / OUT_E5M2 (FP8 codes, the next layer's input) are fp8_gemm_fused only. */
enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_E4M3 = 2, OUT_E5M2 = 3 };

/* Activations of the fused GEMM epilogue (fp8_gemm_fused). */
enum { FP8_ACT_NONE = 0, FP8_ACT_GELU = 1, FP8_ACT_SWIGLU = 2 };

/* Scale granularities ([W] absmax bullet: per tensor, per block; MX: one scale per 32
 * numbers; DeepSeek-V3: per 128 activation values and per 128x128 weight block). */
enum {
  FP8_SCALE_TENSOR = 0,        /* one fp32 scale per tensor (delayed scaling)            */
  FP8_SCALE_TILE_1x128 = 1,    /* one fp32 scale per 1x128 run along the column axis     */
  FP8_SCALE_BLOCK_128x128 = 2, /* one fp32 scale per 128x128 block                       */
  FP8_SCALE_MX_1x32 = 3        /* one e8m0 power-of-two scale per 1x32 run along columns */
};

/* amax_compute_algo of the delayed recipe ([T] DelayedScaling(amax_compute_algo="max")). */
enum { FP8_AMAX_ALGO_MAX = 0 };

enum {
  FP8_OK = 0,
  FP8_ERR_ARG = -1,    /* null pointer, bad enum, misaligned pointer, bad combination */
  FP8_ERR_SHAPE = -2,  /* negative size or a size the granularity cannot tile        */
  FP8_ERR_DTYPE = -3,  /* unsupported element type                                   */
  FP8_ERR_DEVICE = -4, /* no HIP device, or the device is not gfx950                 */
  FP8_ERR_LAUNCH = -5  /* the kernel launch failed                                   */
};

/*
 * fp8_device_check -- is `device` able to run this library?
 *   Mirrors the tutorial's FP8 capability check ([T] capability check cell: the FP8 path
 *   needs hardware FP8 matrix units; the check returns ok plus a reason).  Returns FP8_OK
 *   iff the device exists and is gfx950 (MI350 series).  Otherwise FP8_ERR_DEVICE; there
 *   is no fallback.  `reason` (may be NULL) receives a NUL-terminated description,
 *   truncated to `reason_len` bytes.
 */
int fp8_device_check(int device, char *reason, size_t reason_len);

/*
 * fp8_recipe_update -- end-of-step update of the delayed-scaling recipe state.
 *   [L] Part 01 and Core vocabulary: delayed scaling derives the scale from the amax
 *   history, avoiding an extra pre-quantisation read at the price of lag; [L] Worked
 *   example 01: scale = fmax / amax; [T] DelayedScaling(amax_history_len, "max") and the
 *   readback amax_history[0, :4] (history-major layout).
 *
 *   amax_history  device fp32 [history_len][n]  (row 0 = the current step, filled by
 *                 fp8_quantize / fp8_cast_transpose through their amax_slot pointers)
 *   scale         device fp32 [n]               multiplier used by the casts
 *   scale_inv     device fp32 [n]               = 1 / scale, used by fp8_gemm
 *   fmts          HOST int [n]                  FP8_E4M3 / FP8_E5M2 per slot (its fmax)
 *   algo          FP8_AMAX_ALGO_MAX (the only algorithm)
 *   margin        scale is multiplied by 2^-margin (0 <= margin <= 64)
 *
 *   Per slot j: m = max_i amax_history[i][j].  If m is finite and > 0:
 *   scale[j] = fp32(fp32(fmax / m) * 2^-margin) (overflow clamped to FLT_MAX) and
 *   scale_inv[j] = fp32(1 / scale[j]); otherwise both are kept.  Then the ring rolls:
 *   row i <- row i+1, last row <- old row 0, and row 0 <- 0.
 *   Initial state expected by the protocol: history 0, scale = scale_inv = 1.
 *   Errors: FP8_ERR_ARG (null pointer, n < 1, history_len < 1, bad fmt/algo/margin).
 */
int fp8_recipe_update(float *amax_history, float *scale, float *scale_inv, const int *fmts,
                      int n, int history_len, int algo, int margin, void *stream);

/*
 * fp8_quantize -- fused amax + scale + saturating RNE cast of a [rows][cols] tensor.
 *   [L] Part 01 (a scale maps values into the FP8 range; too small saturates) and Worked
 *   example 02 (a value beyond the range clips at 448); [W] absmax bullet (per-tensor,
 *   per-block and 32-element MX scales; DeepSeek-V3 1x128 / 128x128 blocks computed online);
 *   [L] Core vocabulary (amax).
 *
 *   x          device, x_dtype HP_F32 or HP_BF16, [rows][cols]
 *   q          device uint8 [rows][cols]: q = enc_fmt(fp32(x * s)), round to nearest even,
 *              saturating to +-fmax (+-inf too); NaN -> sign | 0x7F; signed zero kept.
 *   granularity:
 *     FP8_SCALE_TENSOR:   s = *scale (device fp32 scalar, the recipe's current scale).
 *                         If amax_slot != NULL, max(|x|) is max-ed atomically into
 *                         *amax_slot (= &amax_history[0][slot]); NaN propagates.
 *                         scale_inv_out must be NULL.  Any rows, cols.
 *     FP8_SCALE_TILE_1x128: per 1x128 run (cols % 128 == 0): s = fmax / amax_run
 *                         (zero or non-finite amax -> 1; overflow -> FLT_MAX);
 *                         scale_inv_out = device fp32 [cols/128][rows] of 1 / s.
 *     FP8_SCALE_BLOCK_128x128: per 128x128 block (cols % 128 == 0; a partial last
 *                         row-block uses the rows present), same rule;
 *                         scale_inv_out = device fp32 [ceil(rows/128)][cols/128].
 *     FP8_SCALE_MX_1x32:  per 1x32 run (cols % 32 == 0): E = smallest integer with
 *                         amax_run <= fmax * 2^E, clamped to [-127, 127]; elements are
 *                         multiplied by 2^-E exactly; scale_inv_out = device uint8
 *                         [cols/32][rows] of e8m0 codes E + 127 (255 if amax is not finite),
 *                         run-column major like the 1x128 scales, so one K block's scales
 *                         for consecutive rows are contiguous.
 *     For TILE / BLOCK / MX, scale and amax_slot must be NULL.
 *   Errors: FP8_ERR_ARG, FP8_ERR_SHAPE (cols not a multiple of the run), FP8_ERR_DTYPE.
 */
int fp8_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int fmt,
                 int granularity, const float *scale, float *amax_slot, uint8_t *q,
                 void *scale_inv_out, void *stream);

/*
 * fp8_quantize_diag -- fp8_quantize(FP8_SCALE_TENSOR) plus cast diagnostics in the same pass.
 *   [L] Diagnostic playbook (FP8 loss spikes or NaN: inspect per-layer amax and overflow
 *   counts) and Worked example 02 (with a stale delayed scale, a spike clips at 448).
 *
 *   Same arguments, element rule and amax as fp8_quantize with FP8_SCALE_TENSOR, plus
 *   counts     device uint64 [3], 8-byte aligned; the call ADDS (the caller zeroes them):
 *                counts[0]  saturated:   elements with |fp32(x * s)| > fmax (the code was
 *                                        clipped to +-fmax; +-inf inputs included)
 *                counts[1]  underflowed: finite non-zero elements whose code is +-0
 *                counts[2]  nan:         NaN elements
 *   Errors: as fp8_quantize; FP8_ERR_ARG also for a null or misaligned counts.
 */
int fp8_quantize_diag(const void *x, int x_dtype, int64_t rows, int64_t cols, int fmt,
                      const float *scale, float *amax_slot, uint8_t *q,
                      unsigned long long *counts, void *stream);

/*
 * fp8_cast_transpose -- per-tensor cast plus its transpose in one pass (+ amax).
 *   The backward pass of the hybrid recipe ([L] Part 01: E4M3 forward, E5M2 gradients;
 *   [W] FP8 bullet) multiplies by transposed operands; producing the transposed FP8 copy
 *   during the cast keeps every GEMM in the K-contiguous (TN) form.
 *
 *   Same arguments and element rule as fp8_quantize(FP8_SCALE_TENSOR); additionally
 *   qT = device uint8 [cols][rows] with qT[c][r] = q[r][c].  Any rows, cols.
 */
int fp8_cast_transpose(const void *x, int x_dtype, int64_t rows, int64_t cols, int fmt,
                       const float *scale, float *amax_slot, uint8_t *q, uint8_t *qT,
                       void *stream);

/*
 * fp8_cast_transpose_blockwise -- current-scaling cast plus its transpose in one pass, each
 *   copy with the scales its backward GEMM needs.
 *   [W] absmax bullet (DeepSeek-V3: scales per 128 activation values and per 128x128 weight
 *   block, computed from the current block); the backward GEMMs multiply by transposed
 *   operands, and keeping them K-contiguous (TN) means the transposed copy needs runs along
 *   its own K (the source's rows).
 *
 *   x             device, x_dtype HP_F32 or HP_BF16, [rows][cols]
 *   granularity   FP8_SCALE_TILE_1x128 or FP8_SCALE_BLOCK_128x128
 *   q             device uint8 [rows][cols]
 *   qT            device uint8 [cols][rows]
 *   TILE_1x128:   q exactly as fp8_quantize(TILE_1x128): one scale per 1x128 run of a row,
 *                 q_scale_inv = fp32 [cols/128][rows];
 *                 qT = the codes of x^T with one scale per 1x128 run of x^T's rows (a 128x1
 *                 run of a source column), qT_scale_inv = fp32 [rows/128][cols]
 *                 (for wgrad: dW = dY^T X with A = dY^T, B = X^T, both TILE_1x128).
 *   BLOCK_128x128: q exactly as fp8_quantize(BLOCK_128x128), q_scale_inv = fp32
 *                 [rows/128][cols/128]; qT[c][r] = q[r][c] and qT_scale_inv = fp32
 *                 [cols/128][rows/128], its transpose (for dgrad: dX = dY W with B = W^T).
 *   Element rule as fp8_quantize (s = fmax / amax of the run or block, zero or non-finite
 *   amax -> 1, one fp32 multiply, saturating RNE cast, NaN -> sign | 0x7F).
 *   rows % 128 == 0 and cols % 128 == 0.  Empty inputs are a no-op.
 *   Alignment: x, q, qT 16-byte aligned; scale arrays 4-byte aligned.
 *   Errors: FP8_ERR_ARG (null pointer, bad enum, misalignment), FP8_ERR_SHAPE (rows or cols
 *           not a multiple of 128), FP8_ERR_DTYPE (x_dtype).
 */
int fp8_cast_transpose_blockwise(const void *x, int x_dtype, int64_t rows, int64_t cols, int fmt,
                                 int granularity, uint8_t *q, float *q_scale_inv, uint8_t *qT,
                                 float *qT_scale_inv, void *stream);

/*
 * fp8_layernorm_quantize -- LayerNorm whose output goes straight to FP8 (no high-precision
 *   copy of it is written).
 *   [T] module tour cell (te.LayerNorm; te.LayerNormLinear and te.LayerNormMLP feed the norm
 *   into the FP8 linear) and plain-PyTorch block cell (nn.LayerNorm before attention and the
 *   MLP); [L] Part 01 and [W] absmax bullet for the scales, as fp8_quantize.
 *
 *   x          device, x_dtype HP_F32 or HP_BF16, [rows][cols]
 *   gamma      device, w_dtype HP_F32 or HP_BF16, [cols]; beta the same or NULL (no shift)
 *   eps        >= 0 (nn.LayerNorm's default is 1e-5)
 *   Per row, in fp32: mean = sum(x) / cols; var = sum((x - mean)^2) / cols (biased);
 *   rs = 1 / sqrt(var + eps); y = (x - mean) * rs * gamma + beta.
 *   y is then cast exactly as fp8_quantize casts an input at `granularity`:
 *     FP8_SCALE_TENSOR:   codes = enc(fp32(y * scale[0])); amax_slot (may be NULL) max-reduced
 *                         with max |y|; scale_inv_out unused.
 *     FP8_SCALE_TILE_1x128: per 1x128 run of y, s = fmax / amax; scale_inv_out = fp32
 *                         [cols/128][rows].
 *     FP8_SCALE_MX_1x32:  per 1x32 run, e8m0 code and 2^-E; scale_inv_out = uint8
 *                         [cols/32][rows].
 *   q          device uint8 [rows][cols]
 *   mu, rsigma device fp32 [rows] (the row's mean and rs, for the backward), or NULL.
 *   cols % 8 == 0 (TENSOR), % 128 (TILE_1x128), % 32 (MX_1x32); cols <= 8192.
 *   Alignment: x, q, gamma, beta 16-byte aligned; scale, amax_slot, fp32 scales, mu, rsigma
 *   4-byte aligned.  Empty inputs are a no-op.
 *   Errors: FP8_ERR_ARG (null pointer, bad enum or granularity BLOCK_128x128, misalignment,
 *           eps < 0), FP8_ERR_SHAPE (cols not a multiple of the run, cols > 8192),
 *           FP8_ERR_DTYPE (x_dtype, w_dtype).
 */
int fp8_layernorm_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols,
                           const void *gamma, const void *beta, int w_dtype, float eps, int fmt,
                           int granularity, const float *scale, float *amax_slot, uint8_t *q,
                           void *scale_inv_out, float *mu, float *rsigma, void *stream);

/*
 * fp8_gemm -- C[M][N] = sum_k deq(A[m][k]) * deq(B[n][k])  (C = A . B^T, Y = X W^T).
 *   [W] FP8 bullet (matmuls run in FP8) and accumulation-precision bullet (FP8 products are
 *   summed in a wider accumulator and partial sums are promoted to fp32 at fixed
 *   intervals); [W] precision paragraph (bf16 output rounds to nearest even).
 *
 *   A          device uint8 [M][K] FP8 codes in fmt_a;  B device uint8 [N][K] in fmt_b.
 *   Pairs of granularities and their scale arguments:
 *     TENSOR x TENSOR:   a_scale_inv, b_scale_inv = device fp32 scalars (scale_inv of
 *                        the recipe slots); C = acc * (sa * sb).
 *     TILE_1x128 x BLOCK_128x128: a_scale_inv = fp32 [K/128][M], b_scale_inv = fp32
 *                        [ceil(N/128)][K/128]; each 128-long K block's partial sum is
 *                        multiplied by sa[kb][m] * sb[n/128][kb] and added to an fp32
 *                        accumulator (promotion every 128 K).
 *     TILE_1x128 x TILE_1x128: a_scale_inv = fp32 [K/128][M], b_scale_inv = fp32 [K/128][N];
 *                        each K block's partial sum is multiplied by sa[kb][m] * sb[kb][n]
 *                        (the blockwise wgrad, both operands activation-style runs).
 *     MX_1x32 x MX_1x32: a_scale_inv = uint8 e8m0 [K/32][M], b_scale_inv = uint8 e8m0
 *                        [K/32][N] (as fp8_quantize writes them); the matrix cores apply
 *                        2^(ea - 127) * 2^(eb - 127) per 32-long run.
 *   Products are exact; the matrix cores sum runs of 8 products in a fixed-point window
 *   below the run's largest product and promote every run into fp32.
 *   C          device, c_dtype OUT_F32 or OUT_BF16 (round to nearest even), [M][N].
 *   K % 128 == 0 (pad K with zero codes); M, N >= 0 arbitrary; K == 0 gives C = 0.
 *   Errors: FP8_ERR_ARG (null pointer, bad enum, unsupported granularity pair),
 *           FP8_ERR_SHAPE (K % 128 != 0, negative sizes), FP8_ERR_DTYPE (c_dtype).
 */
int fp8_gemm(const uint8_t *A, int fmt_a, const void *a_scale_inv, int gran_a,
             const uint8_t *B, int fmt_b, const void *b_scale_inv, int gran_b, void *C,
             int c_dtype, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * fp8_gemm_fused -- fp8_gemm with the step after the GEMM fused into its epilogue.
 *   [T] module tour cell (te.Linear(bias=True): Y = X W^T + b) and plain-PyTorch block cell
 *   (nn.GELU between the MLP's linears: the exact form x * Phi(x)); [W] MoE exercise (a
 *   SwiGLU expert: silu(x Wg^T) * (x Wu^T)); [L] Part 01 (the amax of every FP8 tensor is
 *   recorded each step, here the output's, for the next layer's delayed scale).
 *
 *   A, B, scales, granularities, M, N, K: as fp8_gemm (N = the pre-activation width), except
 *   that B must be E4M3 (B is a weight, or an activation for wgrad: E4M3 in every recipe of
 *   [W] FP8 bullet); A may be E4M3 or E5M2.
 *   Per output element, in fp32, in this order:
 *     v = the dequantised GEMM result (exactly fp8_gemm's fp32 value)
 *     v = v + bias[n]             if bias != NULL (bias_dtype HP_F32 or HP_BF16, [N])
 *     aux[m][n] = bf16(v)         if aux != NULL (bf16 [M][N], round to nearest even)
 *     act = FP8_ACT_NONE:   y[m][n] = v
 *           FP8_ACT_GELU:   y[m][n] = v * Phi(v)   (Phi = standard normal CDF)
 *           FP8_ACT_SWIGLU: y[m][f] = silu(v[m][2f]) * v[m][2f+1],  silu(g) = g / (1 + e^-g);
 *                           B's rows interleave gate and up units (row 2f = gate f,
 *                           row 2f+1 = up f); C has N/2 columns; N must be even.
 *   C (row-major, N or N/2 columns) by c_dtype:
 *     OUT_F32, OUT_BF16:    y (bf16: round to nearest even)
 *     OUT_E4M3, OUT_E5M2:   code = enc(fp32(y * c_scale[0])) with fp8_quantize's saturating
 *                           cast (NaN -> sign | 0x7F), and c_amax[0] = max(c_amax[0], max |y|)
 *                           (an atomic max, so c_amax accumulates over calls until the
 *                           recipe update reads and clears it).
 *   Alignment: C, aux 16-byte aligned; bias 4-byte (fp32) or 2-byte (bf16) aligned;
 *   c_scale, c_amax 4-byte aligned.  c_scale / c_amax are ignored for fp32 / bf16 output.
 *   Errors: as fp8_gemm; FP8_ERR_ARG (fmt_b not E4M3, bad act, misaligned or missing c_scale /
 *           c_amax for FP8 output), FP8_ERR_SHAPE (SwiGLU with odd N), FP8_ERR_DTYPE (c_dtype,
 *           bias_dtype).
 */
int fp8_gemm_fused(const uint8_t *A, int fmt_a, const void *a_scale_inv, int gran_a,
                   const uint8_t *B, int fmt_b, const void *b_scale_inv, int gran_b,
                   const void *bias, int bias_dtype, int act, void *aux, void *C, int c_dtype,
                   const float *c_scale, float *c_amax, int64_t M, int64_t N, int64_t K,
                   void *stream);

/* Text describing the calling thread's last non-OK status ("" if none).  Owned by the
 * library; valid until the next call on the same thread. */
const char *fp8_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SCALED_FP8_H */
