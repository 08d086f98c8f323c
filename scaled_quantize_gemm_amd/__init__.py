"""Python binding of the FP8 scaled-linear C ABI (include/scaled_fp8.h) for MI355X (gfx950).

Argument marshalling only: every step of the path (amax, scale derivation, cast,
cast-transpose, GEMM, recipe update) runs in the HIP kernels of
``lib/libscaledfp8.so``.  PyTorch provides device memory and the current stream.
The functions carry the C names and take torch tensors; outputs not supplied are
allocated with torch on the input's device.

Importing works without a GPU (the library loads on any x86-64 host with ROCm);
calls that launch kernels need a gfx950 device.  If the library has not been
built, importing raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import List, Optional

import torch

from .build import LIBDIR, LIBNAME

# ------------------------------------------------------------------ constants (scaled_fp8.h)

FP8_E4M3, FP8_E5M2 = 0, 1
HP_F32, HP_BF16 = 0, 1
OUT_F32, OUT_BF16, OUT_E4M3, OUT_E5M2 = 0, 1, 2, 3
FP8_ACT_NONE, FP8_ACT_GELU, FP8_ACT_SWIGLU = 0, 1, 2
FP8_SCALE_TENSOR, FP8_SCALE_TILE_1x128, FP8_SCALE_BLOCK_128x128, FP8_SCALE_MX_1x32 = 0, 1, 2, 3
FP8_AMAX_ALGO_MAX = 0
FP8_OK, FP8_ERR_ARG, FP8_ERR_SHAPE, FP8_ERR_DTYPE, FP8_ERR_DEVICE, FP8_ERR_LAUNCH = 0, -1, -2, -3, -4, -5

EXPORTED = ("fp8_device_check", "fp8_recipe_update", "fp8_quantize", "fp8_quantize_diag", "fp8_cast_transpose",
            "fp8_cast_transpose_blockwise", "fp8_gemm", "fp8_gemm_fused", "fp8_layernorm_quantize",
            "fp8_last_error")

LIB_PATH = os.path.join(LIBDIR, LIBNAME)


class Fp8Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m scaled_quantize_gemm_amd.build` "
                          "(or __graft_entry__.build()). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.fp8_device_check.argtypes = [i32, ctypes.c_char_p, sz]
    lib.fp8_recipe_update.argtypes = [vp, vp, vp, ctypes.POINTER(i32), i32, i32, i32, i32, vp]
    lib.fp8_quantize.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, vp, vp]
    lib.fp8_quantize_diag.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp]
    lib.fp8_cast_transpose.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp]
    lib.fp8_cast_transpose_blockwise.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, vp, vp]
    lib.fp8_gemm.argtypes = [vp, i32, vp, i32, vp, i32, vp, i32, vp, i32, i64, i64, i64, vp]
    lib.fp8_layernorm_quantize.argtypes = [vp, i32, i64, i64, vp, vp, i32, ctypes.c_float, i32, i32, vp, vp, vp, vp,
                                           vp, vp, vp]
    lib.fp8_gemm_fused.argtypes = [vp, i32, vp, i32, vp, i32, vp, i32, vp, i32, i32, vp, vp, i32, vp, vp, i64, i64,
                                   i64, vp]
    lib.fp8_last_error.restype = ctypes.c_char_p
    for name in ("fp8_device_check", "fp8_recipe_update", "fp8_quantize", "fp8_quantize_diag", "fp8_cast_transpose",
                 "fp8_cast_transpose_blockwise", "fp8_gemm"):
        getattr(lib, name).restype = i32
    return lib


lib = _load()


def fp8_last_error() -> str:
    return lib.fp8_last_error().decode()


def _check(rc: int) -> None:
    if rc != FP8_OK:
        raise Fp8Error(rc, fp8_last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    return t.data_ptr()


def _contig(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    return t


# the current stream's raw handle: torch's accessor takes ~0.1 us where building the Stream
# object of torch.cuda.current_stream() takes ~2 us of a ~7 us call; the public route stays as
# the fallback
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor) -> int:
    if _raw_stream is not None:
        return _raw_stream(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _hp_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return HP_BF16
    if x.dtype == torch.float32:
        return HP_F32
    raise TypeError(f"unsupported input dtype {x.dtype} (bf16 or fp32)")


def _as2d(x: torch.Tensor):
    if x.dim() == 1:
        return 1, x.shape[0]
    if x.dim() != 2:
        raise ValueError("1-D or 2-D tensor expected")
    return x.shape[0], x.shape[1]


# ------------------------------------------------------------------ entry points


def fp8_device_check(device: int = 0):
    """(ok, reason) -- ok iff `device` is a gfx950 GPU."""
    buf = ctypes.create_string_buffer(256)
    rc = lib.fp8_device_check(device, buf, 256)
    return rc == FP8_OK, buf.value.decode()


def fp8_recipe_update(amax_history: torch.Tensor, scale: torch.Tensor, scale_inv: torch.Tensor, fmts: List[int],
                      margin: int = 0, algo: int = FP8_AMAX_ALGO_MAX) -> None:
    """End-of-step delayed-scaling update of [H][n] history and [n] scales (in place)."""
    h, n = amax_history.shape
    for t, nm in ((amax_history, "amax_history"), (scale, "scale"), (scale_inv, "scale_inv")):
        _contig(t, nm)
        if t.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32")
    if scale.numel() != n or scale_inv.numel() != n or len(fmts) != n:
        raise ValueError("scale, scale_inv and fmts must have n entries")
    arr = (ctypes.c_int * n)(*fmts)
    _check(lib.fp8_recipe_update(_ptr(amax_history), _ptr(scale), _ptr(scale_inv), arr, n, h, algo, margin,
                                 _stream(amax_history)))


def fp8_quantize(x: torch.Tensor, fmt: int, granularity: int = FP8_SCALE_TENSOR, scale: Optional[torch.Tensor] = None,
                 amax_slot: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
                 scale_inv_out: Optional[torch.Tensor] = None):
    """Fused amax + cast of x [rows][cols] -> (q uint8 [rows][cols], scale_inv_out or None)."""
    _contig(x, "x")
    rows, cols = _as2d(x)
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale_inv_out is None and granularity != FP8_SCALE_TENSOR:
        if granularity == FP8_SCALE_TILE_1x128:
            scale_inv_out = torch.empty((cols // 128, rows), dtype=torch.float32, device=x.device)
        elif granularity == FP8_SCALE_BLOCK_128x128:
            scale_inv_out = torch.empty(((rows + 127) // 128, cols // 128), dtype=torch.float32, device=x.device)
        else:
            scale_inv_out = torch.empty((cols // 32, rows), dtype=torch.uint8, device=x.device)
    _check(lib.fp8_quantize(_ptr(x), _hp_dtype(x), rows, cols, fmt, granularity, _ptr(scale), _ptr(amax_slot),
                            _ptr(q), _ptr(scale_inv_out), _stream(x)))
    return q, scale_inv_out


def fp8_quantize_diag(x: torch.Tensor, fmt: int, scale: torch.Tensor, counts: torch.Tensor,
                      amax_slot: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-tensor cast with diagnostics: adds (saturated, underflowed, nan) element counts to
    `counts` (device int64 [3]); returns q."""
    _contig(x, "x")
    rows, cols = _as2d(x)
    if counts.dtype != torch.int64 or counts.numel() != 3:
        raise TypeError("counts must be a device int64 tensor of 3 entries")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    _check(lib.fp8_quantize_diag(_ptr(x), _hp_dtype(x), rows, cols, fmt, _ptr(scale), _ptr(amax_slot), _ptr(q),
                                 _ptr(counts), _stream(x)))
    return q


def fp8_cast_transpose(x: torch.Tensor, fmt: int, scale: torch.Tensor, amax_slot: Optional[torch.Tensor] = None,
                       q: Optional[torch.Tensor] = None, qT: Optional[torch.Tensor] = None):
    """Per-tensor cast of x [rows][cols] and its transpose -> (q [rows][cols], qT [cols][rows])."""
    _contig(x, "x")
    rows, cols = _as2d(x)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if qT is None:
        qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    _check(lib.fp8_cast_transpose(_ptr(x), _hp_dtype(x), rows, cols, fmt, _ptr(scale), _ptr(amax_slot), _ptr(q),
                                  _ptr(qT), _stream(x)))
    return q, qT


def fp8_cast_transpose_blockwise(x: torch.Tensor, fmt: int, granularity: int, q: Optional[torch.Tensor] = None,
                                 q_scale_inv: Optional[torch.Tensor] = None, qT: Optional[torch.Tensor] = None,
                                 qT_scale_inv: Optional[torch.Tensor] = None):
    """Current-scaling cast of x [rows][cols] and its transpose, each with its own scales ->
    (q [rows][cols], q_scale_inv, qT [cols][rows], qT_scale_inv).  TILE_1x128: q_scale_inv
    [cols/128][rows], qT_scale_inv [rows/128][cols]; BLOCK_128x128: [rows/128][cols/128] and
    its transpose."""
    _contig(x, "x")
    rows, cols = _as2d(x)
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if qT is None:
        qT = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    if granularity == FP8_SCALE_TILE_1x128:
        qs, qts = (cols // 128, rows), (rows // 128, cols)
    else:
        qs, qts = (rows // 128, cols // 128), (cols // 128, rows // 128)
    if q_scale_inv is None:
        q_scale_inv = torch.empty(qs, dtype=torch.float32, device=dev)
    if qT_scale_inv is None:
        qT_scale_inv = torch.empty(qts, dtype=torch.float32, device=dev)
    _check(lib.fp8_cast_transpose_blockwise(_ptr(x), _hp_dtype(x), rows, cols, fmt, granularity, _ptr(q),
                                            _ptr(q_scale_inv), _ptr(qT), _ptr(qT_scale_inv), _stream(x)))
    return q, q_scale_inv, qT, qT_scale_inv


def fp8_gemm(A: torch.Tensor, fmt_a: int, a_scale_inv: torch.Tensor, gran_a: int, B: torch.Tensor, fmt_b: int,
             b_scale_inv: torch.Tensor, gran_b: int, out_dtype: int = OUT_F32,
             C: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[M][N] = deq(A)[M][K] . deq(B)[N][K]^T."""
    _contig(A, "A")
    _contig(B, "B")
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError(f"K mismatch: {K} vs {K2}")
    if C is None:
        dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
        C = torch.empty((M, N), dtype=dt, device=A.device)
    _check(lib.fp8_gemm(_ptr(A), fmt_a, _ptr(a_scale_inv), gran_a, _ptr(B), fmt_b, _ptr(b_scale_inv), gran_b,
                        _ptr(C), out_dtype, M, N, K, _stream(A)))
    return C


def fp8_layernorm_quantize(x: torch.Tensor, gamma: torch.Tensor, beta: Optional[torch.Tensor], eps: float, fmt: int,
                           granularity: int = FP8_SCALE_TENSOR, scale: Optional[torch.Tensor] = None,
                           amax_slot: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
                           scale_inv_out: Optional[torch.Tensor] = None, mu: Optional[torch.Tensor] = None,
                           rsigma: Optional[torch.Tensor] = None):
    """LayerNorm over the last dim of x [rows][cols] cast to FP8 -> (q, scale_inv_out or None)."""
    _contig(x, "x")
    _contig(gamma, "gamma")
    rows, cols = _as2d(x)
    if beta is not None:
        _contig(beta, "beta")
        if beta.dtype != gamma.dtype:
            raise TypeError("gamma and beta must share a dtype")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale_inv_out is None and granularity == FP8_SCALE_TILE_1x128:
        scale_inv_out = torch.empty((cols // 128, rows), dtype=torch.float32, device=x.device)
    elif scale_inv_out is None and granularity == FP8_SCALE_MX_1x32:
        scale_inv_out = torch.empty((cols // 32, rows), dtype=torch.uint8, device=x.device)
    _check(lib.fp8_layernorm_quantize(_ptr(x), _hp_dtype(x), rows, cols, _ptr(gamma), _ptr(beta), _hp_dtype(gamma),
                                      float(eps), fmt, granularity, _ptr(scale), _ptr(amax_slot), _ptr(q),
                                      _ptr(scale_inv_out), _ptr(mu), _ptr(rsigma), _stream(x)))
    return q, scale_inv_out


_OUT_TORCH = {OUT_F32: torch.float32, OUT_BF16: torch.bfloat16, OUT_E4M3: torch.uint8, OUT_E5M2: torch.uint8}


def fp8_gemm_fused(A: torch.Tensor, fmt_a: int, a_scale_inv: torch.Tensor, gran_a: int, B: torch.Tensor, fmt_b: int,
                   b_scale_inv: torch.Tensor, gran_b: int, out_dtype: int = OUT_BF16,
                   bias: Optional[torch.Tensor] = None, act: int = FP8_ACT_NONE, aux: Optional[torch.Tensor] = None,
                   c_scale: Optional[torch.Tensor] = None, c_amax: Optional[torch.Tensor] = None,
                   C: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp8_gemm with bias, optional bf16 pre-activation copy (aux), GELU / SwiGLU and an
    fp32 / bf16 / FP8 output (FP8: codes under c_scale, amax max-reduced into c_amax)."""
    _contig(A, "A")
    _contig(B, "B")
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError(f"K mismatch: {K} vs {K2}")
    if C is None:
        cols = N // 2 if act == FP8_ACT_SWIGLU else N
        C = torch.empty((M, cols), dtype=_OUT_TORCH.get(out_dtype, torch.float32), device=A.device)
    bias_dt = HP_F32
    if bias is not None:
        _contig(bias, "bias")
        bias_dt = _hp_dtype(bias)
    _check(lib.fp8_gemm_fused(_ptr(A), fmt_a, _ptr(a_scale_inv), gran_a, _ptr(B), fmt_b, _ptr(b_scale_inv), gran_b,
                              _ptr(bias), bias_dt, act, _ptr(aux), _ptr(C), out_dtype, _ptr(c_scale), _ptr(c_amax),
                              M, N, K, _stream(A)))
    return C


# ------------------------------------------------------------------ recipe state


@dataclass
class DelayedScalingState:
    """Device-resident delayed-scaling state: amax_history [H][n], scale [n], scale_inv [n].

    Mirrors the tutorial's DelayedScaling(fp8_format, amax_history_len, amax_compute_algo)
    plus margin; `fmts` holds each slot's FP8 format (HYBRID: E4M3 forward, E5M2 gradients).
    """

    fmts: List[int]
    history_len: int = 16
    margin: int = 0
    device: str = "cuda"
    amax_history: torch.Tensor = field(init=False)
    scale: torch.Tensor = field(init=False)
    scale_inv: torch.Tensor = field(init=False)

    def __post_init__(self):
        n = len(self.fmts)
        self.amax_history = torch.zeros((self.history_len, n), dtype=torch.float32, device=self.device)
        self.scale = torch.ones(n, dtype=torch.float32, device=self.device)
        self.scale_inv = torch.ones(n, dtype=torch.float32, device=self.device)

    def slot(self, j: int):
        """(scale, amax_slot, scale_inv) views of slot j for quantize / gemm calls."""
        return self.scale[j:j + 1], self.amax_history[0, j:j + 1], self.scale_inv[j:j + 1]

    def update(self) -> None:
        fp8_recipe_update(self.amax_history, self.scale, self.scale_inv, self.fmts, self.margin)
