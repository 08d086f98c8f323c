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


def _need(t: Optional[torch.Tensor], name: str, dtype, shape=None, min_numel: Optional[int] = None,
          device=None) -> None:
    """A caller-supplied buffer: contiguous, of `dtype`, and of exactly `shape` (or at least
    `min_numel` elements).  The C side sees only pointers, so a mis-sized buffer would be read
    or written out of bounds on the device.  Where each tensor lives is checked afterwards,
    for all of a call's tensors at once (_on_device)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dts)}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} element(s), got {t.numel()}")


def _on_device(**named) -> None:
    """Every given tensor on the same GPU (the first one's)."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the call's other tensors on {dev}")


def _scale_shape(gran: int, rows: int, k: int, operand_b: bool):
    """(dtype, shape) of a GEMM operand's scales in the layouts of scaled_fp8.h."""
    if gran == FP8_SCALE_TENSOR:
        return torch.float32, None
    if gran == FP8_SCALE_TILE_1x128:
        return torch.float32, (k // 128, rows)
    if gran == FP8_SCALE_BLOCK_128x128:
        return torch.float32, ((rows + 127) // 128, k // 128)
    if gran == FP8_SCALE_MX_1x32:
        return torch.uint8, (k // 32, rows)
    raise ValueError(f"unknown granularity {gran}")


def _gemm_operands(A, a_scale_inv, gran_a, B, b_scale_inv, gran_b):
    _need(A, "A", torch.uint8)
    _need(B, "B", torch.uint8)
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError(f"K mismatch: {K} vs {K2}")
    for t, nm, g, rows, isb in ((a_scale_inv, "a_scale_inv", gran_a, M, False),
                                (b_scale_inv, "b_scale_inv", gran_b, N, True)):
        if t is None:
            raise ValueError(f"{nm} is required")
        dt, shp = _scale_shape(g, rows, K, isb)
        _need(t, nm, dt, shape=shp, min_numel=1 if shp is None else None)
    return M, N, K


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


_OUT_TORCH = {OUT_F32: torch.float32, OUT_BF16: torch.bfloat16, OUT_E4M3: torch.uint8, OUT_E5M2: torch.uint8}

# ------------------------------------------------------------------ entry points


def fp8_device_check(device: int = 0):
    """(ok, reason) -- ok iff `device` is a gfx950 GPU."""
    buf = ctypes.create_string_buffer(256)
    rc = lib.fp8_device_check(device, buf, 256)
    return rc == FP8_OK, buf.value.decode()


def fp8_recipe_update(amax_history: torch.Tensor, scale: torch.Tensor, scale_inv: torch.Tensor, fmts: List[int],
                      margin: int = 0, algo: int = FP8_AMAX_ALGO_MAX) -> None:
    """End-of-step delayed-scaling update of [H][n] history and [n] scales (in place)."""
    _need(amax_history, "amax_history", torch.float32)
    if amax_history.dim() != 2:
        raise ValueError("amax_history must be [H][n]")
    h, n = amax_history.shape
    _need(scale, "scale", torch.float32, shape=(n,))
    _need(scale_inv, "scale_inv", torch.float32, shape=(n,))
    if len(fmts) != n:
        raise ValueError("fmts must have n entries")
    _on_device(amax_history=amax_history, scale=scale, scale_inv=scale_inv)
    arr = (ctypes.c_int * n)(*fmts)
    _check(lib.fp8_recipe_update(_ptr(amax_history), _ptr(scale), _ptr(scale_inv), arr, n, h, algo, margin,
                                 _stream(amax_history)))


def fp8_quantize(x: torch.Tensor, fmt: int, granularity: int = FP8_SCALE_TENSOR, scale: Optional[torch.Tensor] = None,
                 amax_slot: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
                 scale_inv_out: Optional[torch.Tensor] = None):
    """Fused amax + cast of x [rows][cols] -> (q uint8 [rows][cols], scale_inv_out or None)."""
    _need(x, "x", (torch.bfloat16, torch.float32))
    rows, cols = _as2d(x)
    _need(q, "q", torch.uint8, shape=tuple(x.shape))
    _need(scale, "scale", torch.float32, min_numel=1)
    _need(amax_slot, "amax_slot", torch.float32, min_numel=1)
    if scale_inv_out is not None:
        if granularity == FP8_SCALE_TILE_1x128:
            _need(scale_inv_out, "scale_inv_out", torch.float32, shape=(cols // 128, rows))
        elif granularity == FP8_SCALE_BLOCK_128x128:
            _need(scale_inv_out, "scale_inv_out", torch.float32, shape=((rows + 127) // 128, cols // 128))
        elif granularity == FP8_SCALE_MX_1x32:
            _need(scale_inv_out, "scale_inv_out", torch.uint8, shape=(cols // 32, rows))
    _on_device(x=x, q=q, scale=scale, amax_slot=amax_slot, scale_inv_out=scale_inv_out)
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
    _need(x, "x", (torch.bfloat16, torch.float32))
    rows, cols = _as2d(x)
    _need(counts, "counts", torch.int64, shape=(3,))
    _need(scale, "scale", torch.float32, min_numel=1)
    _need(amax_slot, "amax_slot", torch.float32, min_numel=1)
    _need(q, "q", torch.uint8, shape=(rows, cols))
    _on_device(x=x, counts=counts, scale=scale, amax_slot=amax_slot, q=q)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    _check(lib.fp8_quantize_diag(_ptr(x), _hp_dtype(x), rows, cols, fmt, _ptr(scale), _ptr(amax_slot), _ptr(q),
                                 _ptr(counts), _stream(x)))
    return q


def fp8_cast_transpose(x: torch.Tensor, fmt: int, scale: torch.Tensor, amax_slot: Optional[torch.Tensor] = None,
                       q: Optional[torch.Tensor] = None, qT: Optional[torch.Tensor] = None):
    """Per-tensor cast of x [rows][cols] and its transpose -> (q [rows][cols], qT [cols][rows])."""
    _need(x, "x", (torch.bfloat16, torch.float32))
    rows, cols = _as2d(x)
    _need(scale, "scale", torch.float32, min_numel=1)
    _need(amax_slot, "amax_slot", torch.float32, min_numel=1)
    _need(q, "q", torch.uint8, shape=(rows, cols))
    _need(qT, "qT", torch.uint8, shape=(cols, rows))
    _on_device(x=x, scale=scale, amax_slot=amax_slot, q=q, qT=qT)
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
    _need(x, "x", (torch.bfloat16, torch.float32))
    rows, cols = _as2d(x)
    dev = x.device
    if granularity == FP8_SCALE_TILE_1x128:
        qs, qts = (cols // 128, rows), (rows // 128, cols)
    else:
        qs, qts = (rows // 128, cols // 128), (cols // 128, rows // 128)
    _need(q, "q", torch.uint8, shape=(rows, cols))
    _need(qT, "qT", torch.uint8, shape=(cols, rows))
    _need(q_scale_inv, "q_scale_inv", torch.float32, shape=qs)
    _need(qT_scale_inv, "qT_scale_inv", torch.float32, shape=qts)
    _on_device(x=x, q=q, qT=qT, q_scale_inv=q_scale_inv, qT_scale_inv=qT_scale_inv)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if qT is None:
        qT = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
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
    M, N, K = _gemm_operands(A, a_scale_inv, gran_a, B, b_scale_inv, gran_b)
    if out_dtype not in (OUT_F32, OUT_BF16):
        raise ValueError(f"out_dtype {out_dtype}: fp8_gemm writes OUT_F32 or OUT_BF16")
    _need(C, "C", _OUT_TORCH[out_dtype], shape=(M, N))
    _on_device(A=A, B=B, a_scale_inv=a_scale_inv, b_scale_inv=b_scale_inv, C=C)
    if C is None:
        C = torch.empty((M, N), dtype=_OUT_TORCH[out_dtype], device=A.device)
    _check(lib.fp8_gemm(_ptr(A), fmt_a, _ptr(a_scale_inv), gran_a, _ptr(B), fmt_b, _ptr(b_scale_inv), gran_b,
                        _ptr(C), out_dtype, M, N, K, _stream(A)))
    return C


def fp8_layernorm_quantize(x: torch.Tensor, gamma: torch.Tensor, beta: Optional[torch.Tensor], eps: float, fmt: int,
                           granularity: int = FP8_SCALE_TENSOR, scale: Optional[torch.Tensor] = None,
                           amax_slot: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
                           scale_inv_out: Optional[torch.Tensor] = None, mu: Optional[torch.Tensor] = None,
                           rsigma: Optional[torch.Tensor] = None):
    """LayerNorm over the last dim of x [rows][cols] cast to FP8 -> (q, scale_inv_out or None)."""
    _need(x, "x", (torch.bfloat16, torch.float32))
    rows, cols = _as2d(x)
    _need(gamma, "gamma", (torch.bfloat16, torch.float32), shape=(cols,))
    if beta is not None:
        _need(beta, "beta", gamma.dtype, shape=(cols,))
    _need(q, "q", torch.uint8, shape=(rows, cols))
    _need(scale, "scale", torch.float32, min_numel=1)
    _need(amax_slot, "amax_slot", torch.float32, min_numel=1)
    _need(mu, "mu", torch.float32, shape=(rows,))
    _need(rsigma, "rsigma", torch.float32, shape=(rows,))
    if scale_inv_out is not None:
        if granularity == FP8_SCALE_TILE_1x128:
            _need(scale_inv_out, "scale_inv_out", torch.float32, shape=(cols // 128, rows))
        elif granularity == FP8_SCALE_MX_1x32:
            _need(scale_inv_out, "scale_inv_out", torch.uint8, shape=(cols // 32, rows))
    _on_device(x=x, gamma=gamma, beta=beta, q=q, scale=scale, amax_slot=amax_slot, mu=mu, rsigma=rsigma,
               scale_inv_out=scale_inv_out)
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


def fp8_gemm_fused(A: torch.Tensor, fmt_a: int, a_scale_inv: torch.Tensor, gran_a: int, B: torch.Tensor, fmt_b: int,
                   b_scale_inv: torch.Tensor, gran_b: int, out_dtype: int = OUT_BF16,
                   bias: Optional[torch.Tensor] = None, act: int = FP8_ACT_NONE, aux: Optional[torch.Tensor] = None,
                   c_scale: Optional[torch.Tensor] = None, c_amax: Optional[torch.Tensor] = None,
                   C: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp8_gemm with bias, optional bf16 pre-activation copy (aux), GELU / SwiGLU and an
    fp32 / bf16 / FP8 output (FP8: codes under c_scale, amax max-reduced into c_amax)."""
    M, N, K = _gemm_operands(A, a_scale_inv, gran_a, B, b_scale_inv, gran_b)
    dev = A.device
    if out_dtype not in _OUT_TORCH:
        raise ValueError(f"unknown out_dtype {out_dtype}")
    cols = N // 2 if act == FP8_ACT_SWIGLU else N
    _need(C, "C", _OUT_TORCH[out_dtype], shape=(M, cols))
    _need(aux, "aux", torch.bfloat16, shape=(M, N))
    _need(bias, "bias", (torch.float32, torch.bfloat16), shape=(N,))
    if out_dtype in (OUT_E4M3, OUT_E5M2):
        _need(c_scale, "c_scale", torch.float32, min_numel=1)
        _need(c_amax, "c_amax", torch.float32, min_numel=1)
    _on_device(A=A, B=B, a_scale_inv=a_scale_inv, b_scale_inv=b_scale_inv, C=C, aux=aux, bias=bias, c_scale=c_scale,
               c_amax=c_amax)
    if C is None:
        C = torch.empty((M, cols), dtype=_OUT_TORCH[out_dtype], device=dev)
    bias_dt = HP_F32
    if bias is not None:
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
