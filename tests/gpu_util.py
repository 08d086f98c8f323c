"""Helpers for the GPU parity tests (imported only by tests marked gpu)."""

from __future__ import annotations

import concurrent.futures as cf
import json
import os
import sys

import numpy as np
import torch

from oracle import fp8 as ofp8

DEV = "cuda:0"

# per-case statistics against the stated GEMM tolerance, written out at the end of the session
TOLERANCE_STATS = {}
OUT_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")


def write_tolerance_stats(name="gemm_tolerance_workloads.json") -> None:
    if TOLERANCE_STATS:
        os.makedirs(OUT_DIR, exist_ok=True)
        with open(os.path.join(OUT_DIR, name), "w") as f:
            json.dump(TOLERANCE_STATS, f, indent=1, sort_keys=True)


def par_rows(fn, x, *args, chunks=16):
    """fn(x[rows], *args) over row chunks in threads (the oracle's elementwise quantisers
    release the interpreter lock); returns the list of per-chunk results in row order."""
    n = x.shape[0]
    edges = np.linspace(0, n, min(chunks, n) + 1).astype(int)
    with cf.ThreadPoolExecutor(max_workers=min(16, len(edges) - 1)) as ex:
        return list(ex.map(lambda i: fn(x[edges[i]:edges[i + 1]], *args), range(len(edges) - 1)))


def announce(*what) -> None:
    """Name the case before any GPU work, flushed, so a fault can be attributed."""
    print("[case]", *what, flush=True)
    sys.stdout.flush()


def np_of(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


def f32_np(x: torch.Tensor) -> np.ndarray:
    """High-precision input as float32 numpy (bf16 widened exactly)."""
    return x.detach().cpu().float().numpy()


def n_roundings(K: int, mode: str) -> int:
    """fp32 roundings an output can see: one per run of 8 promoted into the accumulator,
    three more per 128-K block for blockwise promotion (scale product, multiply, add),
    and the epilogue's scale multiplies."""
    n = K // 8 + 4
    if mode == "block":
        n += 3 * (K // 128)
    return n


def gemm_bound(S, G, K, mode, out_bf16, C_ref, C_gpu):
    """Per-element bound on |C_gpu - C_ref|.

    The matrix cores sum each run of 8 products exactly down to 2^(E - 13), E the run's
    largest operand-exponent sum, truncating the rest (at most 7 products lose less than
    2^(E-13) each: < 2^-10 G per run), then promote the run into fp32 (one rounding of at
    most 2^-24 S per addition).  A bf16 output adds one bf16 ulp.
    """
    b = 2.0 ** -10 * G + n_roundings(K, mode) * 2.0 ** -24 * S
    if out_bf16:
        b = b + ofp8.bf16_ulp(np.maximum(np.abs(C_ref), np.abs(C_gpu)))
    return b


def check_gemm(C_gpu, C_ref, S, G, K, mode, out_bf16, label=""):
    C_gpu = np.asarray(C_gpu, dtype=np.float64)
    err = np.abs(C_gpu - C_ref)
    bound = gemm_bound(S, G, K, mode, out_bf16, C_ref, C_gpu)
    bad = ~(err <= bound)
    ns_bound = 2.0 ** -18 * S + (ofp8.bf16_ulp(np.maximum(np.abs(C_ref), np.abs(C_gpu))) if out_bf16 else 0)
    frac_ns = float(np.mean(err <= ns_bound))
    rel = err / np.where(S > 0, S, 1.0)
    stats = {"max_err_over_S": float(rel.max()), "frac_within_2^-18_S": frac_ns,
             "max_err_over_bound": float((err / np.where(bound > 0, bound, 1.0)).max())}
    print(f"[gemm] {label} {stats}", flush=True)
    TOLERANCE_STATS[label] = stats
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {int(bad.sum())} outputs beyond bound; first {tuple(i)}: gpu={C_gpu[tuple(i)]} "
                             f"ref={C_ref[tuple(i)]} err={err[tuple(i)]} bound={bound[tuple(i)]}")
    return stats


def assert_codes_equal(got: np.ndarray, want: np.ndarray, label="") -> None:
    if not np.array_equal(got, want):
        d = np.argwhere(got != want)
        i = tuple(d[0])
        raise AssertionError(f"{label}: {len(d)} codes differ; first at {i}: gpu={got[i]:#04x} oracle={want[i]:#04x}")


def assert_f32_bits_equal(got, want, label="") -> None:
    """Bit-exact float32 equality, NaN compared by NaN-ness."""
    g = np.asarray(got, dtype=np.float32)
    w = np.asarray(want, dtype=np.float32)
    gn, wn = np.isnan(g), np.isnan(w)
    assert np.array_equal(gn, wn), f"{label}: NaN positions differ"
    gb, wb = g[~gn].view(np.uint32), w[~wn].view(np.uint32)
    if not np.array_equal(gb, wb):
        i = int(np.argmax(gb != wb))
        raise AssertionError(f"{label}: {(gb != wb).sum()} values differ; e.g. gpu={g[~gn][i]!r} oracle={w[~wn][i]!r}")
