"""Seeded synthetic inputs for the five FP8 scaled-linear workloads.

Shared by the tests, the bench and the oracle's callers; holds none of the
method's arithmetic (no scaling, no encoding, no GEMM): only draws from
``torch.randn`` on a CPU generator, a fixed multiplier for the standard
deviation, outlier planting, and the float32 -> bfloat16 conversion of the
inputs that are bf16 by definition.

The pages name no dataset; every input is synthetic with the shapes and value
distributions the workloads specify ("N(0, s)" means standard deviation s).
Each tensor is drawn from its own ``torch.Generator`` seeded with
``seed * 1_000_003 + stream`` so that any tensor (or any step's tensor) can be
regenerated alone, in any order.

Workloads
---------
1  per-tensor delayed scaling, fp32: X_t [256x256] ~N(0,1) for t = 0..15
   (fresh each step), W [256x256] ~N(0,0.02); 16 steps.
2  MiniGPT layer set (hidden 768, FFN 3072, 8 x 256 = 2048 tokens), bf16:
   layers QKV 768 -> 2304, FC1 768 -> 3072, FC2 3072 -> 768; per layer
   X [2048][K_in] ~N(0,1), W [N_out][K_in] ~N(0,0.02), dY [2048][N_out]
   ~N(0,1e-3); X and dY fresh each step, W fixed.
3  blockwise current scaling, bf16: X [4096x7168] ~N(0,1) with 0.1% of the
   entries (uniform positions, no repeats) multiplied by 100 before the bf16
   conversion; W [7168x7168] ~N(0,0.02); for the blockwise backward, the
   output gradient dY [4096x7168] ~N(0,1e-3).
4  large SwiGLU FC1, bf16: X [8192x4096] ~N(0,1), W [14336x4096] ~N(0,0.02),
   dY [8192x14336] ~N(0,1e-4).
5  MX square GEMM, bf16: A, B [8192x8192] ~N(0,1); plus a standalone
   2^28-element bf16 tensor ~N(0,1) for the amax + cast stream.
"""

from __future__ import annotations

import torch

MINIGPT_LAYERS = (("qkv", 768, 2304), ("fc1", 768, 3072), ("fc2", 3072, 768))
MINIGPT_TOKENS = 2048


def _gen(seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1_000_003 + stream)
    return g


def normal(shape, std: float, seed: int, stream: int, dtype=torch.float32) -> torch.Tensor:
    """N(0, std) float32 draw, converted to ``dtype`` (bf16: round to nearest even)."""
    x = torch.randn(*shape, generator=_gen(seed, stream), dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def with_outliers(x: torch.Tensor, fraction: float, factor: float, seed: int, stream: int) -> torch.Tensor:
    """Multiply ``fraction`` of the entries (distinct, uniform positions) by ``factor``."""
    x = x.clone()
    n = x.numel()
    k = int(round(n * fraction))
    idx = torch.randperm(n, generator=_gen(seed, stream))[:k]
    x.view(-1)[idx] *= factor
    return x


# --------------------------------------------------------------------------- workload 1


def w1_weight(seed: int = 0) -> torch.Tensor:
    return normal((256, 256), 0.02, seed, 1)


def w1_input(step: int, seed: int = 0) -> torch.Tensor:
    return normal((256, 256), 1.0, seed, 100 + step)


# --------------------------------------------------------------------------- workload 2


def w2_layer(layer: int, step: int, seed: int = 0, tokens: int = MINIGPT_TOKENS):
    """(X [tokens][K_in], W [N_out][K_in], dY [tokens][N_out]) in bf16 for one layer and step."""
    _, k_in, n_out = MINIGPT_LAYERS[layer]
    bf = torch.bfloat16
    w = normal((n_out, k_in), 0.02, seed, 200 + layer, bf)
    x = normal((tokens, k_in), 1.0, seed, 1000 + 16 * layer + step, bf)
    dy = normal((tokens, n_out), 1e-3, seed, 2000 + 16 * layer + step, bf)
    return x, w, dy


# --------------------------------------------------------------------------- workload 3


def w3_inputs(seed: int = 0, m: int = 4096, k: int = 7168, n: int = 7168):
    x = normal((m, k), 1.0, seed, 300)
    x = with_outliers(x, 0.001, 100.0, seed, 301).to(torch.bfloat16)
    w = normal((n, k), 0.02, seed, 302, torch.bfloat16)
    return x, w


def w3_grad(seed: int = 0, m: int = 4096, n: int = 7168):
    """Output gradient dY [m][n] for the blockwise backward."""
    return normal((m, n), 1e-3, seed, 303, torch.bfloat16)


# --------------------------------------------------------------------------- workload 4


def w4_inputs(seed: int = 0, m: int = 8192, k: int = 4096, n: int = 14336):
    bf = torch.bfloat16
    x = normal((m, k), 1.0, seed, 400, bf)
    w = normal((n, k), 0.02, seed, 401, bf)
    dy = normal((m, n), 1e-4, seed, 402, bf)
    return x, w, dy


# --------------------------------------------------------------------------- workload 5


def w5_inputs(seed: int = 0, m: int = 8192, n: int = 8192, k: int = 8192):
    bf = torch.bfloat16
    return normal((m, k), 1.0, seed, 500, bf), normal((n, k), 1.0, seed, 501, bf)


def w5_stream(seed: int = 0, numel: int = 1 << 28) -> torch.Tensor:
    return normal((numel,), 1.0, seed, 502, torch.bfloat16)
