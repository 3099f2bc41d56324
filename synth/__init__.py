"""Seeded synthetic inputs for the W4A4 linear layer (shared by tests, bench and smoke).

This module only draws random tensors of the right shapes and distributions.  It holds
none of the layer's arithmetic (no outlier statistic, no reordering, no quantisation):
both the CPU oracle and the HIP path receive the same arrays from here.

Workload shapes follow Llama-7B / Llama-70B linear layers.  Every draw uses
``numpy.random.default_rng(seed)`` in a fixed order:

1. the seeded outlier channel indices ``rng.choice(K, n, replace=False)`` (if any),
2. the activations X (float32 draws, rounded to fp16),
3. the weights W (float32 N(0,1) draws times the std, rounded to fp16).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_linear", "make_inputs", "quant_only_x"]


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str            # short key used on the command line and in test ids
    name: str           # descriptive name
    M: int              # tokens
    K: int              # input channels (including the 128 outlier channels)
    N: int              # output channels
    x_kind: str         # "outliers" | "laplace" | "silu" | "rows_of_quant"
    n_out: int          # number of seeded outlier channels
    out_scale: float    # multiplier applied to the seeded outlier channels
    w_std: float        # standard deviation of W
    seed: int = 0

    @property
    def ops(self) -> int:
        """Integer operations of the contraction: 2*M*N*K over the full K."""
        return 2 * self.M * self.N * self.K


WORKLOADS: dict[str, Workload] = {
    w.key: w
    for w in [
        Workload("T", "tiny_w4a4_linear_16x1024x512", 16, 1024, 512, "outliers", 128, 20.0, 0.02),
        Workload("A", "llama7b_attn_proj_256x4096x4096", 256, 4096, 4096, "laplace",
                 int(round(0.01 * 4096)), 25.0, 0.02),
        Workload("B", "llama7b_mlp_gate_up_1024x4096x11008", 1024, 4096, 11008, "outliers", 128, 20.0, 0.02),
        Workload("C", "llama7b_mlp_down_2048x11008x4096", 2048, 11008, 4096, "silu", 0, 1.0, 0.015),
        Workload("D", "llama70b_mlp_4096x8192x28672", 4096, 8192, 28672, "rows_of_quant", 128, 30.0, 0.02),
        # decode-sized batches (16 tokens) through the same three Llama-7B weight shapes
        Workload("dA", "llama7b_attn_proj_decode_16x4096x4096", 16, 4096, 4096, "laplace",
                 int(round(0.01 * 4096)), 25.0, 0.02),
        Workload("dB", "llama7b_mlp_gate_up_decode_16x4096x11008", 16, 4096, 11008, "outliers", 128, 20.0, 0.02),
        Workload("dC", "llama7b_mlp_down_decode_16x11008x4096", 16, 11008, 4096, "silu", 0, 1.0, 0.015),
    ]
}

# The standalone activation-quantize workload: 8192 x 8192 fp16, 128 channels x30.
QUANT_ONLY = dict(key="Dq", name="quantize_only_8192x8192", M=8192, K=8192, n_out=128, out_scale=30.0, seed=0)


def get(key: str) -> Workload:
    return WORKLOADS[key]


def _fp16(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float16)


def _x_outliers(rng, M, K, n_out, scale):
    idx = rng.choice(K, n_out, replace=False) if n_out else np.zeros(0, np.int64)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if n_out:
        x[:, idx] *= np.float32(scale)
    return _fp16(x), np.sort(idx)


def quant_only_x(rows: int | None = None):
    """X of the standalone quantize workload (8192x8192, N(0,1), 128 channels x30).

    ``rows`` keeps only the first rows (the draw itself is always the full matrix so that
    a prefix is the same data as the full workload).  Returns (X fp16, seeded outlier idx, rng)."""
    q = QUANT_ONLY
    rng = np.random.default_rng(q["seed"])
    x, idx = _x_outliers(rng, q["M"], q["K"], q["n_out"], q["out_scale"])
    if rows is not None:
        x = np.ascontiguousarray(x[:rows])
    return x, idx, rng


def make_inputs(w: Workload, with_w: bool = True):
    """Return (X fp16 [M,K], W fp16 [N,K] or None, seeded outlier channel indices)."""
    if w.x_kind == "rows_of_quant":
        x, idx, rng = quant_only_x(rows=w.M)
    else:
        rng = np.random.default_rng(w.seed)
        if w.x_kind == "outliers":
            x, idx = _x_outliers(rng, w.M, w.K, w.n_out, w.out_scale)
        elif w.x_kind == "laplace":
            idx = np.sort(rng.choice(w.K, w.n_out, replace=False))
            x = rng.standard_normal((w.M, w.K), dtype=np.float32)
            lap = rng.laplace(0.0, 1.0 / math.sqrt(2.0), size=(w.M, w.n_out)).astype(np.float32)
            x[:, idx] = lap * np.float32(w.out_scale)
            x = _fp16(x)
        elif w.x_kind == "silu":
            a = _fp16(rng.standard_normal((w.M, w.K), dtype=np.float32)).astype(np.float32)
            b = _fp16(rng.standard_normal((w.M, w.K), dtype=np.float32)).astype(np.float32)
            x = _fp16(a / (np.float32(1.0) + np.exp(-a)) * b)
            idx = np.zeros(0, np.int64)
        else:
            raise ValueError(w.x_kind)
    wt = None
    if with_w:
        wt = _fp16(rng.standard_normal((w.N, w.K), dtype=np.float32) * np.float32(w.w_std))
    return x, wt, idx


def make_linear(M: int, K: int, N: int, seed: int = 0, n_out: int = 128, out_scale: float = 20.0,
                w_std: float = 0.02):
    """Generic small case: X ~ N(0,1) with ``n_out`` seeded channels scaled, W ~ N(0, w_std)."""
    rng = np.random.default_rng(seed)
    x, idx = _x_outliers(rng, M, K, min(n_out, K), out_scale)
    wt = _fp16(rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_std))
    return x, wt, idx
