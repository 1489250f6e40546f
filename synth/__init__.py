"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module draws random numbers and rounds them to the input dtypes; it holds
none of the quantization or linear-layer arithmetic.  bf16 tensors are
returned as uint16 bit patterns (numpy), float32 tensors as float32.

Workloads (d_in = K, d_out = N, W stored [N, K]; LLaMA-shaped dimensions
stand in for pretrained weights, which the pages model as roughly zero-mean
normal):

1. one 1024 -> 1024 linear, M = 64, r = 8, alpha = 16, W fp32 N(0, 0.02^2);
   B is run once as zeros and once as N(0, 0.01^2).
2. LLaMA-7B-shaped linears 4096->4096, 4096->11008, 11008->4096, M = 4096
   (batch 4 x seq 1024), r = 64, alpha = 16, W bf16 N(0, 0.02^2).
3. small-M forward on 4096->11008 and 11008->4096, M in {1, 4, 16}, r = 16,
   alpha = 32.
4. a LLaMA-65B-shaped decoder layer: q, k, v, o 8192->8192, gate and up
   8192->22016, down 22016->8192, M = 2048, r = 64, alpha = 16,
   W bf16 N(0, 0.015^2).
5. quantization stress: W [8192, 22016] bf16 = 0.02 * Student-t(df=3), 0.1 %
   of entries replaced by +-50 * std outliers (std = 0.02 * sqrt(3)), and one
   all-zero 64-block per row; 12 such matrices (about 4 GiB of bf16); an
   M = 512, r = 32, alpha = 16 forward.

All draws: X ~ N(0, 1), A ~ N(0, 1/r), B ~ N(0, 0.01^2), dY ~ N(0, 1), then
rounded to bf16 (RNE).  Linear i of workload c uses its own generator
``numpy.random.default_rng([c - 1, i, extra])``, drawing W, X, A, B, dY in
that order, so any one linear can be regenerated alone.
"""

from dataclasses import dataclass, field
import math

import numpy as np


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    linears: tuple            # ((K, N), ...) = ((d_in, d_out), ...)
    M: tuple                  # token counts
    r: int
    alpha: float
    w_dtype: str              # "f32" or "bf16"
    w_std: float
    w_kind: str = "normal"    # "normal" or "stress"
    linear_names: tuple = field(default_factory=tuple)


WORKLOADS = {
    1: Workload(1, "single linear 1024->1024, M=64, r=8", ((1024, 1024),), (64,), 8, 16.0, "f32", 0.02),
    2: Workload(2, "LLaMA-7B linears, M=4096, r=64",
                ((4096, 4096), (4096, 11008), (11008, 4096)), (4096,), 64, 16.0, "bf16", 0.02,
                linear_names=("attn 4096->4096", "mlp 4096->11008", "mlp 11008->4096")),
    3: Workload(3, "small-M forward, r=16", ((4096, 11008), (11008, 4096)), (1, 4, 16), 16, 32.0, "bf16", 0.02),
    4: Workload(4, "LLaMA-65B decoder layer, M=2048, r=64",
                ((8192, 8192),) * 4 + ((8192, 22016),) * 2 + ((22016, 8192),), (2048,), 64, 16.0, "bf16", 0.015,
                linear_names=("q", "k", "v", "o", "gate", "up", "down")),
    5: Workload(5, "quantization stress 8192x22016 x12, M=512, r=32",
                ((22016, 8192),) * 12, (512,), 32, 16.0, "bf16", 0.02, w_kind="stress"),
}


def to_bf16_bits(x):
    """Round float32 to bf16 (RNE) with torch's CPU conversion; return uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape, std):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def stress_weight(rng, N, K, scale=0.02, outlier_frac=1e-3, outlier_mult=50.0):
    """Student-t(3) * scale weights with outliers and one zero 64-block per row (float32)."""
    W = (rng.standard_t(3.0, size=(N, K)) * scale).astype(np.float32)
    std = scale * math.sqrt(3.0)               # std of scale * t(3)
    mask = rng.random((N, K)) < outlier_frac
    sign = np.where(rng.integers(0, 2, size=(N, K)) == 1, 1.0, -1.0).astype(np.float32)
    W[mask] = (sign[mask] * np.float32(outlier_mult * std)).astype(np.float32)
    zb = rng.integers(0, K // 64, size=N)
    for n in range(N):
        W[n, zb[n] * 64:(zb[n] + 1) * 64] = 0.0
    return W


def draw_weight(rng, N, K, w_std=0.02, w_dtype="bf16", w_kind="normal"):
    """W [N, K]: float32 array for "f32", uint16 bf16 bits for "bf16"."""
    if w_kind == "stress":
        W = stress_weight(rng, N, K, scale=w_std)
    else:
        W = _normal(rng, (N, K), w_std)
    return W if w_dtype == "f32" else to_bf16_bits(W)


def draw_linear(key, N, K, M, r, w_std=0.02, w_dtype="bf16", w_kind="normal", b_std=0.01,
                parts=("W", "X", "A", "B", "dY")):
    """Draw one linear's inputs from ``default_rng(key)`` in the order W, X, A, B, dY.

    Parts not requested are still drawn (so the stream stays aligned) unless
    they come after every requested part.
    """
    rng = np.random.default_rng(key)
    order = ("W", "X", "A", "B", "dY")
    last = max(order.index(p) for p in parts)
    out = {}
    for name in order[:last + 1]:
        if name == "W":
            v = draw_weight(rng, N, K, w_std, w_dtype, w_kind)
        elif name == "X":
            v = to_bf16_bits(_normal(rng, (M, K), 1.0))
        elif name == "A":
            v = to_bf16_bits(_normal(rng, (r, K), 1.0 / math.sqrt(r))) if r > 0 else np.zeros((0, K), np.uint16)
        elif name == "B":
            v = to_bf16_bits(_normal(rng, (N, r), b_std)) if r > 0 else np.zeros((N, 0), np.uint16)
        else:
            v = to_bf16_bits(_normal(rng, (M, N), 1.0))
        if name in parts:
            out[name] = v
    return out


def workload_linear(number, i, M=None, parts=("W", "X", "A", "B", "dY")):
    """Inputs of linear ``i`` of workload ``number`` (M defaults to the workload's first M)."""
    wl = WORKLOADS[number]
    K, N = wl.linears[i]
    M = wl.M[0] if M is None else M
    key = [number - 1, i, M]
    return draw_linear(key, N, K, M, wl.r, wl.w_std, wl.w_dtype, wl.w_kind, parts=parts)


def case(M, K, N, r, seed, w_std=0.02, w_dtype="bf16", w_kind="normal", b_std=0.01,
         parts=("W", "X", "A", "B", "dY")):
    """A free-shape test case with the workloads' distributions."""
    return draw_linear([1000 + seed, M, K, N, r], N, K, M, r, w_std, w_dtype, w_kind, b_std, parts)
