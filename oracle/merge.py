"""LoRA merge / unmerge into a bf16 copy of the dequantized base (test
infrastructure only).

[Repro] "官方代码阅读路线": the adapter update B A can be added into the frozen
weight for inference and removed again (merge / unmerge); "失败排查清单" items 4
and 6: merge exactly once, and compare the logits before and after.  [QLoRA
note] (merging into a 4-bit base adds error): the merge target is a higher
precision copy of the base, here bf16.  Reading of the rounding:

    delta  = sum_j B[n, j] A[j, k]          (exact here; fp32 accumulation on the GPU)
    merge:   out = bf16_rne(W' + RN32(scale * RN32(delta)))    W' = the bf16 decode
    unmerge: out = bf16_rne(Wm - RN32(scale * RN32(delta)))    Wm = a merged bf16 matrix

with scale = alpha / r (fp32) and every other operation one fp32 rounding.  With
r = 0 there is no adapter and the merge returns the base unchanged (scale taken as 0).
"""

import numpy as np

from .fp import bf16_bits, bf16_to_f32


def lora_delta_f32(A_bits, B_bits):
    """RN32 of the exact sum_j B[n, j] A[j, k] (float64 products of bf16 values are exact;
    the float64 sum of r <= 256 of them is within a few ulp of double, far below fp32)."""
    A = bf16_to_f32(A_bits).astype(np.float64)
    B = bf16_to_f32(B_bits).astype(np.float64)
    return (B @ A).astype(np.float32)


def _scale(alpha, r):
    return np.float32(np.float32(alpha) / np.float32(r)) if r > 0 else np.float32(0.0)


def merge(Wd_bits, A_bits, B_bits, alpha, r):
    """bf16 bits of the merged weight from the bf16 decode of the base."""
    scale = _scale(alpha, r)
    d = lora_delta_f32(A_bits, B_bits)
    return bf16_bits(bf16_to_f32(Wd_bits) + scale * d)


def unmerge(Wm_bits, A_bits, B_bits, alpha, r):
    """bf16 bits of Wm - scale * B A (one fp32 rounding per operation, then bf16)."""
    scale = _scale(alpha, r)
    d = lora_delta_f32(A_bits, B_bits)
    return bf16_bits(bf16_to_f32(Wm_bits) - scale * d)
