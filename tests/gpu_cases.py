"""Helpers for the GPU parity tests: move synthetic inputs to the device, and build
oracle references (from the oracle only, on the same seeded inputs)."""

import numpy as np

import synth
from oracle import linear, nf4


from synth.device import dev_bf16, dev_f32, dev_weight  # noqa: F401


def torch_mod():
    import torch
    return torch


def host_bits(t):
    """bf16 CUDA tensor -> uint16 numpy bit patterns."""
    torch = torch_mod()
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_f32_from_bf16(t):
    return synth.bf16_bits_to_f32(host_bits(t)).astype(np.float64)


def weight_f32(d):
    """The weight of a case as float32 values (fp32 input, or bf16 widened)."""
    W = d["W"]
    return W if W.dtype == np.float32 else synth.bf16_bits_to_f32(W)


def oracle_group_slice(Wf, g0, g1):
    """Oracle quantization of DQ groups [g0, g1) of a flat weight (groups are self-contained)."""
    flat = Wf.reshape(-1)
    lo, hi = g0 * 16384, min(g1 * 16384, flat.size)
    return nf4.quantize_nf4(flat[lo:hi].reshape(1, -1))


def oracle_rows(Wf, rows):
    """W' (bf16 values as float64) of the given weight rows, quantizing only the
    DQ groups that cover them."""
    N, K = Wf.shape
    out = np.empty((len(rows), K), np.float64)
    for i, n in enumerate(rows):
        b0, b1 = n * K // 64, (n + 1) * K // 64
        g0, g1 = b0 // 256, (b1 - 1) // 256 + 1
        qs = oracle_group_slice(Wf, g0, g1)
        Wd = nf4.dequantize_bf16(qs).reshape(-1).astype(np.float64)
        off = n * K - g0 * 16384
        out[i] = Wd[off:off + K]
    return out


def f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def rel_err(G, R):
    return linear.rel_err(G, R)
