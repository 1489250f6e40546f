"""Move seeded synthetic inputs (numpy arrays from ``synth``) to the GPU as torch
tensors.  Plumbing only: no arithmetic of the method."""

import numpy as np


def _torch():
    import torch
    return torch


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> bf16 CUDA tensor."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_f32(a):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_weight(d):
    """The weight of a case on the device: fp32 as drawn, or bf16 bit patterns."""
    W = d["W"]
    return dev_f32(W) if W.dtype == np.float32 else dev_bf16(W)


def stress_weight_device(key, N, K, scale=0.02, outlier_frac=1e-3, outlier_mult=50.0, device="cuda"):
    """A quantization-stress weight [N, K] drawn on the device from a seeded torch
    generator (bf16): scale * Student-t(3), a fraction ``outlier_frac`` of entries
    replaced by +-outlier_mult * std (std = scale * sqrt(3), the std of scale * t(3)),
    and one all-zero 64-block per row.  Student-t(3) is drawn as the ratio
    z0 / sqrt((z1^2 + z2^2 + z3^2) / 3) of independent standard normals.  Fast enough
    for a 4 GB stream of 8192 x 22016 matrices; the host copy of any part of it is the
    input the oracle sees.  ``key`` is a sequence of small non-negative integers."""
    torch = _torch()
    seed = 0
    for k in key:
        seed = (seed * 1000003 + int(k) + 1) % (1 << 62)
    g = torch.Generator(device=device).manual_seed(seed)
    W = torch.empty((N, K), dtype=torch.bfloat16, device=device)
    rows = max(1, (1 << 26) // K)  # about 64 M values per chunk
    std = scale * 3.0 ** 0.5
    for r0 in range(0, N, rows):
        n = min(rows, N - r0)
        z = torch.randn((4, n, K), device=device, generator=g)
        t = z[0] / torch.sqrt((z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / 3.0) * scale
        hit = torch.rand((n, K), device=device, generator=g) < outlier_frac
        sign = torch.randint(0, 2, (n, K), device=device, generator=g).to(torch.float32) * 2.0 - 1.0
        t = torch.where(hit, sign * (outlier_mult * std), t)
        zb = torch.randint(0, K // 64, (n,), device=device, generator=g)
        t.view(n, K // 64, 64)[torch.arange(n, device=device), zb] = 0.0
        W[r0:r0 + n] = t.to(torch.bfloat16)
        del z, t, hit, sign
    return W
