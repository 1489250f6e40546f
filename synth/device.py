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
