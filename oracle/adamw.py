"""AdamW step on the LoRA parameters (test infrastructure only).

[Digest] "方法步骤与流程" step 5: after the backward, an optimizer such as Adam
updates only the adapter matrices; the pages give no formula.  Reading: AdamW
with decoupled weight decay and bias correction (Loshchilov & Hutter), fp32
master parameters and moments, bf16 gradients (the backward's dA, dB), every
element computed by this exact sequence of fp32 operations, each rounded to
nearest-even (no fused multiply-add):

    g     = float(grad)                          bf16 -> fp32, exact
    p1    = p * decay                            decay = fp32(1 - lr * wd)
    m1    = beta1 * m + (1 - beta1) * g
    v1    = beta2 * v + (1 - beta2) * (g * g)
    denom = sqrt(v1) / bc2s + eps                bc2s = fp32(sqrt(1 - beta2^t))
    p2    = p1 - step_size * (m1 / denom)        step_size = fp32(lr / (1 - beta1^t))
    out   = bf16_rne(p2)                         the adapter copy the layer reads

The scalar factors are computed once in double precision from the (double)
hyper-parameters and rounded to fp32.  ``sqrt`` and ``/`` are correctly rounded.
"""

import math

import numpy as np

from .fp import bf16_bits, bf16_to_f32


def step_constants(lr, beta1, beta2, eps, weight_decay, step):
    """fp32 scalars of one step, from double hyper-parameters."""
    lr, beta1, beta2, eps, wd = (float(x) for x in (lr, beta1, beta2, eps, weight_decay))
    f32 = np.float32
    return {
        "decay": f32(1.0 - lr * wd),
        "b1": f32(beta1), "ob1": f32(1.0 - beta1),
        "b2": f32(beta2), "ob2": f32(1.0 - beta2),
        "step_size": f32(lr / (1.0 - beta1 ** step)),
        "bc2s": f32(math.sqrt(1.0 - beta2 ** step)),
        "eps": f32(eps),
    }


def adamw_step(p, grad_bits, m, v, lr, beta1, beta2, eps, weight_decay, step):
    """One step; returns (p, m, v, bf16 bits of p), all new arrays (fp32 / uint16)."""
    c = step_constants(lr, beta1, beta2, eps, weight_decay, step)
    p = np.asarray(p, dtype=np.float32)
    m = np.asarray(m, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    g = bf16_to_f32(grad_bits)
    p1 = p * c["decay"]
    m1 = c["b1"] * m + c["ob1"] * g
    v1 = c["b2"] * v + c["ob2"] * (g * g)
    denom = np.sqrt(v1) / c["bc2s"] + c["eps"]
    p2 = p1 - c["step_size"] * (m1 / denom)
    return p2, m1, v1, bf16_bits(p2)
