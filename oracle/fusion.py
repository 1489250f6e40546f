"""Horizontally fused linears that read the same X (test infrastructure only).

[Ch. 11.3] and [Paper note] apply LoRA to every linear layer of a decoder block; the
query, key and value projections (and the gate and up projections) all read the same
input.  Fusing P such linears stacks their frozen weights along rows and their
adapters: A_cat [P r, K] (part q in rows [q r, q r + r)), B_cat [N, r] (part q in rows
[q N/P, (q + 1) N/P)).  What the fused layer computes is, by definition, the P separate
linears:

    Y[:, part q]   = X W_q'^T + (alpha/r) (X A_q^T) B_q^T
    dX             = sum_q dY_q W_q' + (alpha/r) (dY_q B_q) A_q      (X feeds every part)
    dA, dB         = the parts' own gradients, stacked like A_cat and B_cat

Weights quantized separately concatenate into the quantization of the stacked matrix
when every part but the last ends on a double-quantization group boundary (a multiple
of 256 blocks): the stored arrays are then simply appended.
"""

import numpy as np

from . import linear
from .nf4 import BLOCK

GROUP = 256


def concat_quantized(qws):
    """Append the stored arrays of row-stacked quantized weights (dicts of quantize_nf4)."""
    K = qws[0]["shape"][1]
    for q in qws[:-1]:
        if (q["shape"][0] * K // BLOCK) % GROUP:
            raise ValueError("a part's double-quantization groups would straddle the next part")
    cat = lambda key: np.concatenate([q[key] for q in qws])  # noqa: E731
    return {
        "shape": (sum(q["shape"][0] for q in qws), K),
        "codes": cat("codes"),
        "absmax_q": cat("absmax_q"),
        "dq_scale": cat("dq_scale"),
        "dq_offset": cat("dq_offset"),
    }


def split_rows(M, parts):
    """The parts' row blocks (None stays None: no adapter)."""
    if M is None:
        return [None] * parts
    n = M.shape[0] // parts
    return [M[q * n:(q + 1) * n] for q in range(parts)]


def forward(X, Wd_cat, A_cat, B_cat, alpha, r, parts):
    """Y [M, N] of the fused linears in float64 (the parts' outputs side by side)."""
    Ws, As, Bs = split_rows(Wd_cat, parts), split_rows(A_cat, parts), split_rows(B_cat, parts)
    return np.concatenate([linear.forward(X, Ws[q], As[q], Bs[q], alpha, r) for q in range(parts)], axis=1)


def backward(dY, X, Wd_cat, A_cat, B_cat, alpha, r, parts):
    """(dX, dA_cat, dB_cat) of the fused linears in float64."""
    Ws, As, Bs = split_rows(Wd_cat, parts), split_rows(A_cat, parts), split_rows(B_cat, parts)
    n = Wd_cat.shape[0] // parts
    dX = 0.0
    dAs, dBs = [], []
    for q in range(parts):
        dXq, dAq, dBq = linear.backward(dY[:, q * n:(q + 1) * n], X, Ws[q], As[q], Bs[q], alpha, r)
        dX = dX + dXq
        dAs.append(dAq)
        dBs.append(dBq)
    if r == 0:
        return dX, None, None
    return dX, np.concatenate(dAs), np.concatenate(dBs)
