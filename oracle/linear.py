"""Forward and backward of the QLoRA linear layer in float64 (oracle).

Test infrastructure only; see ``oracle/__init__.py`` for the page names.

Shapes follow [Repro] "LoRA 的公式和张量形状": W0 is [d_out, d_in] = [N, K],
A is [r, K], B is [N, r], X is [M, K], Y and dY are [M, N]:

    Y = X W'^T + (alpha/r) (X A^T) B^T

with W' the bf16 dequantized weight ([Digest] "数学公式与关键细节" item 3;
[Paper note] "关键设计 3", equation and ``qlora_linear`` listing).  The
[Digest] equation omits alpha/r; the other pages and the LoRA scaling
``lora_alpha / r`` of [Repro] include it, and so does this oracle.

Backward ([Digest] "方法步骤与流程" step 4; [QLoRA note] "5. QLoRA 训练方式本身"):
gradients flow through W' to the LoRA weights only; W gets no gradient.
With U = X A^T and V = (alpha/r) dY B:

    dX = dY W' + V A,    dB = (alpha/r) dY^T U,    dA = V^T X

Every operand is widened exactly to float64 and each formula is evaluated
with plain float64 matmuls; no intermediate rounding to bf16 takes place.
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def forward(X, Wd, A, B, alpha, r):
    """Y = X W'^T + (alpha/r) (X A^T) B^T in float64. ``Wd`` is W' [N, K]."""
    X, Wd = _f64(X), _f64(Wd)
    Y = X @ Wd.T
    if r > 0:
        Y = Y + (alpha / r) * ((X @ _f64(A).T) @ _f64(B).T)
    return Y


def base_forward(X, Wd):
    """The frozen path alone, X W'^T."""
    return _f64(X) @ _f64(Wd).T


def lora_down(X, A, alpha, r):
    """U_s = (alpha/r) X A^T, the scaled down-projection [M, r]."""
    return (alpha / r) * (_f64(X) @ _f64(A).T)


def backward(dY, X, Wd, A, B, alpha, r):
    """Return (dX, dA, dB) in float64.  No gradient for the frozen W."""
    dY, X, Wd = _f64(dY), _f64(X), _f64(Wd)
    dX = dY @ Wd
    if r == 0:
        return dX, None, None
    A, B = _f64(A), _f64(B)
    scale = alpha / r
    V = scale * (dY @ B)                 # [M, r]
    dX = dX + V @ A
    dB = scale * (dY.T @ (X @ A.T))      # [N, r]
    dA = V.T @ X                         # [r, K]
    return dX, dA, dB


def rel_err(G, R):
    """max|G - R| / max|R|; if R is all zero, G must be all zero (returns 0 or inf)."""
    G, R = _f64(G), _f64(R)
    den = np.max(np.abs(R)) if R.size else 0.0
    num = np.max(np.abs(G - R)) if R.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
