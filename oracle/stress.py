"""Decode error of the NF4 + double-quantized weight format and its per-element bound.

Test infrastructure only; see ``oracle/__init__.py`` for the page names.

[Ch. 11.3] "核心创新二：双重量化" and [QLoRA note] "2. NF4" motivate blockwise
constants by outliers: one extreme weight only coarsens the 64-weight block that holds
it.  Double quantization then codes the block constants in groups of 256, so an outlier
block also widens the 8-bit grid of its whole group.  The pages state no error bound.
Reading: for every element, with c the fp32 block absmax, c' its decoded double-quantized
value, q the level table and code the stored index,

    |w - w'| <= c (h(code) + 2^-22) + |q[code]| |c - c'| + u32/2 + u16/2,

derived step by step from the decode chain w' = bf16(RN(q[code] c')):

* the quantizer compares x = RN(w RN(1/c)) with the exact level midpoints, so x lies in
  the half-open interval of its code between the neighbouring midpoints (the ends are
  capped by |x| <= 1); h(code) is the larger distance from q[code] to those interval
  ends (half the gap to a neighbour, one-sided at the two ends of the table);
* |x - w/c| <= 2^-22 |w/c| covers the two roundings of x (relative 2^-24 each);
* |q c - q c'| = |q| |c - c'| is the double-quantization error of the constant;
* u32 is the spacing of float32 at RN(q c'), u16 the spacing of bf16 at w'.

A block whose absmax is zero or subnormal takes the zero code everywhere and decodes to
zeros, so its bound is |w| <= c (zero error for an all-zero block).
"""

import numpy as np

from . import fp, nf4


def half_gaps(q=None):
    """h(code) for each of the 16 codes (float64): the larger distance from q[code]
    to the midpoints with its neighbours; the table ends count one side only."""
    q = nf4.codebook() if q is None else q
    qd = np.asarray(q, dtype=np.float64)
    mids = (qd[:-1] + qd[1:]) / 2.0
    h = np.empty(16)
    for j in range(16):
        lo = qd[j] - mids[j - 1] if j > 0 else 0.0
        hi = mids[j] - qd[j] if j < 15 else 0.0
        h[j] = max(lo, hi)
    return h


def _bf16_spacing(v32):
    """Spacing of bf16 numbers at |v| (float64): 2^(e - 7) for |v| in [2^e, 2^(e+1))."""
    a = np.abs(np.asarray(v32, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    sp = np.ldexp(1.0, (e - 7).astype(np.int64))
    return np.where(a > 0, np.maximum(sp, 2.0 ** -133), 0.0)


def decode_error(W, qw, q=None):
    """Per-element |w - w'|, the bound above, and the block absmax c of each element.

    ``W`` is the quantized input as float32 values [N, K] (bf16 inputs widened exactly);
    ``qw`` is the oracle's ``nf4.quantize_nf4(W)``.  Returns float64 arrays of W's shape.
    """
    q = nf4.codebook() if q is None else q
    W = np.asarray(W, dtype=np.float32)
    shape = W.shape
    codes = nf4.unpack_codes(qw["codes"]).reshape(-1, nf4.BLOCK)
    c = np.asarray(qw["absmax"], dtype=np.float32)
    cp = nf4.decode_absmax(qw["absmax_q"], qw["dq_scale"], qw["dq_offset"])
    v32 = (q[codes] * cp[:, None]).astype(np.float32)            # RN(q[code] c')
    w16 = fp.bf16_to_f32(fp.bf16_bits(v32)).astype(np.float64)    # w'
    err = np.abs(W.reshape(-1, nf4.BLOCK).astype(np.float64) - w16)
    cd = c.astype(np.float64)[:, None]
    qv = np.asarray(q, dtype=np.float64)[codes]
    bound = (cd * (half_gaps(q)[codes] + 2.0 ** -22)
             + np.abs(qv) * np.abs(cd - cp.astype(np.float64)[:, None])
             + np.spacing(np.abs(v32)).astype(np.float64) / 2.0
             + _bf16_spacing(v32) / 2.0)
    # absmax zero or subnormal: every code is the zero level, w' = 0 and |w| <= c
    zero_block = (c < nf4.TINY)[:, None]
    bound = np.where(zero_block, np.broadcast_to(cd, bound.shape), bound)
    return err.reshape(shape), bound.reshape(shape), np.broadcast_to(cd, err.shape).reshape(shape)


def block_kinds(W, outlier_abs):
    """Label each 64-block of W: 'zero' (absmax 0), 'outlier' (an element with
    |w| >= outlier_abs), else 'bulk'.  Returns a string array [n_blocks]."""
    Wb = np.abs(np.asarray(W, dtype=np.float32)).reshape(-1, nf4.BLOCK)
    mx = Wb.max(axis=1)
    kinds = np.full(mx.size, "bulk", dtype=object)
    kinds[mx >= outlier_abs] = "outlier"
    kinds[mx == 0] = "zero"
    return kinds


def error_report(W, qw, block_labels, q=None):
    """Per label: blocks, max and RMS of |w - w'| / c over the label's elements (blocks
    with c = 0 report their plain max error, which must be 0), and the largest ratio of
    the error to its bound (<= 1 when the bound holds).  ``block_labels`` gives one
    label per 64-block."""
    err, bound, c = decode_error(W, qw, q)
    err = err.reshape(-1, nf4.BLOCK)
    bound = bound.reshape(-1, nf4.BLOCK)
    c = c.reshape(-1, nf4.BLOCK)
    labels = np.asarray(block_labels, dtype=object)
    out = {}
    for lab in sorted(set(labels.tolist())):
        m = labels == lab
        e, b, cc = err[m], bound[m], c[m]
        pos = cc > 0
        rel = e[pos] / cc[pos]
        ratio = np.where(b > 0, e / np.where(b > 0, b, 1.0), np.where(e > 0, np.inf, 0.0))
        out[lab] = {
            "blocks": int(m.sum()),
            "max_err_over_c": float(rel.max()) if rel.size else 0.0,
            "rms_err_over_c": float(np.sqrt(np.mean(rel * rel))) if rel.size else 0.0,
            "max_abs_err_zero_c": float(e[~pos].max()) if (~pos).any() else 0.0,
            "max_err_over_bound": float(ratio.max()),
        }
    return out
