"""Exact IEEE-754 helpers for the oracle (test infrastructure only).

The pages fix bf16 as the compute type ([Digest] "4. 方法论", 方法原理; [Paper
note] "关键设计 3": dequantize to bf16 on the fly) but say nothing about
rounding.  The readings used throughout the oracle are:

* fp32 arithmetic is IEEE round-to-nearest-even (numpy float32 ops are);
* fp32 -> bf16 is round-to-nearest-even on the bit pattern;
* the constant decode ``fma(c8, s, o)`` is ONE rounding of the exact value.
"""

from fractions import Fraction

import numpy as np


def bf16_bits(x):
    """Round float32 values to bf16 (RNE); return the 16-bit patterns as uint16.

    Definition of RNE on the top 16 bits: add 0x7FFF plus the lowest kept bit,
    then truncate.  Valid for every finite input (overflow goes to inf, as RNE
    must).  NaN is outside the library's contract and is not handled.
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_fraction_to_f32(q):
    """Correctly rounded (RNE) float32 nearest to the exact rational ``q``."""
    q = Fraction(q)
    if q == 0:
        return np.float32(0.0)
    f = np.float32(float(q))  # within one float32 step of the answer
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - q)
        if best is None or d < best[0]:
            best = (d, cand)
        elif d == best[0]:
            # tie: keep the candidate whose significand is even
            if int(np.array(cand, np.float32).view(np.uint32)) & 1 == 0:
                best = (d, cand)
    return np.float32(best[1])


def fma_f32(a, b, c):
    """Elementwise float32 fma: ``a*b + c`` with a single rounding to float32.

    ``a*b`` must be exact in float64 (true for the constant decode, where
    ``a`` is an int8 code and ``b`` a float32 scale: 8 + 24 significant bits).
    The sum is done in float64; TwoSum tells whether it was exact.  Exact
    sums are then rounded once to float32; the rare inexact ones are redone
    in exact rational arithmetic.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    a, b, c = np.broadcast_arrays(a, b, c)
    if not (np.all(a == np.round(a)) and np.all(np.abs(a) < 2.0**29)):
        raise ValueError("fma_f32: first operand must be a small integer (exact product)")
    p = a * b
    if not np.all(np.isfinite(p)):
        raise ValueError("fma_f32: non-finite product")
    s = p + c
    bb = s - p
    err = (p - (s - bb)) + (c - bb)  # TwoSum error term
    out = s.astype(np.float32)
    bad = np.nonzero(err != 0)
    for idx in zip(*bad):
        exact = Fraction(float(a[idx])) * Fraction(float(b[idx])) + Fraction(float(c[idx]))
        out[idx] = round_fraction_to_f32(exact)
    return out
