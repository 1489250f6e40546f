"""Data-type variants of the blockwise 4-bit format (test infrastructure only).

The pages' ablation compares Float4 (FP4), NF4 and NF4 with double quantization
([Digest] "6. 实验结果与分析", "核心结果分析" item 2 and its figure), and one page writes
the double-quantized constants as c_2^{FP8} ([Digest] "数学公式与关键细节" item 2).
Readings (the pages give no value set for FP4 and no FP8 encoding details):

* Quant type FP4: the OCP E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign,
  divided by 6 so that the block absmax maps to +-1, as the NF4 levels are.  E2M1 has
  two zeros, so the 16 codes index the ascending table
      -1, -2/3, -1/2, -1/3, -1/4, -1/6, -1/12, 0, 0, 1/12, 1/6, 1/4, 1/3, 1/2, 2/3, 1
  (each value computed exactly and rounded once to fp32).  Everything else (blocks,
  nearest code with ties to the lower code, packing, decode) is as for NF4.
* Constant type DQ_FP8: the affine double quantization of the block constants with the
  int8 code replaced by an FP8 E4M3 code (OCP E4M3: 4 exponent bits with bias 7, 3
  mantissa bits, subnormals, largest finite value 448, no infinities): per group of 256
  blocks, o = RN(min + max) * 0.5, d = RN(c - o), h = max|d|, s = RN(h / 448),
  c8 = e4m3(RN(d / s)) rounded to nearest even and saturated at +-448 (h = 0: s = 0 and
  c8 = 0); decode c' = fma(e4m3_value(c8), s, o), one rounding.  A value below zero gets
  the sign bit even when its magnitude rounds to zero.
* Constant type FP32: no double quantization; the fp32 block absmax is stored as is and
  c' = absmax (the pages' 0.5 bit per parameter of constants).
"""

from fractions import Fraction

import numpy as np

from . import fp, nf4

QUANT_NF4, QUANT_FP4 = 0, 1
CONST_DQ_INT8, CONST_DQ_FP8, CONST_FP32 = 0, 1, 2

E2M1_MAGNITUDES = (Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
                   Fraction(4), Fraction(6))
E4M3_MAX = 448.0


def fp4_levels():
    """The 16 FP4 levels (E2M1 / 6), ascending, float32."""
    mags = [m / 6 for m in E2M1_MAGNITUDES]
    vals = [-m for m in reversed(mags)] + list(mags)  # -1 .. -0, +0 .. 1
    # float(Fraction) is correctly rounded to double; none of these values lies on an
    # fp32 rounding midpoint in double, so the second rounding to fp32 is exact-correct
    return np.array([float(v) for v in vals], dtype=np.float32)


def levels(quant_type):
    return nf4.codebook() if quant_type == QUANT_NF4 else fp4_levels()


# ---- FP8 E4M3 -----------------------------------------------------------------

def e4m3_value(code):
    """Exact value of an E4M3 code (0..255; the NaN codes 0x7F / 0xFF are not used)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0:
        return sign * m * 2.0 ** -9          # subnormal: m / 8 * 2^-6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_POS_VALUES = np.array([e4m3_value(c) for c in range(0x7F)])  # codes 0x00 .. 0x7E, ascending


def e4m3_encode(x):
    """E4M3 codes (uint8) of float32 values: the nearest representable magnitude, ties to
    the even code (whose last mantissa bit is 0), saturated at 448; the sign bit is set
    when x < 0.  Works on scalars and arrays."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    lo = np.clip(np.searchsorted(_POS_VALUES, a, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    dlo = a - _POS_VALUES[lo]              # exact in double: few significant bits
    dhi = _POS_VALUES[hi] - a
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code | np.where(x < 0, 0x80, 0x00)
    return code.astype(np.uint8) if code.ndim else np.uint8(code)


def double_quantize_fp8(absmax):
    """FP8-coded double quantization: (c8 uint8 E4M3 codes [n_blocks], s [n_groups], o)."""
    c = np.asarray(absmax, dtype=np.float32).reshape(-1)
    nb = c.size
    ng = (nb + nf4.GROUP - 1) // nf4.GROUP
    c8 = np.zeros(nb, dtype=np.uint8)
    s_out = np.zeros(ng, dtype=np.float32)
    o_out = np.zeros(ng, dtype=np.float32)
    for g in range(ng):
        cg = c[g * nf4.GROUP:(g + 1) * nf4.GROUP]
        mn, mx = np.min(cg), np.max(cg)
        o = np.float32(np.float32(mn + mx) * np.float32(0.5))
        d = (cg - o).astype(np.float32)
        h = np.float32(np.max(np.abs(d)))
        o_out[g] = o
        if h == 0:
            continue
        s = np.float32(h / np.float32(E4M3_MAX))
        s_out[g] = s
        x = (d / s).astype(np.float32)
        c8[g * nf4.GROUP:g * nf4.GROUP + cg.size] = e4m3_encode(x)
    return c8, s_out, o_out


def decode_absmax_fp8(c8, s, o):
    """c'_b = fma(e4m3_value(c8_b), s_g, o_g), rounded once to float32."""
    c8 = np.asarray(c8, dtype=np.uint8).reshape(-1)
    # every E4M3 value is an integer multiple of 2^-9 (at most 4 significant bits), so
    # value * s = (value * 2^9) * (s * 2^-9) with both factors exact in double
    table = np.array([e4m3_value(v) * 512.0 if (v & 0x7F) != 0x7F else np.nan for v in range(256)])
    g = np.arange(c8.size) // nf4.GROUP
    s64 = np.asarray(s, np.float32).astype(np.float64) * 2.0 ** -9
    return fp.fma_f32(table[c8], s64[g], np.asarray(o, np.float32)[g])


# ---- quantize / decode for any (quant type, constant type) ----------------------

def quantize(W, quant_type=QUANT_NF4, const_type=CONST_DQ_INT8):
    """Blockwise 4-bit quantization of W[d_out, d_in] with the given level table and
    block-constant encoding.  Returns a dict with the stored arrays."""
    W = np.asarray(W, dtype=np.float32)
    if W.ndim != 2 or W.shape[1] % nf4.BLOCK:
        raise ValueError("W must be 2-D with d_in a multiple of 64")
    c = nf4.block_absmax(W)
    codes = nf4.nearest_codes(W, c, levels(quant_type))
    out = {"shape": W.shape, "quant_type": quant_type, "const_type": const_type,
           "codes": nf4.pack_codes(codes), "codes_unpacked": codes, "absmax": c}
    if const_type == CONST_DQ_INT8:
        out["absmax_q"], out["dq_scale"], out["dq_offset"] = nf4.double_quantize(c)
    elif const_type == CONST_DQ_FP8:
        out["absmax_q"], out["dq_scale"], out["dq_offset"] = double_quantize_fp8(c)
    elif const_type == CONST_FP32:
        out["absmax_f32"] = c.copy()
    else:
        raise ValueError("unknown constant type")
    return out


def block_constants(qw):
    """The decoded block constants c' of a quantized weight."""
    ct = qw["const_type"]
    if ct == CONST_DQ_INT8:
        return nf4.decode_absmax(qw["absmax_q"], qw["dq_scale"], qw["dq_offset"])
    if ct == CONST_DQ_FP8:
        return decode_absmax_fp8(qw["absmax_q"], qw["dq_scale"], qw["dq_offset"])
    return np.asarray(qw["absmax_f32"], dtype=np.float32)


def dequantize_f32(qw):
    """RN(q[code] * c'_b) as float32 [d_out, d_in]."""
    q = levels(qw["quant_type"])
    codes = nf4.unpack_codes(qw["codes"])
    vals = q[codes].reshape(-1, nf4.BLOCK) * block_constants(qw)[:, None]
    return vals.astype(np.float32).reshape(qw["shape"])


def dequantize_bf16_bits(qw):
    return fp.bf16_bits(dequantize_f32(qw))


def dequantize_bf16(qw):
    return fp.bf16_to_f32(dequantize_bf16_bits(qw))
