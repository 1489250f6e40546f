"""NF4 codebook, blockwise NF4 quantization and double quantization (oracle).

Test infrastructure only; see ``oracle/__init__.py`` for the page names.

What the pages fix, and the readings taken where they are silent:

* Codebook ([QLoRA note] "2. NF4"; [Paper note] "关键设计 1", quantile
  equation; [Digest] "数学公式与关键细节" item 1, q_i equation and "特点"):
  2^k = 16 values built from N(0,1) quantiles, each bin holding the same
  probability mass, normalised to [-1, 1], with zero represented exactly by
  treating the negative and positive halves asymmetrically.  The printed
  midpoint formula has no index range (i = 0 would need the quantile at 0).
  Reading: 7 negative levels, an exact 0 and 8 positive levels.  Each half
  takes quantiles on an equally spaced probability grid from 1/2 to
  delta = 31/32, which is the probability centre of the outermost of 16
  equal-mass bins (the midpoint rule applied to the one bin whose outer
  quantile is infinite).  Both halves are divided by the quantile at delta,
  so the ends are exactly -1 and +1.  Values are computed in double and
  rounded once to float32.
* Blocks ([Ch. 11.3] "核心创新二"; [Digest] item 2): 64 weights per block,
  one absmax constant each.  Reading: 64 consecutive elements of one row of
  W[d_out, d_in] (row-major flattening; d_in % 64 == 0).
* Rescale and nearest code ([QLoRA note] "2. NF4"): divide by the block
  absmax, take the nearest codebook value, store its 4-bit index.  Readings:
  x = RN(w * RN(1/c)); ties between two levels go to the lower index; a
  block whose absmax is zero or subnormal gets the zero code (7) everywhere.
* Packing: two codes per byte (0.5 byte per parameter, [Ch. 11.3]
  "核心创新一").  Reading: the even element sits in the low nibble.
* Double quantization ([Digest] item 2; [Paper note] "关键设计 2";
  [Ch. 11.3] "核心创新二"): the fp32 block constants are quantized again to
  8 bits in groups of 256 with one fp32 second-level constant per group.
  Reading: affine symmetric int8 with a per-group fp32 scale and offset:
  o = RN(min+max) * 0.5, s = RN(h/127) with h = max|RN(c - o)|,
  c8 = clamp(rint_even(RN(RN(c - o) / s)), -127, 127); decode
  c' = fma(c8, s, o) with one rounding.  Groups are 256 consecutive blocks
  in flat block order; the last group may be partial.
* Weight decode ([Digest] item 3, doubleDequant equation):
  w' = bf16_RNE(RN(q[code] * c')).
"""

from statistics import NormalDist

import numpy as np

from . import fp

BLOCK = 64          # weights per first-level block
GROUP = 256         # first-level constants per double-quantization group
DELTA = 31.0 / 32.0  # outermost probability level (see module docstring)
ZERO_CODE = 7
TINY = np.float32(2.0 ** -126)  # smallest normal float32


def _phi_inv(p):
    """Standard-normal quantile (Wichura's AS241, via ``statistics``)."""
    return NormalDist().inv_cdf(p)


def codebook_levels_f64(phi_inv=_phi_inv):
    """The 16 NF4 levels in double precision, ascending, ends exactly -1 and +1."""
    z = phi_inv(DELTA)
    neg = [-phi_inv(0.5 + j * (DELTA - 0.5) / 7.0) / z for j in range(1, 8)]
    pos = [phi_inv(0.5 + j * (DELTA - 0.5) / 8.0) / z for j in range(1, 9)]
    levels = sorted(neg) + [0.0] + pos
    levels[0] = -1.0
    levels[-1] = 1.0
    return levels


def codebook(phi_inv=_phi_inv):
    """NF4 codebook q[0..15] as float32 (q[0] = -1, q[7] = 0, q[15] = +1)."""
    return np.array(codebook_levels_f64(phi_inv), dtype=np.float32)


def threshold_midpoints(q=None):
    """Exact midpoints t_j = (q[j] + q[j+1]) / 2 as Python floats (exact in double)."""
    q = codebook() if q is None else q
    return [(float(q[j]) + float(q[j + 1])) / 2.0 for j in range(15)]


def thresholds(q=None):
    """T_j = the largest float32 <= t_j, so that for float32 x: x > T_j <=> x > t_j."""
    out = np.empty(15, dtype=np.float32)
    for j, t in enumerate(threshold_midpoints(q)):
        f = np.float32(t)
        if float(f) > t:
            f = np.nextafter(f, np.float32(-np.inf))
        out[j] = f
    return out


def block_absmax(w):
    """c_b = max |w| over each block of 64 consecutive elements (float32)."""
    w = np.asarray(w, dtype=np.float32).reshape(-1, BLOCK)
    return np.max(np.abs(w), axis=1)


def nearest_codes(w, absmax, q=None, chunk_blocks=1 << 16):
    """Unpacked 4-bit codes (uint8, one per element) for float32 weights ``w``."""
    T = thresholds(q)
    w = np.asarray(w, dtype=np.float32).reshape(-1, BLOCK)
    absmax = np.asarray(absmax, dtype=np.float32)
    codes = np.empty(w.shape, dtype=np.uint8)
    for b0 in range(0, w.shape[0], chunk_blocks):
        wb = w[b0:b0 + chunk_blocks]
        cb = absmax[b0:b0 + chunk_blocks]
        normal = cb >= TINY
        inv = np.where(normal, np.float32(1.0) / np.where(normal, cb, np.float32(1.0)), np.float32(0.0))
        x = wb * inv.astype(np.float32)[:, None]                # RN(w * RN(1/c)), float32
        code = np.zeros(wb.shape, dtype=np.uint8)
        for j in range(15):
            code += (x > T[j]).astype(np.uint8)                  # #{j : x > T_j}
        code[~normal] = ZERO_CODE
        codes[b0:b0 + chunk_blocks] = code
    return codes.reshape(-1)


def pack_codes(codes):
    """Two codes per byte: element 2i in the low nibble, element 2i+1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        raise ValueError("odd number of codes")
    return (c[0::2] & 0xF) | ((c[1::2] & 0xF) << 4)


def unpack_codes(packed):
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0xF
    out[1::2] = p >> 4
    return out


def double_quantize(absmax):
    """8-bit double quantization of the block constants, groups of 256.

    Returns (c8 int8 [n_blocks], s float32 [n_groups], o float32 [n_groups]).
    """
    c = np.asarray(absmax, dtype=np.float32).reshape(-1)
    nb = c.size
    ng = (nb + GROUP - 1) // GROUP
    c8 = np.zeros(nb, dtype=np.int8)
    s_out = np.zeros(ng, dtype=np.float32)
    o_out = np.zeros(ng, dtype=np.float32)
    for g in range(ng):
        cg = c[g * GROUP:(g + 1) * GROUP]
        mn, mx = np.min(cg), np.max(cg)
        o = np.float32(np.float32(mn + mx) * np.float32(0.5))
        d = (cg - o).astype(np.float32)
        h = np.float32(np.max(np.abs(d)))
        o_out[g] = o
        if h == 0:
            s_out[g] = np.float32(0.0)
            continue
        s = np.float32(h / np.float32(127.0))
        s_out[g] = s
        r = np.rint((d / s).astype(np.float32))                  # half to even
        c8[g * GROUP:(g + 1) * GROUP] = np.clip(r, -127, 127).astype(np.int8)
    return c8, s_out, o_out


def decode_absmax(c8, s, o):
    """c'_b = fma(c8_b, s_g, o_g) rounded once to float32 (g = b // 256)."""
    c8 = np.asarray(c8, dtype=np.int8).reshape(-1)
    g = np.arange(c8.size) // GROUP
    return fp.fma_f32(c8.astype(np.float64), np.asarray(s, np.float32)[g], np.asarray(o, np.float32)[g])


def quantize_nf4(W):
    """Blockwise NF4 + double quantization of W[d_out, d_in] (float32 or bf16-as-float32).

    Returns a dict with the stored format (``codes`` packed uint8,
    ``absmax_q`` int8, ``dq_scale`` and ``dq_offset`` float32) plus the
    first-level constants ``absmax`` (float32) and the unpacked codes.
    """
    W = np.asarray(W, dtype=np.float32)
    if W.ndim != 2 or W.shape[1] % BLOCK:
        raise ValueError("W must be 2-D with d_in a multiple of 64")
    c = block_absmax(W)
    codes = nearest_codes(W, c)
    c8, s, o = double_quantize(c)
    return {
        "shape": W.shape,
        "codes": pack_codes(codes),
        "codes_unpacked": codes,
        "absmax": c,
        "absmax_q": c8,
        "dq_scale": s,
        "dq_offset": o,
    }


def dequantize_f32(qw, q=None):
    """float32 weights RN(q[code] * c'_b), shape [d_out, d_in]."""
    q = codebook() if q is None else q
    codes = unpack_codes(qw["codes"])
    cprime = decode_absmax(qw["absmax_q"], qw["dq_scale"], qw["dq_offset"])
    vals = q[codes].reshape(-1, BLOCK) * cprime[:, None]        # float32 multiply, RN
    return vals.astype(np.float32).reshape(qw["shape"])


def dequantize_bf16_bits(qw, q=None):
    """bf16 weights W' = bf16_RNE(RN(q[code] * c'_b)) as uint16 bit patterns."""
    return fp.bf16_bits(dequantize_f32(qw, q))


def dequantize_bf16(qw, q=None):
    """W' widened back to float32 (exact), for use in the contractions."""
    return fp.bf16_to_f32(dequantize_bf16_bits(qw, q))
