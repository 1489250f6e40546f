"""Pins of the oracle's blockwise NF4 quantization, packing and double quantization (CPU only).

Nearest-code selection is checked by brute force in exact rational arithmetic
over all 16 levels; the double-quantization decode (a single-rounding fma) is
checked against the definition of correct rounding; bf16 rounding is checked
against torch's independent CPU conversion.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp, nf4


def _exact_nearest(x, q):
    """Lowest index j minimising |x - q[j]|, in exact rationals."""
    fx = Fraction(float(x))
    d = [abs(fx - Fraction(float(v))) for v in q]
    m = min(d)
    return d.index(m)


@pytest.mark.parametrize("scale", [1.0, 0.02, 3.0e-30, 7.5e3])
def test_nearest_code_bruteforce(scale):
    rng = np.random.default_rng(11)
    q = nf4.codebook()
    W = (rng.standard_normal((8, 128)) * scale).astype(np.float32)
    c = nf4.block_absmax(W)
    codes = nf4.nearest_codes(W, c)
    wb = W.reshape(-1, 64)
    for b in range(wb.shape[0]):
        inv = np.float32(1.0) / c[b]
        for e in range(64):
            x = np.float32(wb[b, e] * inv)
            assert codes[b * 64 + e] == _exact_nearest(x, q), (b, e, x)


def test_ties_go_to_lower_index():
    q = nf4.codebook()
    t = nf4.threshold_midpoints()
    for j in range(15):
        tj = np.float32(t[j])
        block = np.zeros(64, np.float32)
        block[0] = 1.0                       # absmax 1 => x = w exactly
        block[1] = tj
        block[2] = np.nextafter(tj, np.float32(np.inf))
        block[3] = np.nextafter(tj, np.float32(-np.inf))
        codes = nf4.nearest_codes(block, nf4.block_absmax(block))
        for e in (1, 2, 3):
            assert codes[e] == _exact_nearest(block[e], q)
        if float(tj) == t[j]:                # an exact tie: lower index wins
            assert codes[1] == j
    assert codes[0] == 15


def test_codebook_values_round_trip():
    q = nf4.codebook()
    W = np.tile(q, 8).reshape(2, 64).astype(np.float32)   # every block holds +-1 => absmax 1
    qw = nf4.quantize_nf4(W)
    assert np.array_equal(qw["codes_unpacked"], np.tile(np.arange(16, dtype=np.uint8), 8))
    # constant group (absmax 1 everywhere) => decoded constants are exactly 1
    assert np.all(nf4.decode_absmax(qw["absmax_q"], qw["dq_scale"], qw["dq_offset"]) == 1.0)
    assert np.array_equal(nf4.dequantize_f32(qw), W)
    assert np.array_equal(nf4.dequantize_bf16_bits(qw), fp.bf16_bits(W))


def test_absmax_element_maps_to_an_end():
    rng = np.random.default_rng(5)
    W = (rng.standard_t(3, size=(16, 256)) * 0.02).astype(np.float32)
    c = nf4.block_absmax(W)
    codes = nf4.nearest_codes(W, c).reshape(-1, 64)
    wb = W.reshape(-1, 64)
    for b in range(wb.shape[0]):
        e = int(np.argmax(np.abs(wb[b])))
        assert codes[b, e] == (15 if wb[b, e] > 0 else 0)
        x = np.float32(wb[b, e] * (np.float32(1.0) / c[b]))
        assert abs(x) <= 1.0 and abs(x) >= 1.0 - 2.0 ** -23


def test_zero_and_subnormal_blocks_get_zero_code():
    W = np.zeros((1, 192), np.float32)
    W[0, 64:128] = 1e-40          # subnormal absmax
    W[0, 128] = -0.0
    W[0, 129] = np.float32(2.0 ** -126)   # smallest normal: quantized normally
    codes = nf4.nearest_codes(W, nf4.block_absmax(W))
    assert np.all(codes[:128] == 7)
    assert codes[129] == 15 and codes[128] == 7


def test_pack_hand_built_bytes():
    codes = np.array([1, 10, 15, 0, 7, 7, 0, 15], np.uint8)
    packed = nf4.pack_codes(codes)
    assert packed.tolist() == [0xA1, 0x0F, 0x77, 0xF0]
    assert np.array_equal(nf4.unpack_codes(packed), codes)
    # little-endian u32 of 4 bytes holds elements e..e+7 at bits 4*(e mod 8)
    word = int(packed.view(np.uint32)[0])
    assert [(word >> (4 * i)) & 0xF for i in range(8)] == codes.tolist()


def test_double_quant_constant_group_exact():
    c = np.full(256, np.float32(0.0371), np.float32)
    c8, s, o = nf4.double_quantize(c)
    assert s[0] == 0 and np.all(c8 == 0)
    assert np.array_equal(nf4.decode_absmax(c8, s, o), c)


def test_double_quant_extremes_and_bound():
    rng = np.random.default_rng(3)
    c = np.abs(rng.standard_normal(256 * 5 + 37)).astype(np.float32) * np.float32(0.05)
    c[300] = 0.0
    c8, s, o = nf4.double_quantize(c)
    assert s.shape == (6,) and o.shape == (6,)
    dec = nf4.decode_absmax(c8, s, o)
    for g in range(6):
        cg = c[g * 256:(g + 1) * 256]
        c8g = c8[g * 256:(g + 1) * 256]
        d = (cg - o[g]).astype(np.float32)
        h = np.max(np.abs(d))
        assert np.any(np.abs(c8g) == 127)                     # the block achieving h
        assert int(np.abs(c8g[np.argmax(np.abs(d))])) == 127
        # the offset is the midrange, which minimises the largest deviation h:
        # h equals half the range up to rounding
        half_range = (float(cg.max()) - float(cg.min())) / 2
        assert abs(float(h) - half_range) <= 2 * float(np.spacing(np.float32(max(abs(cg.max()), 1e-30))))
        err = np.abs(dec[g * 256:(g + 1) * 256].astype(np.float64) - cg)
        ulp = np.spacing(np.maximum(np.abs(cg), np.abs(o[g]))).astype(np.float64)
        assert np.all(err <= float(s[g]) / 2 + 2 * ulp)


def _check_correctly_rounded(r, exact):
    fr = Fraction(float(r))
    for nb in (np.nextafter(r, np.float32(-np.inf)), np.nextafter(r, np.float32(np.inf))):
        dn = abs(Fraction(float(nb)) - exact)
        dr = abs(fr - exact)
        assert dr < dn or (dr == dn and int(np.array(r, np.float32).view(np.uint32)) & 1 == 0)


def test_fma_single_rounding_against_definition():
    rng = np.random.default_rng(9)
    a = rng.integers(-127, 128, 400).astype(np.float64)
    b = (np.abs(rng.standard_normal(400)) * 10.0 ** rng.integers(-12, 2, 400)).astype(np.float32)
    c = (rng.standard_normal(400) * 10.0 ** rng.integers(-3, 3, 400)).astype(np.float32)
    r = fp.fma_f32(a, b, c)
    n_inexact_in_double = 0
    for i in range(400):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        _check_correctly_rounded(r[i], exact)
        if Fraction(float(a[i]) * float(b[i]) + float(c[i])) != exact:
            n_inexact_in_double += 1
    assert n_inexact_in_double > 0     # the rational fallback was exercised


def test_round_fraction_ties_to_even():
    one = Fraction(1)
    half_ulp = Fraction(1, 2 ** 24)
    assert fp.round_fraction_to_f32(one + half_ulp) == np.float32(1.0)
    r = fp.round_fraction_to_f32(one + 3 * half_ulp)
    assert r == np.float32(1.0 + 2.0 ** -22)


def test_bf16_matches_torch_and_hand_cases():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),          # subnormals
        (rng.standard_normal(2000) * 1e38).astype(np.float32),
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0, 3.3895314e38], np.float32),
    ])
    mine = fp.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert mine[-6] == 0x3F80 and mine[-5] == 0x3F82 and mine[-4] == 0xBF80
    assert mine[-3] == 0x0000 and mine[-2] == 0x8000
    assert np.array_equal(fp.bf16_to_f32(mine).view(np.uint32) >> 16, mine.astype(np.uint32))


def test_group_counts_of_the_workloads():
    def n_groups(N, K):
        return (N * K // 64 + 255) // 256
    assert n_groups(1024, 1024) == 64
    assert n_groups(4096, 4096) == 1024
    assert n_groups(11008, 4096) == 2752
    assert n_groups(8192, 8192) == 4096
    assert n_groups(8192, 22016) == 11008


def test_partial_last_group():
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((3, 64 * 100)) * 0.02).astype(np.float32)   # 300 blocks
    qw = nf4.quantize_nf4(W)
    assert qw["absmax_q"].shape == (300,) and qw["dq_scale"].shape == (2,)
    tail = qw["absmax"][256:]
    c8, s, o = nf4.double_quantize(tail)     # the partial group is a group of its own
    assert np.array_equal(c8, qw["absmax_q"][256:]) and s[0] == qw["dq_scale"][1]
