"""Pins of the data-type variants (oracle/variants.py): the FP4 level table against exact
rationals, the FP4 quantizer against brute force, the E4M3 encoding against torch's
float8_e4m3fn conversion (an independent implementation), the FP8-coded and fp32 block
constants against closed-form bounds, and NF4 + int8 DQ against the NF4 oracle."""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import nf4, variants as v


def test_fp4_levels_are_e2m1_over_6():
    q = v.fp4_levels()
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
            Fraction(6)]
    want = sorted({-m / 6 for m in mags} | {m / 6 for m in mags})
    assert len(want) == 15                       # two zeros share one value
    vals = list(q[:8]) + list(q[8:])
    assert q[7] == 0.0 and q[8] == 0.0 and q[0] == -1.0 and q[15] == 1.0
    assert np.all(np.diff(q) >= 0) and np.count_nonzero(np.diff(q) == 0) == 1
    for x in vals:
        nearest = min(want, key=lambda w: abs(Fraction(float(x)) - w))
        assert np.float32(float(nearest)) == x     # each level is its rational rounded once


def test_fp4_quantizer_brute_force():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    qw = v.quantize(W, v.QUANT_FP4, v.CONST_FP32)
    q = v.fp4_levels()
    c = nf4.block_absmax(W)
    x = (W.reshape(-1, 64) * (np.float32(1.0) / c)[:, None].astype(np.float32)).astype(np.float32).reshape(-1)
    codes = qw["codes_unpacked"]
    for xi, ci in zip(x[:2048], codes[:2048]):
        d = abs(Fraction(float(xi)) - Fraction(float(q[ci])))
        for j in range(16):
            dj = abs(Fraction(float(xi)) - Fraction(float(q[j])))
            assert dj >= d                           # no level strictly nearer
            if dj == d and q[j] != q[ci]:
                assert ci < j                        # ties between distinct levels go low
    # the absmax element of every block maps to an end of the table
    blk = W.reshape(-1, 64)
    arg = np.argmax(np.abs(blk), axis=1)
    ends = codes.reshape(-1, 64)[np.arange(blk.shape[0]), arg]
    assert set(ends.tolist()) <= {0, 15}


def test_e4m3_decode_matches_torch():
    torch = pytest.importorskip("torch")
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([v.e4m3_value(c) for c in codes])
    assert np.array_equal(ours, ref)
    assert v.e4m3_value(0x7E) == 448.0


def test_e4m3_encode_matches_torch_and_round_trips():
    torch = pytest.importorskip("torch")
    for c in range(256):
        if (c & 0x7F) == 0x7F or c == 0x80:
            continue
        assert v.e4m3_encode(v.e4m3_value(c)) == c
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 1e-2,
                        rng.standard_normal(20000) * 3e-3]).astype(np.float32)
    x = x[x != 0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(v.e4m3_encode(x), ref)
    # saturation (torch's cast does not saturate, so this is pinned on its own)
    assert v.e4m3_encode(np.float32(1e6)) == 0x7E and v.e4m3_encode(np.float32(-500.0)) == 0xFE


def test_fp8_double_quantization_bounds():
    rng = np.random.default_rng(5)
    c = np.abs(rng.standard_normal(700) * 0.02).astype(np.float32)
    c8, s, o = v.double_quantize_fp8(c)
    cd = v.decode_absmax_fp8(c8, s, o)
    g = np.arange(c.size) // 256
    d = np.abs(c.astype(np.float64) - o[g])
    err = np.abs(cd.astype(np.float64) - c)
    # e4m3 keeps 3 mantissa bits: relative step 2^-3, half of it 2^-4; subnormal step s 2^-9
    bound = d * 2.0 ** -4 + s[g].astype(np.float64) * 2.0 ** -10 + 4 * np.spacing(c).astype(np.float64)
    assert np.all(err <= bound)
    # the block achieving h of each group maps to +-448
    for gi in range(len(s)):
        cg = c[gi * 256:(gi + 1) * 256]
        k = gi * 256 + int(np.argmax(np.abs(cg - o[gi])))
        assert c8[k] in (0x7E, 0xFE)
    # a constant group decodes exactly
    c8, s, o = v.double_quantize_fp8(np.full(256, 0.0123, np.float32))
    assert s[0] == 0 and not c8.any()
    assert np.all(v.decode_absmax_fp8(c8, s, o) == np.float32(0.0123))


def test_fp32_constants_and_nf4_consistency():
    W = synth.bf16_bits_to_f32(synth.case(4, 256, 64, 4, seed=8, parts=("W",))["W"])
    q32 = v.quantize(W, v.QUANT_NF4, v.CONST_FP32)
    assert np.array_equal(v.block_constants(q32), nf4.block_absmax(W))
    ref = nf4.quantize_nf4(W)
    q8 = v.quantize(W, v.QUANT_NF4, v.CONST_DQ_INT8)
    for key in ("codes", "absmax_q", "dq_scale", "dq_offset"):
        assert np.array_equal(q8[key], ref[key])
    assert np.array_equal(v.dequantize_bf16_bits(q8), nf4.dequantize_bf16_bits(ref))
    # a block of table values times an exact power of two round-trips (no rounding anywhere)
    for qt in (v.QUANT_NF4, v.QUANT_FP4):
        lv = v.levels(qt)
        blk = np.tile(lv, 4).reshape(1, 64).astype(np.float32) * np.float32(0.25)
        back = v.dequantize_f32(v.quantize(blk, qt, v.CONST_FP32))
        assert np.array_equal(back, blk)
