"""Pins of oracle/stress.py: the per-element decode error bound of the NF4 + double-
quantized format, and the error report used for the quantization-stress workload.

The bound is checked to hold on ordinary, heavy-tailed and adversarial weights (level
midpoints, the absmax element, zero and subnormal blocks, a group widened by an outlier
block), to be tight on normal weights, and its pieces against values computed by hand
from the printed level table.  The decode inside decode_error is checked against a
scalar decode of single elements.
"""

import math

import numpy as np
import pytest

import synth
from oracle import fp, nf4, stress

# the NF4 level table as printed (7 decimals) by the pages' reading of the codebook
PRINTED = [-1.0, -0.6934942, -0.5225630, -0.3928682, -0.2829018, -0.1837497, -0.0905394, 0.0,
           0.0791337, 0.1600351, 0.2447663, 0.3361187, 0.4384772, 0.5600153, 0.7202957, 1.0]


def _check_bound(W):
    qw = nf4.quantize_nf4(W)
    err, bound, _ = stress.decode_error(W, qw)
    assert np.all(err <= bound), f"bound violated: max ratio {np.max(err / np.maximum(bound, 1e-300))}"
    return err, bound, qw


def test_half_gaps_by_hand():
    h = stress.half_gaps()
    p = PRINTED
    assert abs(h[0] - (p[1] - p[0]) / 2) < 1e-6
    assert abs(h[15] - (p[15] - p[14]) / 2) < 1e-6
    for j in range(1, 15):
        assert abs(h[j] - max(p[j] - p[j - 1], p[j + 1] - p[j]) / 2) < 1e-6
    assert abs(h[15] - 0.13985215) < 1e-7


def test_bound_holds_normal_and_is_tight():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    err, bound, _ = _check_bound(W)
    assert np.max(err / bound) > 0.5  # not vacuous


def test_bound_holds_stress_weights():
    rng = np.random.default_rng(2)
    W = synth.stress_weight(rng, 48, 2048)
    _check_bound(W)
    Wb = synth.bf16_bits_to_f32(synth.to_bf16_bits(W))
    _check_bound(Wb)


def test_bound_holds_adversarial_blocks():
    q = nf4.codebook()
    mids = np.array(nf4.threshold_midpoints(q), dtype=np.float64)
    rows = []
    # c = 1 exactly (an element at +1), the other elements at the exact level midpoints (ties)
    r = np.zeros(64, np.float32)
    r[0] = 1.0
    r[1:16] = mids.astype(np.float32)
    r[16:31] = np.nextafter(mids.astype(np.float32), np.float32(2))
    rows.append(r)
    # the levels themselves scaled by a non-power-of-two absmax
    rows.append((q * np.float32(0.0371)).astype(np.float32).repeat(4))
    # all zero; subnormal absmax; negative absmax element
    rows.append(np.zeros(64, np.float32))
    rows.append(np.full(64, np.float32(1e-40)))
    rows.append(-np.abs(np.linspace(0.001, 0.3, 64, dtype=np.float32)))
    W = np.stack(rows)
    W = np.concatenate([W, np.tile(W[:1] * np.float32(0.01), (3, 1))]).astype(np.float32)
    _check_bound(W)
    # one group (256 blocks) widened by an outlier block: the 8-bit grid of the constants
    # is coarse for every other block of the group, and the bound still holds
    rng = np.random.default_rng(3)
    G = (rng.standard_normal((256, 64)) * 0.02).astype(np.float32)
    G[17, 5] = 1.7320508
    err, bound, qw = _check_bound(G.reshape(16, 1024))
    c = qw["absmax"]
    cp = nf4.decode_absmax(qw["absmax_q"], qw["dq_scale"], qw["dq_offset"])
    rel_dq = np.abs(c.astype(np.float64) - cp) / c
    G2 = G.copy()
    G2[17, 5] = 0.0
    qw2 = nf4.quantize_nf4(G2.reshape(16, 1024))
    rel_dq2 = np.abs(qw2["absmax"].astype(np.float64) -
                     nf4.decode_absmax(qw2["absmax_q"], qw2["dq_scale"], qw2["dq_offset"])) / qw2["absmax"]
    assert np.max(np.delete(rel_dq, 17)) > 4 * np.max(np.delete(rel_dq2, 17))


def test_decode_error_matches_scalar_decode():
    rng = np.random.default_rng(4)
    W = synth.stress_weight(rng, 8, 1024)
    qw = nf4.quantize_nf4(W)
    err, _, cblk = stress.decode_error(W, qw)
    q = nf4.codebook()
    codes = nf4.unpack_codes(qw["codes"])
    for idx in rng.choice(W.size, 200, replace=False):
        b = idx // 64
        g = b // 256
        cp = fp.fma_f32(float(qw["absmax_q"][b]), qw["dq_scale"][g:g + 1], qw["dq_offset"][g:g + 1])[0]
        v = np.float32(q[codes[idx]] * np.float32(cp))
        w16 = float(fp.bf16_to_f32(fp.bf16_bits(np.array([v], np.float32)))[0])
        assert err.reshape(-1)[idx] == abs(float(W.reshape(-1)[idx]) - w16)
        assert cblk.reshape(-1)[idx] == float(np.max(np.abs(W.reshape(-1)[b * 64:(b + 1) * 64])))


def test_report_categories():
    rng = np.random.default_rng(5)
    W = synth.stress_weight(rng, 64, 4096)
    qw = nf4.quantize_nf4(W)
    kinds = stress.block_kinds(W, outlier_abs=25 * 0.02 * math.sqrt(3))
    rep = stress.error_report(W, qw, kinds)
    assert set(rep) == {"zero", "outlier", "bulk"}
    assert rep["zero"]["blocks"] == 64 and rep["zero"]["max_abs_err_zero_c"] == 0.0
    assert rep["outlier"]["blocks"] > 0
    for k, v in rep.items():
        assert v["max_err_over_bound"] <= 1.0, k
        if k != "zero":
            assert 0 < v["rms_err_over_c"] <= v["max_err_over_c"] < 0.5
    # a planted mistake in the decode (dropping the bf16 rounding) shows in the scalar pin,
    # and a bound that omits the double-quantization term fails on the widened group
    with pytest.raises(AssertionError):
        G = (rng.standard_normal((256, 64)) * 0.02).astype(np.float32)
        G[3, 3] = 1.7320508
        qg = nf4.quantize_nf4(G.reshape(16, 1024))
        e, b, c = stress.decode_error(G.reshape(16, 1024), qg)
        codes = nf4.unpack_codes(qg["codes"]).reshape(16, 1024)
        qv = np.abs(nf4.codebook().astype(np.float64)[codes])
        cp = np.repeat(nf4.decode_absmax(qg["absmax_q"], qg["dq_scale"], qg["dq_offset"]), 64).reshape(16, 1024)
        assert np.all(e <= b - qv * np.abs(c - cp))
