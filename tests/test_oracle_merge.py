"""Pins of the oracle's merge / unmerge (oracle/merge.py): B = 0 is the identity,
the merged linear reproduces the adapter path ([Repro] "失败排查清单" item 6:
logits before and after the merge), and brute force on a tiny shape."""

import numpy as np

import synth
from oracle import linear, merge, nf4
from oracle.fp import bf16_bits, bf16_to_f32


def _case(M=24, K=128, N=40, r=8, seed=5):
    d = synth.case(M, K, N, r, seed=seed)
    Wd = nf4.dequantize_bf16_bits(nf4.quantize_nf4(synth.bf16_bits_to_f32(d["W"])))
    return d, Wd


def test_zero_B_merge_is_identity():
    d, Wd = _case()
    out = merge.merge(Wd, d["A"], np.zeros_like(d["B"]), 16.0, 8)
    assert np.array_equal(out, Wd)
    assert np.array_equal(merge.unmerge(out, d["A"], np.zeros_like(d["B"]), 16.0, 8), Wd)


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    A = bf16_bits(rng.standard_normal((3, 8)).astype(np.float32))
    B = bf16_bits(rng.standard_normal((2, 3)).astype(np.float32))
    W = bf16_bits(rng.standard_normal((2, 8)).astype(np.float32))
    out = merge.merge(W, A, B, 6.0, 3)
    Af, Bf, Wf = (bf16_to_f32(x).astype(np.float64) for x in (A, B, W))
    for n in range(2):
        for k in range(8):
            delta = sum(Bf[n, j] * Af[j, k] for j in range(3))
            v = np.float32(Wf[n, k]) + np.float32(2.0) * np.float32(delta)
            assert out[n, k] == bf16_bits(np.float32(v))


def test_merged_logits_match_adapter_path():
    """X W_m^T against the fp64 adapter path X W'^T + (alpha/r) X A^T B^T: the merge
    only adds the bf16 rounding of W_m (<= 2^-9 relative per weight)."""
    d, Wd = _case(M=32, K=256, N=64, r=16, seed=9)
    alpha, r = 16.0, 16
    Wm = merge.merge(Wd, d["A"], d["B"], alpha, r)
    X = synth.bf16_bits_to_f32(d["X"]).astype(np.float64)
    ref = linear.forward(X, bf16_to_f32(Wd).astype(np.float64), bf16_to_f32(d["A"]).astype(np.float64),
                         bf16_to_f32(d["B"]).astype(np.float64), alpha, r)
    got = X @ bf16_to_f32(Wm).astype(np.float64).T
    assert linear.rel_err(got, ref) < 1e-2
    # and the merged weight differs from the base by the scaled delta, to bf16 rounding
    dW = bf16_to_f32(Wm).astype(np.float64) - bf16_to_f32(Wd).astype(np.float64)
    delta = (alpha / r) * bf16_to_f32(d["B"]).astype(np.float64) @ bf16_to_f32(d["A"]).astype(np.float64)
    assert np.max(np.abs(dW - delta)) <= 2.0 ** -8 * np.max(np.abs(bf16_to_f32(Wm)))


def test_unmerge_inverts_merge_up_to_rounding():
    d, Wd = _case(seed=11)
    Wm = merge.merge(Wd, d["A"], d["B"], 16.0, 8)
    back = bf16_to_f32(merge.unmerge(Wm, d["A"], d["B"], 16.0, 8)).astype(np.float64)
    base = bf16_to_f32(Wd).astype(np.float64)
    # two bf16 roundings: within 2 ulp of the larger magnitude involved
    assert np.max(np.abs(back - base)) <= 2 * 2.0 ** -8 * np.max(np.abs(bf16_to_f32(Wm)))
