"""GPU parity of qlora_lora_merge / qlora_lora_unmerge against the oracle
(oracle/merge.py) on the same seeded inputs, and the logits check before and after a
merge ([Repro] "失败排查清单" items 4 and 6).

The GPU accumulates D = B A in fp32 in its own order, the oracle exactly, so a result
may differ from the oracle's by one bf16 step; every such element must sit on a bf16
rounding boundary to within the fp32 accumulation bound, which the check proves."""

import numpy as np
import pytest

import synth
from oracle import merge, nf4
from oracle.fp import bf16_bits
from tests.gpu_cases import dev_bf16, f64, host_bits, oracle_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_lora_nf4_amd as lib
    return lib


def _scale(alpha, r):
    return float(np.float32(alpha) / np.float32(r)) if r else 0.0


def check_merge(got, want, base, A_bits, B_bits, alpha, r, sign, label):
    """got/want bf16 bits [n, K] (GPU, oracle); base the fp64 values they start from."""
    A = f64(A_bits)
    B = f64(B_bits)
    s = _scale(alpha, r)
    exact = base + sign * s * (B @ A) if r else base
    bound = s * (np.abs(B) @ np.abs(A)) * (r + 2) * 2.0 ** -24 + np.abs(exact) * 2.0 ** -23 if r \
        else np.zeros_like(base)
    bad = got != want
    frac = 1.0 - bad.mean()
    print(f"{label}: {bad.sum()} of {bad.size} differ from the oracle (bit-equal fraction {frac:.6f})",
          flush=True)
    if bad.any():
        g, w, v, b = f64(got[bad]), f64(want[bad]), exact[bad], bound[bad]
        mag = np.maximum(np.abs(g), np.abs(w))
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -133))) - 7)
        assert np.all(np.abs(g - w) <= ulp), f"{label}: a difference of more than one bf16 step"
        assert np.all(np.abs(v - 0.5 * (g + w)) <= b + 2.0 ** -149), \
            f"{label}: a difference away from a rounding boundary"
    assert frac > 0.99, label


def _weight_case(N, K, r, seed):
    d = synth.case(8, K, N, r, seed=seed, parts=("W", "A", "B"))
    return d


# (N, K, r): ragged rows, K below / above one 256-column tile, r not a multiple of 8
# (element-wise B staging), several 64-rank chunks, r = 0 and r = 1.
SMALL = [(40, 128, 8), (100, 320, 16), (64, 512, 64), (33, 192, 70), (96, 256, 256),
         (50, 384, 0), (17, 64, 1), (129, 1024, 40)]


@pytest.mark.parametrize("N,K,r", SMALL)
def test_merge_small(q, N, K, r):
    print(f"merge N={N} K={K} r={r}", flush=True)
    d = _weight_case(N, K, r, seed=N + K + r)
    alpha = 16.0
    Wf = synth.bf16_bits_to_f32(d["W"])
    Wd = nf4.dequantize_bf16_bits(nf4.quantize_nf4(Wf))
    want = merge.merge(Wd, d["A"], d["B"], alpha, r)
    qw = q.quantize(dev_bf16(d["W"]))
    A = dev_bf16(d["A"]) if r else None
    B = dev_bf16(d["B"]) if r else None
    got = host_bits(q.lora_merge(qw, A, B, alpha))
    if r == 0:
        assert np.array_equal(got, Wd)
    check_merge(got, want, f64(Wd), d["A"], d["B"], alpha, r, +1.0, f"merge {N}x{K} r={r}")


@pytest.mark.parametrize("N,K,r", SMALL)
def test_unmerge_small(q, N, K, r):
    print(f"unmerge N={N} K={K} r={r}", flush=True)
    d = _weight_case(N, K, r, seed=7 * N + K + r)
    alpha = 32.0
    Wm = d["W"]  # a seeded bf16 matrix stands in for a merged weight
    want = merge.unmerge(Wm, d["A"], d["B"], alpha, r)
    A = dev_bf16(d["A"]) if r else None
    B = dev_bf16(d["B"]) if r else None
    dWm = dev_bf16(Wm)
    got = host_bits(q.lora_unmerge(dWm, A, B, alpha))
    check_merge(got, want, f64(Wm), d["A"], d["B"], alpha, r, -1.0, f"unmerge {N}x{K} r={r}")
    # in place gives the same bits
    q.lora_unmerge(dWm, A, B, alpha, out=dWm)
    assert np.array_equal(host_bits(dWm), got)


def test_zero_B_merge_is_the_decode(q):
    import torch
    d = _weight_case(256, 1024, 16, seed=3)
    qw = q.quantize(dev_bf16(d["W"]))
    A = dev_bf16(d["A"])
    B = torch.zeros(256, 16, dtype=torch.bfloat16, device="cuda")
    got = host_bits(q.lora_merge(qw, A, B, 16.0))
    Wd = nf4.dequantize_bf16_bits(nf4.quantize_nf4(synth.bf16_bits_to_f32(d["W"])))
    assert np.array_equal(got, Wd)


def _logits(q, N, K, r, M, alpha, seed):
    import torch
    d = synth.case(M, K, N, r, seed=seed, parts=("W", "X", "A", "B"))
    qw = q.quantize(dev_bf16(d["W"]))
    X, A, B = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"])
    Y, _ = q.linear_fwd(qw, X, A, B, alpha)
    Wm = q.lora_merge(qw, A, B, alpha)
    Ym = X.float() @ Wm.float().t()
    Yf = Y.float()
    err = ((Ym - Yf).abs().max() / Yf.abs().max()).item()
    Wmm = q.lora_unmerge(Wm, A, B, -alpha)  # the same update added a second time
    err2 = ((X.float() @ Wmm.float().t() - Yf).abs().max() / Yf.abs().max()).item()
    return err, err2


@pytest.mark.parametrize("N,K,r,alpha", [(1024, 1024, 8, 16.0), (4096, 4096, 64, 16.0)])
def test_logits_before_and_after_merge(q, N, K, r, alpha):
    """[Repro] "失败排查清单" item 6: the merged weight gives the adapter path's logits
    (up to the bf16 rounding of the merged weight and of Y); item 4: a second merge is
    caught by the same check."""
    print(f"logits N={N} K={K} r={r}", flush=True)
    err, err2 = _logits(q, N, K, r, 64, alpha, seed=N + r)
    print(f"  merged vs adapter path: {err:.2e}; merged twice: {err2:.2e}", flush=True)
    assert err < 2e-2
    assert err2 > 10 * err and err2 > 2e-2


# LLaMA-65B layer shapes (d_out, d_in) with r = 64: rows sampled against the oracle.
@pytest.mark.parametrize("N,K", [(8192, 8192), (22016, 8192), (8192, 22016)])
def test_merge_full_size_sampled_rows(q, N, K):
    print(f"merge full size N={N} K={K}", flush=True)
    r, alpha = 64, 16.0
    d = synth.case(8, K, N, r, seed=11, w_std=0.015, parts=("W", "A", "B"))
    qw = q.quantize(dev_bf16(d["W"]))
    got = host_bits(q.lora_merge(qw, dev_bf16(d["A"]), dev_bf16(d["B"]), alpha))
    rows = np.array([0, 1, 31, 32, N // 2 + 5, N - 33, N - 2, N - 1])
    Wf = synth.bf16_bits_to_f32(d["W"])
    Wd = oracle_rows(Wf, rows)
    want = merge.merge(bf16_bits(Wd.astype(np.float32)), d["A"], d["B"][rows], alpha, r)
    check_merge(got[rows], want, Wd, d["A"], d["B"][rows], alpha, r, +1.0, f"merge {N}x{K} rows")


# Block-constant types and level tables other than NF4 + int8 double quantization, with
# ranks that take the workgroup-shared stage of B, the constants and the codes (r <= 64,
# r % 8 == 0): K / 64 odd (a row's blocks not aligned to 4), ragged rows, r below 64.
@pytest.mark.parametrize("qt,ct", [(0, 1), (0, 2), (1, 0), (1, 2)], ids=["nf4-dqfp8", "nf4-f32", "fp4-dq8", "fp4-f32"])
@pytest.mark.parametrize("N,K,r", [(100, 320, 16), (77, 1088, 64), (64, 256, 8)])
def test_merge_variants_with_rank(q, qt, ct, N, K, r):
    from oracle import variants as v
    print(f"merge variant qt={qt} ct={ct} N={N} K={K} r={r}", flush=True)
    d = _weight_case(N, K, r, seed=3 * N + K + r + 10 * ct + qt)
    alpha = 16.0
    Wf = synth.bf16_bits_to_f32(d["W"])
    Wd = v.dequantize_bf16_bits(v.quantize(Wf, qt, ct))
    want = merge.merge(Wd, d["A"], d["B"], alpha, r)
    qw = q.quantize(dev_bf16(d["W"]), quant_type=qt, const_type=ct)
    got = host_bits(q.lora_merge(qw, dev_bf16(d["A"]), dev_bf16(d["B"]), alpha))
    check_merge(got, want, f64(Wd), d["A"], d["B"], alpha, r, +1.0, f"merge qt={qt} ct={ct} {N}x{K} r={r}")
