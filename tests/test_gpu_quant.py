"""GPU parity of quantization and dequantization: bit-exact against the oracle.

Runs the HIP library through the C ABI (the Python binding only marshals
arguments) and compares codes, int8 constants, fp32 group scale/offset,
first-level constants and decoded weights bit for bit with the oracle run on
the same seeded inputs.
"""

import numpy as np
import pytest

import synth
from oracle import fp, nf4
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_lora_nf4_amd as q
    return q


def _run(lib, d):
    import torch
    qw, c = lib.quantize(gc.dev_weight(d), return_absmax=True)
    torch.cuda.synchronize()
    return {
        "codes": qw.codes.cpu().numpy(),
        "absmax_q": qw.absmax_q.cpu().numpy(),
        "dq_scale": qw.dq_scale.cpu().numpy(),
        "dq_offset": qw.dq_offset.cpu().numpy(),
        "absmax": c.cpu().numpy(),
    }, qw


def _assert_same(got, ref, sl=slice(None)):
    for k in ("codes", "absmax_q", "absmax", "dq_scale", "dq_offset"):
        g = got[k][sl] if k not in ("dq_scale", "dq_offset") else got[k]
        assert g.dtype == ref[k].dtype, k
        assert np.array_equal(g.view(np.uint8), ref[k].view(np.uint8)), \
            f"{k}: {np.count_nonzero(g != ref[k])} mismatches"


CASES = [
    (1, 64, "f32", "normal"),       # a single block, partial group
    (7, 192, "bf16", "normal"),
    (37, 1088, "f32", "stress"),     # ragged last group, outliers, zero blocks
    (64, 4096, "bf16", "normal"),
    (5, 22016, "bf16", "stress"),
    (300, 1024, "f32", "normal"),
]


@pytest.mark.parametrize("N,K,dt,kind", CASES)
def test_quantize_small_bitexact(lib, N, K, dt, kind):
    print(f"quantize case N={N} K={K} {dt} {kind}", flush=True)
    d = synth.case(1, K, N, 0, seed=N + K, w_dtype=dt, w_kind=kind, parts=("W",))
    got, qw = _run(lib, d)
    ref = nf4.quantize_nf4(gc.weight_f32(d))
    _assert_same(got, ref)
    # dequantize: bf16 and fp32, bit-exact
    import torch
    wb = gc.host_bits(lib.dequantize(qw, torch.bfloat16))
    wf = lib.dequantize(qw, torch.float32).cpu().numpy()
    assert np.array_equal(wb, nf4.dequantize_bf16_bits(ref))
    assert np.array_equal(wf.view(np.uint32), nf4.dequantize_f32(ref).view(np.uint32))


def test_quantize_special_blocks(lib):
    """Ties at representable midpoints, absmax elements, zero, -0 and subnormal blocks,
    constant groups (s = 0) and the codebook round trip."""
    q = nf4.codebook()
    t = nf4.threshold_midpoints()
    rows = []
    tie = np.zeros(64, np.float32)
    tie[0] = 1.0
    for j in range(15):
        tie[1 + j] = np.float32(t[j])
        tie[16 + j] = np.nextafter(np.float32(t[j]), np.float32(np.inf))
        tie[31 + j] = np.nextafter(np.float32(t[j]), np.float32(-np.inf))
    rows.append(tie)
    rows.append(np.tile(q, 4))                                   # round trip
    rows.append(np.zeros(64, np.float32))                        # zero block
    z = np.zeros(64, np.float32)
    z[::2] = -0.0
    rows.append(z)                                               # -0 only
    rows.append(np.full(64, 1e-40, np.float32))                  # subnormal absmax
    sm = np.full(64, -3e-39, np.float32)
    sm[5] = np.float32(2.0 ** -126)
    rows.append(sm)                                              # smallest normal absmax
    big = np.linspace(-3e38, 3e38, 64).astype(np.float32)
    rows.append(big)
    W = np.stack(rows + [np.tile(q, 4)] * (256 - len(rows)) + [np.full(64, 0.5, np.float32)] * 256)
    W = W.reshape(-1, 128)                                       # 2 blocks per row
    d = {"W": W.astype(np.float32)}
    got, qw = _run(lib, d)
    ref = nf4.quantize_nf4(W)
    _assert_same(got, ref)
    assert ref["dq_scale"][1] == 0.0                            # the constant group
    import torch
    wb = gc.host_bits(lib.dequantize(qw, torch.bfloat16))
    assert np.array_equal(wb, nf4.dequantize_bf16_bits(ref))
    wf = lib.dequantize(qw, torch.float32).cpu().numpy()
    assert np.array_equal(wf.view(np.uint32), nf4.dequantize_f32(ref).view(np.uint32))


def test_quantize_workload1_full(lib):
    d = synth.workload_linear(1, 0, parts=("W",))
    assert d["W"].dtype == np.float32
    got, _ = _run(lib, d)
    _assert_same(got, nf4.quantize_nf4(d["W"]))


@pytest.mark.parametrize("i", [0, 1])
def test_quantize_workload2_full(lib, i):
    d = synth.workload_linear(2, i, parts=("W",))
    print(f"workload 2 linear {i} W {d['W'].shape}", flush=True)
    got, _ = _run(lib, d)
    _assert_same(got, nf4.quantize_nf4(gc.weight_f32(d)))


def test_quantize_stress_matrix_sampled_groups(lib):
    """One full 8192 x 22016 stress matrix on the GPU; the oracle checks sampled DQ groups
    (each group is self-contained) plus the first and the last."""
    import torch
    rng = np.random.default_rng(123)
    d = synth.workload_linear(5, 0, parts=("W",))
    Wf = gc.weight_f32(d)
    got, qw = _run(lib, d)
    n_groups = got["dq_scale"].size
    assert n_groups == 11008
    groups = sorted(set([0, n_groups - 1] + rng.choice(n_groups, 48, replace=False).tolist()))
    wb = gc.host_bits(lib.dequantize(qw, torch.bfloat16)).reshape(-1)
    for g in groups:
        ref = gc.oracle_group_slice(Wf, g, g + 1)
        e0, e1 = g * 16384, (g + 1) * 16384
        assert np.array_equal(got["codes"][e0 // 2:e1 // 2], ref["codes"]), g
        assert np.array_equal(got["absmax_q"][g * 256:(g + 1) * 256], ref["absmax_q"]), g
        assert np.array_equal(got["absmax"][g * 256:(g + 1) * 256].view(np.uint32),
                              ref["absmax"].view(np.uint32)), g
        assert got["dq_scale"][g] == ref["dq_scale"][0] and got["dq_offset"][g] == ref["dq_offset"][0]
        assert np.array_equal(wb[e0:e1], nf4.dequantize_bf16_bits(ref).reshape(-1)), g


def test_quantize_stress_stream_twelve_matrices(lib):
    """The quantization-stress stream: 12 distinct seeded 8192 x 22016 stress weights (about
    4.3 GB of bf16, drawn on the device), each quantized and decoded on the GPU.  Per matrix
    the first and last DQ groups and 6 random ones are checked bit for bit against the
    oracle (codes, int8 constants, scale, offset, decoded bf16); over all checked groups the
    oracle's per-element decode error stays within its bound, and the error statistics per
    kind of block (bulk Student-t, outlier, all-zero) are printed."""
    import torch
    from oracle import stress
    from synth.device import stress_weight_device
    N, K = 8192, 22016
    n_groups = N * K // 16384
    rng = np.random.default_rng(321)
    std = 0.02 * 3.0 ** 0.5
    W_all, labels_all, qws_ref = [], [], []
    for i in range(12):
        W = stress_weight_device([5, i], N, K)
        qw, c = lib.quantize(W, return_absmax=True)
        wb = lib.dequantize(qw)
        torch.cuda.synchronize()
        groups = sorted(set([0, n_groups - 1] + rng.choice(n_groups, 6, replace=False).tolist()))
        flat = W.view(-1)
        for g in groups:
            e0, e1 = g * 16384, (g + 1) * 16384
            Wg = gc.host_f32_from_bf16(flat[e0:e1]).astype(np.float32).reshape(1, -1)
            ref = nf4.quantize_nf4(Wg)
            assert np.array_equal(qw.codes[e0 // 2:e1 // 2].cpu().numpy(), ref["codes"]), (i, g)
            assert np.array_equal(qw.absmax_q[g * 256:(g + 1) * 256].cpu().numpy(), ref["absmax_q"]), (i, g)
            assert np.array_equal(c[g * 256:(g + 1) * 256].cpu().numpy().view(np.uint32),
                                  ref["absmax"].view(np.uint32)), (i, g)
            assert qw.dq_scale[g].item() == ref["dq_scale"][0] and qw.dq_offset[g].item() == ref["dq_offset"][0]
            assert np.array_equal(gc.host_bits(wb.view(-1)[e0:e1]), nf4.dequantize_bf16_bits(ref).reshape(-1)), (i, g)
            W_all.append(Wg)
            labels_all.append(stress.block_kinds(Wg, outlier_abs=25 * std))
            qws_ref.append(ref)
        print(f"  stress matrix {i}: {len(groups)} groups bit-exact", flush=True)
        del W, qw, c, wb
        torch.cuda.empty_cache()
    report = {}
    for Wg, lab, ref in zip(W_all, labels_all, qws_ref):
        for k, v in stress.error_report(Wg, ref, lab).items():
            agg = report.setdefault(k, {"blocks": 0, "max_err_over_c": 0.0, "sq": 0.0, "n": 0,
                                        "max_err_over_bound": 0.0})
            agg["blocks"] += v["blocks"]
            agg["max_err_over_c"] = max(agg["max_err_over_c"], v["max_err_over_c"])
            agg["sq"] += v["rms_err_over_c"] ** 2 * v["blocks"]
            agg["max_err_over_bound"] = max(agg["max_err_over_bound"], v["max_err_over_bound"])
    for k, v in sorted(report.items()):
        rms = (v["sq"] / v["blocks"]) ** 0.5
        print(f"  {k}: {v['blocks']} blocks, |w - w'|/c max {v['max_err_over_c']:.4f} rms {rms:.4f}, "
              f"error/bound max {v['max_err_over_bound']:.3f}", flush=True)
        assert v["max_err_over_bound"] <= 1.0, k
    assert set(report) == {"bulk", "outlier", "zero"}


def test_quantize_deterministic(lib):
    d = synth.case(1, 4096, 256, 0, seed=5, parts=("W",))
    a, _ = _run(lib, d)
    b, _ = _run(lib, d)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8))
