"""GPU parity of the data-type variants (FP4 levels; FP8-coded and fp32 block constants)
against the oracle (oracle/variants.py), through the C ABI.

Exact checks: codes, stored constants and decode (bf16 and fp32) of qlora_quantize /
qlora_dequantize; the decode inside the GEMM, the small-M GEMV, both dX GEMMs and the
merge kernel, read out through one-hot inputs (each output is the single product
1 * W'[n, k], added to a zero accumulator) and a rank-0 merge (out = W' + 0).
Tolerance checks (2e-2 max-abs-relative, as for the NF4 layer): Y, U, dX, dA, dB
against the float64 oracle on the variant's decoded weight.
"""

import numpy as np
import pytest

import synth
from oracle import linear
from oracle import variants as v
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu
TOL = 2e-2
VARIANTS = [(qt, ct) for qt in (v.QUANT_NF4, v.QUANT_FP4)
            for ct in (v.CONST_DQ_INT8, v.CONST_DQ_FP8, v.CONST_FP32)]
IDS = [f"{'nf4' if qt == 0 else 'fp4'}-{('dq8', 'dqfp8', 'f32')[ct]}" for qt, ct in VARIANTS]


@pytest.fixture(scope="module")
def q():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_lora_nf4_amd as lib
    return lib


def _check(name, G, R, tol=TOL):
    e = gc.rel_err(G, R)
    print(f"  {name}: rel err {e:.3e}", flush=True)
    assert e <= tol, f"{name}: {e}"


def _compare_stored(qw, ref):
    """The device arrays of a quantized weight against the oracle's, bit for bit."""
    assert np.array_equal(qw.codes.cpu().numpy(), ref["codes"])
    if ref["const_type"] == v.CONST_FP32:
        assert qw.absmax_q is None
        assert np.array_equal(qw.absmax.cpu().numpy().view(np.uint32), ref["absmax_f32"].view(np.uint32))
    else:
        assert np.array_equal(qw.absmax_q.cpu().numpy().view(np.uint8), ref["absmax_q"].view(np.uint8))
        assert np.array_equal(qw.dq_scale.cpu().numpy().view(np.uint32), ref["dq_scale"].view(np.uint32))
        assert np.array_equal(qw.dq_offset.cpu().numpy().view(np.uint32), ref["dq_offset"].view(np.uint32))


def _constant_group_weight():
    """4 x 4096 (one group of 256 blocks) whose blocks all have absmax 0.5: h = 0."""
    rng = np.random.default_rng(17)
    W = (rng.uniform(-0.4, 0.4, size=(4, 4096))).astype(np.float32)
    W.reshape(-1, 64)[:, 5] = 0.5
    return W


@pytest.mark.parametrize("qt,ct", VARIANTS, ids=IDS)
@pytest.mark.parametrize("N,K,w_dtype,kind", [(5, 192, "bf16", "normal"), (300, 640, "f32", "stress"),
                                               (1, 64, "f32", "normal"), (257, 1088, "bf16", "stress")])
def test_quantize_dequantize_exact(q, qt, ct, N, K, w_dtype, kind):
    import torch
    print(f"variant quantize qt={qt} ct={ct} N={N} K={K} {w_dtype} {kind}", flush=True)
    d = synth.case(1, K, N, 0, seed=N + K + 10 * qt + ct, w_dtype=w_dtype, w_kind=kind, parts=("W",))
    Wf = gc.weight_f32(d)
    qw, c = q.quantize(gc.dev_weight(d), return_absmax=True, quant_type=qt, const_type=ct)
    Wb = q.dequantize(qw)
    W32 = q.dequantize(qw, dtype=torch.float32)
    torch.cuda.synchronize()
    ref = v.quantize(Wf, qt, ct)
    _compare_stored(qw, ref)
    assert np.array_equal(c.cpu().numpy().view(np.uint32), ref["absmax"].view(np.uint32))
    assert np.array_equal(gc.host_bits(Wb), v.dequantize_bf16_bits(ref))
    assert np.array_equal(W32.cpu().numpy().view(np.uint32), v.dequantize_f32(ref).view(np.uint32))


@pytest.mark.parametrize("qt,ct", VARIANTS, ids=IDS)
def test_constant_group(q, qt, ct):
    """A double-quantization group with equal constants (h = 0, s = 0) decodes exactly."""
    import torch
    W = _constant_group_weight()
    qw = q.quantize(gc.dev_f32(W), quant_type=qt, const_type=ct)
    Wb = q.dequantize(qw)
    torch.cuda.synchronize()
    ref = v.quantize(W, qt, ct)
    _compare_stored(qw, ref)
    assert np.all(v.block_constants(ref) == np.float32(0.5))
    assert np.array_equal(gc.host_bits(Wb), v.dequantize_bf16_bits(ref))


def _plus_zero(bits):
    """bf16 bit patterns with -0 replaced by +0: a sum 0 + 1 * (-0) is +0, so outputs
    that add a decoded -0 (a zero block whose decoded constant is a tiny negative
    number) to the zero accumulator read +0."""
    b = np.array(bits, dtype=np.uint16)
    b[b == 0x8000] = 0
    return b


@pytest.mark.parametrize("qt,ct", VARIANTS, ids=IDS)
@pytest.mark.parametrize("K,N", [(320, 200), (1088, 77)])
def test_kernel_decode_one_hot(q, qt, ct, K, N):
    """The decode inside each kernel equals the oracle's W' bit for bit: X = I gives
    Y = W'^T (GEMM), 16 one-hot rows give 16 columns of W' (GEMV), dY = I gives dX = W'
    (pipelined dX GEMM when N % 8 == 0, the plain one otherwise), rank-0 merge gives W'."""
    import torch
    print(f"variant one-hot qt={qt} ct={ct} K={K} N={N}", flush=True)
    d = synth.case(1, K, N, 0, seed=K + N + qt, w_kind="stress", parts=("W",))
    qw = q.quantize(gc.dev_weight(d), quant_type=qt, const_type=ct)
    ref = v.dequantize_bf16_bits(v.quantize(gc.weight_f32(d), qt, ct))
    Y, _ = q.linear_fwd(qw, torch.eye(K, dtype=torch.bfloat16, device="cuda"))
    cols = np.linspace(0, K - 1, 16).astype(np.int64)
    Xs = torch.zeros((16, K), dtype=torch.bfloat16, device="cuda")
    Xs[torch.arange(16), torch.from_numpy(cols).cuda()] = 1.0
    Ys, _ = q.linear_fwd(qw, Xs)
    dX, _, _ = q.linear_bwd(qw, torch.eye(N, dtype=torch.bfloat16, device="cuda"), None)
    Wm = q.lora_merge(qw, None, None)
    torch.cuda.synchronize()
    ref = _plus_zero(ref)
    assert np.array_equal(_plus_zero(gc.host_bits(Y)), ref.T)
    assert np.array_equal(_plus_zero(gc.host_bits(Ys)), ref[:, cols].T)
    assert np.array_equal(_plus_zero(gc.host_bits(dX)), ref)
    assert np.array_equal(_plus_zero(gc.host_bits(Wm)), ref)


@pytest.mark.parametrize("qt,ct", VARIANTS, ids=IDS)
@pytest.mark.parametrize("M,K,N,r", [(300, 1088, 520, 16), (5, 1088, 200, 8), (130, 256, 96, 64)])
def test_forward_backward(q, qt, ct, M, K, N, r):
    import torch
    print(f"variant linear qt={qt} ct={ct} M={M} K={K} N={N} r={r}", flush=True)
    alpha = 16.0
    d = synth.case(M, K, N, r, seed=M + N + 3 * ct + qt, w_kind="stress")
    qw = q.quantize(gc.dev_weight(d), quant_type=qt, const_type=ct)
    X, A, B = gc.dev_bf16(d["X"]), gc.dev_bf16(d["A"]), gc.dev_bf16(d["B"])
    Y, U = q.linear_fwd(qw, X, A, B, alpha)
    dX, dA, dB = q.linear_bwd(qw, gc.dev_bf16(d["dY"]), X, A, B, alpha, U)
    torch.cuda.synchronize()
    Wd = v.dequantize_bf16(v.quantize(gc.weight_f32(d), qt, ct)).astype(np.float64)
    Xf, Af, Bf, dYf = (gc.f64(d[k]) for k in ("X", "A", "B", "dY"))
    _check("Y", gc.host_f32_from_bf16(Y), linear.forward(Xf, Wd, Af, Bf, alpha, r))
    _check("U", gc.host_f32_from_bf16(U), linear.lora_down(Xf, Af, alpha, r))
    rdX, rdA, rdB = linear.backward(dYf, Xf, Wd, Af, Bf, alpha, r)
    _check("dX", gc.host_f32_from_bf16(dX), rdX)
    _check("dA", gc.host_f32_from_bf16(dA), rdA)
    _check("dB", gc.host_f32_from_bf16(dB), rdB)


@pytest.mark.parametrize("ct", [v.CONST_DQ_FP8, v.CONST_FP32])
def test_concat_rows_variants(q, ct):
    """Concatenation keeps the types; with fp32 constants no group rule applies."""
    import torch
    rows = (100, 156) if ct == v.CONST_FP32 else (256, 100)
    cs = [synth.case(1, 64, n, 0, seed=60 + n, parts=("W",)) for n in rows]
    qws = [q.quantize(gc.dev_weight(c), quant_type=v.QUANT_FP4, const_type=ct) for c in cs]
    fused = q.concat_rows(qws)
    whole = q.quantize(gc.dev_bf16(np.concatenate([c["W"] for c in cs])), quant_type=v.QUANT_FP4,
                       const_type=ct)
    torch.cuda.synchronize()
    assert (fused.quant_type, fused.const_type) == (v.QUANT_FP4, ct)
    _compare_stored(fused, v.quantize(np.concatenate([gc.weight_f32(c) for c in cs]), v.QUANT_FP4, ct))
    assert torch.equal(q.dequantize(fused).view(torch.int16), q.dequantize(whole).view(torch.int16))
