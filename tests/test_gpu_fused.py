"""GPU parity of the horizontally fused linears (qlora_linear_fwd_fused / _bwd_fused,
qlora_nf4_concat_rows) against the oracle (oracle/fusion.py) and against the parts run
one by one.

Exact checks: the concatenated NF4 arrays equal the GPU quantization of the stacked
matrix and the oracle's appended arrays; Y, the stacked U_s, dA and dB of the fused call
equal the separate calls bit for bit (each output element sees the same operations).
Tolerance checks (2e-2 max-abs-relative, as for the single linear): Y, dX, dA, dB
against the float64 oracle; dX also against the sum of the separate calls' dX.
"""

import numpy as np
import pytest

import synth
from oracle import fusion, nf4
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu
TOL = 2e-2


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


def _parts(P, Np, K, r, M, seed):
    """P seeded linears sharing X (one case each; X and dY taken from part 0 / all)."""
    cs = [synth.case(M, K, Np, r, seed=seed + q, parts=("W", "X", "A", "B", "dY")) for q in range(P)]
    X = cs[0]["X"]
    dY = np.concatenate([c["dY"] for c in cs], axis=1)
    return cs, X, dY


def _stack(q, cs, r):
    import torch
    qws = [q.quantize(gc.dev_bf16(c["W"])) for c in cs]
    fused = q.concat_rows(qws)
    A = torch.cat([gc.dev_bf16(c["A"]) for c in cs]) if r else None
    B = torch.cat([gc.dev_bf16(c["B"]) for c in cs]) if r else None
    return qws, fused, A, B


def test_concat_rows_is_the_stacked_quantization(q):
    cs = [synth.case(4, 256, 256, 4, seed=40 + i, parts=("W",)) for i in range(3)]
    qws = [q.quantize(gc.dev_bf16(c["W"])) for c in cs]
    fused = q.concat_rows(qws)
    whole = q.quantize(gc.dev_bf16(np.concatenate([c["W"] for c in cs])))
    oc = fusion.concat_quantized([nf4.quantize_nf4(synth.bf16_bits_to_f32(c["W"])) for c in cs])
    for key in ("codes", "absmax_q", "dq_scale", "dq_offset"):
        g = getattr(fused, key).cpu().numpy()
        assert np.array_equal(g, getattr(whole, key).cpu().numpy()), key
        assert np.array_equal(g.view(np.uint8), np.asarray(oc[key]).view(np.uint8)), key


# (P, part rows, K, r, M): GEMV path (M <= 16) and GEMM path, ragged K and M, the
# q/k/v (3 parts) and gate/up (2 parts) layouts, and no adapter.
CASES = [(3, 256, 320, 8, 5), (3, 256, 320, 16, 300), (2, 512, 1024, 32, 1), (2, 256, 512, 64, 257),
         (3, 256, 256, 0, 70), (4, 256, 192, 8, 33),
         # M = 16 with X shared by 2 row groups per workgroup (parts of 160 tiles align with
         # the groups), and with parts of 272 tiles, which workgroups of 3 row groups would
         # straddle (one row group per workgroup then)
         (2, 2560, 4096, 8, 16), (2, 4352, 4096, 8, 16)]


@pytest.mark.parametrize("P,Np,K,r,M", CASES)
def test_fused_matches_parts_and_oracle(q, P, Np, K, r, M):
    import torch
    print(f"fused case P={P} Np={Np} K={K} r={r} M={M}", flush=True)
    alpha = 16.0
    cs, Xh, dYh = _parts(P, Np, K, r, M, seed=100 * P + r + M)
    qws, fused, A, B = _stack(q, cs, r)
    X = gc.dev_bf16(Xh)
    dY = gc.dev_bf16(dYh)
    Y, U = q.linear_fwd_fused(fused, P, X, A, B, alpha)
    dX, dA, dB = q.linear_bwd_fused(fused, P, dY, X, A, B, alpha, U)
    # the parts one by one
    Ys, Us, dXs, dAs, dBs = [], [], [], [], []
    for i in range(P):
        Ai = A[i * r:(i + 1) * r].contiguous() if r else None
        Bi = B[i * Np:(i + 1) * Np].contiguous() if r else None
        Yi, Ui = q.linear_fwd(qws[i], X, Ai, Bi, alpha)
        # the backward of a part from the fused call's U_s columns: at M <= 16 the parts'
        # own U_s may round differently (see below)
        Uf = U[:, i * r:(i + 1) * r].contiguous() if r else None
        dXi, dAi, dBi = q.linear_bwd(qws[i], dY[:, i * Np:(i + 1) * Np].contiguous(), X, Ai, Bi, alpha, Uf)
        Ys.append(gc.host_bits(Yi))
        dXs.append(gc.host_f32_from_bf16(dXi))
        if r:
            Us.append(gc.host_bits(Ui))
            dAs.append(gc.host_bits(dAi))
            dBs.append(gc.host_bits(dBi))
    torch.cuda.synchronize()
    if M > 16:
        assert np.array_equal(gc.host_bits(Y), np.concatenate(Ys, axis=1))
        if r:
            assert np.array_equal(gc.host_bits(U), np.concatenate(Us, axis=1))
    else:
        # the small-M forward splits K over a number of waves (and U_s over slices) chosen
        # for the launch's shape, so the fused call and its parts may round their fp32 sums
        # differently
        f32 = lambda bits: synth.bf16_bits_to_f32(bits).astype(np.float64)  # noqa: E731
        _check("Y vs the parts", gc.host_f32_from_bf16(Y), f32(np.concatenate(Ys, axis=1)))
        if r:
            _check("U vs the parts", gc.host_f32_from_bf16(U), f32(np.concatenate(Us, axis=1)))
    if r:
        assert np.array_equal(gc.host_bits(dA), np.concatenate(dAs))
        assert np.array_equal(gc.host_bits(dB), np.concatenate(dBs))
    # oracle
    Wd = np.concatenate([nf4.dequantize_bf16(nf4.quantize_nf4(synth.bf16_bits_to_f32(c["W"])))
                         for c in cs]).astype(np.float64)
    Af = np.concatenate([gc.f64(c["A"]) for c in cs]) if r else None
    Bf = np.concatenate([gc.f64(c["B"]) for c in cs]) if r else None
    Xf, dYf = gc.f64(Xh), gc.f64(dYh)
    _check("Y", gc.host_f32_from_bf16(Y), fusion.forward(Xf, Wd, Af, Bf, alpha, r, P))
    rdX, rdA, rdB = fusion.backward(dYf, Xf, Wd, Af, Bf, alpha, r, P)
    _check("dX", gc.host_f32_from_bf16(dX), rdX)
    _check("dX vs the parts' sum", gc.host_f32_from_bf16(dX), sum(dXs))
    if r:
        _check("dA", gc.host_f32_from_bf16(dA), rdA)
        _check("dB", gc.host_f32_from_bf16(dB), rdB)


@pytest.mark.parametrize("layer", ["qkv", "gate_up"])
def test_fused_full_size(q, layer):
    """LLaMA-65B layer shapes at M = 2048, r = 64: q/k/v (3 x 8192 rows) or gate/up
    (2 x 22016 rows) on K = 8192.  Every output of the fused call against the oracle
    (oracle/fusion.py on the same seeded inputs, float64); Y, dA and dB also bitwise
    against the parts run one by one, dX against the separate calls' sum."""
    import torch
    P, Np = (3, 8192) if layer == "qkv" else (2, 22016)
    K, r, M, alpha = 8192, 64, 2048, 16.0
    print(f"fused full size {layer}: P={P} Np={Np} K={K} M={M}", flush=True)
    cs = [synth.case(M, K, Np, r, seed=700 + i, w_std=0.015) for i in range(P)]
    qws, fused, A, B = _stack(q, cs, r)
    Xh = cs[0]["X"]
    dYh = np.concatenate([c["dY"] for c in cs], axis=1)
    X, dY = gc.dev_bf16(Xh), gc.dev_bf16(dYh)
    Y, U = q.linear_fwd_fused(fused, P, X, A, B, alpha)
    Y0, U0 = Y.clone(), U.clone()
    dX, dA, dB = q.linear_bwd_fused(fused, P, dY, X, A, B, alpha, U)
    assert torch.equal(Y, Y0) and torch.equal(U, U0), "the backward changed its inputs"
    dXsum = torch.zeros(M, K, dtype=torch.float32, device="cuda")
    for i in range(P):
        Ai, Bi = A[i * r:(i + 1) * r].contiguous(), B[i * Np:(i + 1) * Np].contiguous()
        Yi, Ui = q.linear_fwd(qws[i], X, Ai, Bi, alpha)
        # the backward of a part from the fused call's U_s columns: at M <= 16 the parts'
        # own U_s may round differently (see below)
        Uf = U[:, i * r:(i + 1) * r].contiguous() if r else None
        dXi, dAi, dBi = q.linear_bwd(qws[i], dY[:, i * Np:(i + 1) * Np].contiguous(), X, Ai, Bi, alpha, Uf)
        assert torch.equal(Y[:, i * Np:(i + 1) * Np], Yi)
        assert torch.equal(U[:, i * r:(i + 1) * r], Ui)
        assert torch.equal(dA[i * r:(i + 1) * r], dAi)
        assert torch.equal(dB[i * Np:(i + 1) * Np], dBi)
        dXsum += dXi.float()
        del Yi, Ui, dXi, dAi, dBi
    torch.cuda.synchronize()
    _check("dX vs the parts' sum", gc.host_f32_from_bf16(dX), dXsum.cpu().numpy().astype(np.float64))
    Yg, dXg, dAg, dBg = (gc.host_f32_from_bf16(t) for t in (Y, dX, dA, dB))
    del Y, U, dX, dA, dB, dXsum, fused, qws
    torch.cuda.empty_cache()
    Wd = np.concatenate([nf4.dequantize_bf16(nf4.quantize_nf4(synth.bf16_bits_to_f32(c["W"])))
                         for c in cs]).astype(np.float64)
    Af = np.concatenate([gc.f64(c["A"]) for c in cs])
    Bf = np.concatenate([gc.f64(c["B"]) for c in cs])
    Xf, dYf = gc.f64(Xh), gc.f64(dYh)
    _check("Y", Yg, fusion.forward(Xf, Wd, Af, Bf, alpha, r, P))
    rdX, rdA, rdB = fusion.backward(dYf, Xf, Wd, Af, Bf, alpha, r, P)
    _check("dX", dXg, rdX)
    _check("dA", dAg, rdA)
    _check("dB", dBg, rdB)


def test_fused_without_adapter_any_part_height(q):
    """No adapter (r = 0): the fused weight is one linear to the kernels, so part heights
    need not be multiples of 256 (here 100 rows each, M = 40 > 16, the GEMM path; and
    M = 3, the small-M path).  K = 4096 keeps each part's DQ groups whole, as
    concatenation requires."""
    import torch
    P, Np, K = 3, 100, 4096  # 100 rows x 64 blocks = 25 whole DQ groups per part
    cs = [synth.case(40, K, Np, 0, seed=900 + i, parts=("W", "X", "A", "B", "dY")) for i in range(P)]
    qws = [q.quantize(gc.dev_bf16(c["W"])) for c in cs]
    fused = q.concat_rows(qws)
    Wd = np.concatenate([nf4.dequantize_bf16(nf4.quantize_nf4(synth.bf16_bits_to_f32(c["W"])))
                         for c in cs]).astype(np.float64)
    for M in (40, 3):
        Xh = cs[0]["X"][:M]
        X = gc.dev_bf16(Xh)
        Y, U = q.linear_fwd_fused(fused, P, X)
        dYh = np.concatenate([c["dY"][:M] for c in cs], axis=1)
        dX, _, _ = q.linear_bwd_fused(fused, P, gc.dev_bf16(dYh), X)
        torch.cuda.synchronize()
        assert U is None
        _check(f"Y (M={M})", gc.host_f32_from_bf16(Y), fusion.forward(gc.f64(Xh), Wd, None, None, 16.0, 0, P))
        rdX, _, _ = fusion.backward(gc.f64(dYh), gc.f64(Xh), Wd, None, None, 16.0, 0, P)
        _check(f"dX (M={M})", gc.host_f32_from_bf16(dX), rdX)
