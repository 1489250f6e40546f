"""Pins of the fused-linear oracle (oracle/fusion.py): appending separately quantized
weights is the quantization of the stacked matrix when the DQ groups align (and not
otherwise); the fused gradients match autodiff of the three-linear layer; the fused
forward equals one linear with a block-diagonal B."""

import numpy as np
import pytest

import synth
from oracle import fusion, linear, nf4


def _w(N, K, seed):
    return synth.bf16_bits_to_f32(synth.case(4, K, N, 4, seed=seed, parts=("W",))["W"])


def test_concat_is_quantization_of_stacked_matrix():
    Ws = [_w(256, 128, s) for s in (1, 2, 3)]  # 256 * 128 / 64 = 512 blocks: two groups each
    cat = fusion.concat_quantized([nf4.quantize_nf4(W) for W in Ws])
    whole = nf4.quantize_nf4(np.concatenate(Ws))
    for key in ("codes", "absmax_q", "dq_scale", "dq_offset"):
        assert np.array_equal(cat[key], whole[key]), key


def test_misaligned_groups_are_refused_and_differ():
    Ws = [_w(100, 128, 5), 10.0 * _w(100, 128, 6)]  # 200 blocks: a group straddles the seam
    with pytest.raises(ValueError):
        fusion.concat_quantized([nf4.quantize_nf4(W) for W in Ws])
    whole = nf4.quantize_nf4(np.concatenate(Ws))
    parts = [nf4.quantize_nf4(W) for W in Ws]
    # the stacked matrix's first group spans both parts, so its constants differ
    assert not np.array_equal(whole["dq_scale"], np.concatenate([p["dq_scale"] for p in parts]))
    assert not np.array_equal(whole["absmax_q"], np.concatenate([p["absmax_q"] for p in parts]))


def _layer(M=6, K=64, n=32, r=4, P=3, seed=9):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((P * n, K)) * 0.05
    A = rng.standard_normal((P * r, K)) / np.sqrt(r)
    B = rng.standard_normal((P * n, r)) * 0.1
    dY = rng.standard_normal((M, P * n))
    return X, W, A, B, dY, r, P


def test_fused_backward_matches_autodiff():
    torch = pytest.importorskip("torch")
    X, W, A, B, dY, r, P = _layer()
    alpha = 8.0
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=k in ("X", "A", "B"))
         for k, v in dict(X=X, W=W, A=A, B=B).items()}
    n = W.shape[0] // P
    ys = []
    for q in range(P):
        Wq, Aq, Bq = t["W"][q * n:(q + 1) * n], t["A"][q * r:(q + 1) * r], t["B"][q * n:(q + 1) * n]
        ys.append(t["X"] @ Wq.T + (alpha / r) * (t["X"] @ Aq.T) @ Bq.T)
    (torch.cat(ys, dim=1) * torch.tensor(dY)).sum().backward()
    dX, dA, dB = fusion.backward(dY, X, W, A, B, alpha, r, P)
    assert np.allclose(dX, t["X"].grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dA, t["A"].grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dB, t["B"].grad.numpy(), rtol=1e-12, atol=1e-12)


def test_fused_forward_is_one_linear_with_block_diagonal_B():
    X, W, A, B, dY, r, P = _layer(seed=4)
    alpha = 16.0
    n = W.shape[0] // P
    Bbd = np.zeros((P * n, P * r))
    for q in range(P):
        Bbd[q * n:(q + 1) * n, q * r:(q + 1) * r] = B[q * n:(q + 1) * n]
    # one linear of rank P r with the block-diagonal B and scale alpha / r
    Y1 = linear.forward(X, W, A, Bbd, alpha * P, P * r)
    Yf = fusion.forward(X, W, A, B, alpha, r, P)
    assert np.allclose(Y1, Yf, rtol=1e-13, atol=1e-13)
    # and the first part alone is the plain linear
    assert np.allclose(Yf[:, :n], linear.forward(X, W[:n], A[:r], B[:n], alpha, r), rtol=0, atol=0)
