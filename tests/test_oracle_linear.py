"""Pins of the oracle's forward and backward (CPU only).

* brute-force triple loops on tiny shapes ([Paper note] "关键设计 3" equation,
  [Repro] "LoRA 的公式和张量形状" shapes);
* zero-initialised B leaves the output equal to the frozen base path
  ([Repro] "最小实验与验收协议", no-op init);
* gradients by central differences of L = sum(dY * Y), which are exact up to
  rounding because Y is linear in X, in A and in B separately;
* the adjoint identity <dY, X W'^T> = <dY W', X>;
* decode error bound of the stress weights.
"""

import numpy as np
import pytest

import synth
from oracle import accounting, linear, nf4


def _tiny(seed=0, M=3, K=128, N=5, r=2):
    d = synth.case(M, K, N, r, seed)
    qw = nf4.quantize_nf4(synth.bf16_bits_to_f32(d["W"]))
    Wd = nf4.dequantize_bf16(qw).astype(np.float64)
    f = lambda k: synth.bf16_bits_to_f32(d[k]).astype(np.float64)  # noqa: E731
    return f("X"), Wd, f("A"), f("B"), f("dY")


def _brute_forward(X, W, A, B, alpha, r):
    M, K, N = len(X), len(X[0]), len(W)
    Y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        U = [sum(X[m][k] * A[j][k] for k in range(K)) for j in range(r)]
        for n in range(N):
            base = sum(X[m][k] * W[n][k] for k in range(K))
            lora = sum(U[j] * B[n][j] for j in range(r))
            Y[m][n] = base + (alpha / r) * lora
    return np.array(Y)


def test_forward_matches_brute_force():
    X, W, A, B, _ = _tiny()
    Y = linear.forward(X, W, A, B, 16.0, 2)
    Yb = _brute_forward(X.tolist(), W.tolist(), A.tolist(), B.tolist(), 16.0, 2)
    assert np.max(np.abs(Y - Yb)) <= 1e-12 * np.max(np.abs(Yb))


def test_zero_B_is_the_base_path():
    X, W, A, _, _ = _tiny(1)
    B0 = np.zeros((W.shape[0], 2))
    assert np.array_equal(linear.forward(X, W, A, B0, 16.0, 2), linear.base_forward(X, W))
    assert np.array_equal(linear.forward(X, W, A, B0, 16.0, 0), linear.base_forward(X, W))


def test_zero_weight_leaves_only_the_lora_term():
    d = synth.case(4, 256, 6, 4, 7)
    qw = nf4.quantize_nf4(np.zeros((6, 256), np.float32))
    Wd = nf4.dequantize_bf16(qw)
    assert np.all(Wd == 0)
    X, A, B = (synth.bf16_bits_to_f32(d[k]).astype(np.float64) for k in ("X", "A", "B"))
    Y = linear.forward(X, Wd, A, B, 8.0, 4)
    assert np.array_equal(Y, linear.lora_down(X, A, 8.0, 4) @ B.T) or \
        np.max(np.abs(Y - linear.lora_down(X, A, 8.0, 4) @ B.T)) <= 1e-15 * np.max(np.abs(Y))


def _loss(dY, X, W, A, B, alpha, r):
    return float(np.sum(dY * linear.forward(X, W, A, B, alpha, r)))


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_central_differences(seed):
    alpha, r = 16.0, 2
    X, W, A, B, dY = _tiny(seed)
    dX, dA, dB = linear.backward(dY, X, W, A, B, alpha, r)
    rng = np.random.default_rng(seed)
    h = 0.5
    for name, P, G in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in P.shape)
            Pp, Pm = P.copy(), P.copy()
            Pp[idx] += h
            Pm[idx] -= h
            args = {"X": X, "A": A, "B": B}
            args[name] = Pp
            lp = _loss(dY, args["X"], W, args["A"], args["B"], alpha, r)
            args[name] = Pm
            lm = _loss(dY, args["X"], W, args["A"], args["B"], alpha, r)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - G[idx]) <= 1e-9 * max(1.0, abs(G[idx])), (name, idx, fd, G[idx])


def test_adjoint_identity_and_zero_B_gradient():
    X, W, A, _, dY = _tiny(3)
    lhs = np.sum(dY * linear.base_forward(X, W))
    rhs = np.sum((dY @ W) * X)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    B0 = np.zeros((W.shape[0], 2))
    dX, dA, dB = linear.backward(dY, X, W, A, B0, 16.0, 2)
    assert np.all(dA == 0)
    assert np.array_equal(dX, dY @ W)
    assert np.any(dB != 0)


def test_rel_err_rule():
    assert linear.rel_err(np.zeros(3), np.zeros(3)) == 0.0
    assert linear.rel_err(np.array([0, 1e-30, 0]), np.zeros(3)) == float("inf")
    assert linear.rel_err(np.array([1.0, 2.1]), np.array([1.0, 2.0])) == pytest.approx(0.05)


def test_lora_param_count():
    assert accounting.lora_param_count(8, 4096, 4096) == 65536
    # the 65B-shaped layer (four 8192^2, two 8192->22016, one 22016->8192) at r = 64
    layer = 4 * accounting.lora_param_count(64, 8192, 8192) + 3 * accounting.lora_param_count(64, 8192, 22016)
    assert layer == 9994240


def test_stress_decode_error_bound():
    """|w - w'| <= c*g/2 + |q|*|c - c'| + ulp_bf16(w')/2 + ulp_fp32(q*c'), per element."""
    rng = np.random.default_rng(4)
    W = synth.bf16_bits_to_f32(synth.draw_weight(rng, 16, 22016, 0.02, "bf16", "stress"))
    qw = nf4.quantize_nf4(W)
    q = nf4.codebook().astype(np.float64)
    gaps = np.maximum(np.r_[np.diff(q), 0.0], np.r_[0.0, np.diff(q)])   # widest neighbouring gap
    codes = qw["codes_unpacked"].reshape(-1, 64)
    c = qw["absmax"].astype(np.float64)[:, None]
    cp = nf4.decode_absmax(qw["absmax_q"], qw["dq_scale"], qw["dq_offset"]).astype(np.float64)[:, None]
    wq = nf4.dequantize_bf16(qw).reshape(-1, 64).astype(np.float64)
    w = W.reshape(-1, 64).astype(np.float64)
    bound = c * gaps[codes] / 2 + np.abs(q[codes]) * np.abs(c - cp) \
        + np.spacing(np.abs(wq).astype(np.float32)).astype(np.float64) * 2 ** 16 / 2 \
        + np.spacing(np.abs(q[codes] * cp).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(w - wq) <= bound)
    # all-zero blocks decode to exact zeros
    zero_blocks = np.all(w == 0, axis=1)
    assert zero_blocks.sum() >= 16 and np.all(wq[zero_blocks] == 0)
