"""Pins of the oracle's AdamW step (oracle/adamw.py) to facts other than itself:
torch's own AdamW implementation, and closed forms of Adam's first step."""

import numpy as np
import pytest

from oracle import adamw
from oracle.fp import bf16_bits, bf16_to_f32


def _draw(n, seed):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = bf16_bits(rng.standard_normal(n).astype(np.float32) * 0.1)
    return p, g


def test_matches_torch_adamw_over_steps():
    """Independent implementation: torch.optim.AdamW on the CPU (float32)."""
    torch = pytest.importorskip("torch")
    n, steps = 1000, 5
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
    p, _ = _draw(n, 0)
    rng = np.random.default_rng(1)
    grads = [bf16_bits(rng.standard_normal(n).astype(np.float32) * 0.1) for _ in range(steps)]
    tp = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    q = p.copy()
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.from_numpy(bf16_to_f32(g).copy())
        opt.step()
        q, m, v, _ = adamw.adamw_step(q, g, m, v, lr, b1, b2, eps, wd, t)
    ref = tp.detach().numpy()
    # same update rule, different fp32 operation order: a few ulps of the step
    assert np.max(np.abs(q - ref)) <= 1e-6 * steps
    st = opt.state[tp]
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-5, atol=1e-9)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-5, atol=1e-12)


def test_first_step_is_lr_times_sign():
    """Step 1 from zero moments: m^ = g and v^ = g^2, so the update is lr g / (|g| + eps),
    i.e. lr sign(g) up to eps / |g|."""
    n = 4096
    p, g = _draw(n, 2)
    lr = 1e-2
    q, m, v, _ = adamw.adamw_step(p, g, np.zeros(n), np.zeros(n), lr, 0.9, 0.999, 1e-8, 0.0, 1)
    gf = bf16_to_f32(g).astype(np.float64)
    nz = np.abs(gf) > 1e-3
    step = (p.astype(np.float64) - q.astype(np.float64))[nz]
    np.testing.assert_allclose(step, lr * np.sign(gf[nz]), rtol=1e-4, atol=2e-9)
    np.testing.assert_allclose(m.astype(np.float64), 0.1 * gf, rtol=1e-6, atol=0)
    np.testing.assert_allclose(v.astype(np.float64), 0.001 * gf * gf, rtol=1e-6, atol=0)


def test_zero_gradient_is_pure_weight_decay():
    """g = 0 and zero moments: the parameter is scaled by exactly fp32(1 - lr wd)."""
    n = 1000
    p, _ = _draw(n, 3)
    g = np.zeros(n, np.uint16)
    lr, wd = 1e-3, 0.1
    q, m, v, bits = adamw.adamw_step(p, g, np.zeros(n), np.zeros(n), lr, 0.9, 0.999, 1e-8, wd, 7)
    decay = np.float32(1.0 - lr * wd)
    assert np.array_equal(q, p * decay)
    assert not m.any() and not v.any()
    assert np.array_equal(bits, bf16_bits(q))


def test_bias_correction_constants():
    """Closed forms of the bias corrections at step 1 and in the limit."""
    c1 = adamw.step_constants(1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    assert c1["step_size"] == np.float32(1e-3 / 0.1)
    assert c1["bc2s"] == np.float32(np.sqrt(1 - 0.999))
    cinf = adamw.step_constants(1e-3, 0.9, 0.999, 1e-8, 0.0, 100000)
    assert cinf["step_size"] == np.float32(1e-3)
    assert cinf["bc2s"] == np.float32(1.0)
