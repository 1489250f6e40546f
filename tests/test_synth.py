"""The seeded input generators: shapes, dtypes and the distribution features the
workloads name (heavy tails, outlier fraction and magnitude, one zero block per row)."""

import math

import numpy as np


def test_stress_weight_device_features():
    import torch
    from synth.device import stress_weight_device
    N, K = 256, 4096
    W = stress_weight_device([4, 0], N, K, device="cpu")
    assert W.dtype == torch.bfloat16 and tuple(W.shape) == (N, K)
    Wf = W.float().numpy()
    again = stress_weight_device([4, 0], N, K, device="cpu").float().numpy()
    assert np.array_equal(Wf, again)                                   # seeded
    other = stress_weight_device([4, 1], N, K, device="cpu").float().numpy()
    assert not np.array_equal(Wf, other)                               # distinct per key
    blocks = np.abs(Wf).reshape(N, K // 64, 64).max(axis=2)
    assert np.all((blocks == 0).sum(axis=1) >= 1)                      # a zero block in every row
    big = float(np.float32(torch.tensor(50 * 0.02 * math.sqrt(3)).to(torch.bfloat16).float()))
    frac = np.mean(np.abs(Wf) == big)
    assert 0.0007 < frac < 0.0013                                     # 0.1 % outliers at 50 std
    bulk = Wf[(np.abs(Wf) < big) & (Wf != 0)]
    assert abs(np.median(np.abs(bulk)) / 0.02 - 0.765) < 0.05         # median |t(3)| = 0.765
    assert np.mean(np.abs(bulk) > 0.02 * 5.841) > 0.005               # heavy tail: P(|t3| > 5.841) = 1 %
