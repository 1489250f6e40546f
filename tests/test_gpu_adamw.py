"""GPU parity of qlora_adamw_step against the oracle's AdamW step (oracle/adamw.py):
bit-exact on the fp32 parameter and moments and on the bf16 copy, over several steps,
ragged sizes, and the parameter count of the LLaMA-65B layer's adapters (r = 64 on
q, k, v, o, gate, up, down: 9,994,240 values)."""

import numpy as np
import pytest

from oracle import adamw
from oracle.fp import bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_lora_nf4_amd as q
    return q


HP = dict(lr=2e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)


def _run(lib, n, steps, seed, with_bf16=True):
    import torch
    print(f"adamw n={n} steps={steps}", flush=True)
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [bf16_bits(rng.standard_normal(n).astype(np.float32) * 0.05) for _ in range(steps)]
    dp = torch.from_numpy(p.copy()).cuda()
    dm = torch.zeros(n, dtype=torch.float32, device="cuda")
    dv = torch.zeros(n, dtype=torch.float32, device="cuda")
    db = torch.empty(n, dtype=torch.bfloat16, device="cuda") if with_bf16 else None
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    bits = None
    for t, g in enumerate(grads, start=1):
        dg = torch.from_numpy(g.view(np.int16).copy()).view(torch.bfloat16).cuda()
        lib.adamw_step(dp, dg, dm, dv, t, HP["lr"], HP["betas"], HP["eps"], HP["weight_decay"], param_bf16=db)
        p, m, v, bits = adamw.adamw_step(p, g, m, v, HP["lr"], HP["betas"][0], HP["betas"][1], HP["eps"],
                                          HP["weight_decay"], t)
    torch.cuda.synchronize()
    assert np.array_equal(dp.cpu().numpy().view(np.uint32), p.view(np.uint32))
    assert np.array_equal(dm.cpu().numpy().view(np.uint32), m.view(np.uint32))
    assert np.array_equal(dv.cpu().numpy().view(np.uint32), v.view(np.uint32))
    if with_bf16:
        assert np.array_equal(db.cpu().view(torch.int16).numpy().view(np.uint16), bits)


@pytest.mark.parametrize("n", [1, 3, 4, 1000, 65536 + 5])
def test_adamw_bitexact_small(lib, n):
    _run(lib, n, 3, seed=n)


def test_adamw_without_bf16_copy(lib):
    _run(lib, 4099, 2, seed=7, with_bf16=False)


def test_adamw_65b_layer_adapters(lib):
    """r (d_in + d_out) summed over the seven linears of the 65B layer ([Repro] "LoRA 的公式和张量形状")."""
    n = 4 * 64 * (8192 + 8192) + 2 * 64 * (8192 + 22016) + 64 * (22016 + 8192)
    assert n == 9_994_240
    _run(lib, n, 2, seed=65)
