"""The Python binding checks every tensor's dtype, shape, contiguity and device before
calling the library (the C ABI takes bare pointers, so a mismatched tensor would be read
or written past its end).  Runs on the CPU: a mismatch raises ValueError / TypeError
before anything reaches the library; matching CPU tensors stop at the device check."""

import pytest
import torch

import bit_quantized_lora_nf4_amd as q

N, K, M, r = 256, 128, 8, 4


def _qw():
    return q.NF4Weight(torch.zeros(N * K // 2, dtype=torch.uint8), torch.zeros(N * K // 64, dtype=torch.int8),
                       torch.zeros(2, dtype=torch.float32), torch.zeros(2, dtype=torch.float32), N, K)


def bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


FWD_BAD = [
    dict(X=bf(M, K + 64)),
    dict(X=bf(M, K), A=bf(r, K + 64), B=bf(N, r)),
    dict(X=bf(M, K), A=bf(r, K), B=bf(N, r + 1)),
    dict(X=bf(M, K), A=bf(r, K), B=None),
    dict(X=bf(M, K), Y=bf(M, N - 1)),
    dict(X=bf(M, K), A=bf(r, K), B=bf(N, r), U=bf(M, r + 2)),
    dict(X=bf(M, K), A=bf(r, K), B=bf(N, r), ws=torch.zeros(16, dtype=torch.uint8)),
    dict(X=bf(K, M).t()),  # right shape, not contiguous
]


@pytest.mark.parametrize("kw", FWD_BAD)
def test_linear_fwd_rejects_mismatch(kw):
    kw = dict(kw)
    X = kw.pop("X")
    with pytest.raises(ValueError):
        q.linear_fwd(_qw(), X, **kw)


def test_linear_fwd_dtype_and_device():
    with pytest.raises(TypeError):
        q.linear_fwd(_qw(), torch.zeros(M, K))                 # fp32 X
    with pytest.raises(TypeError, match="CUDA"):
        q.linear_fwd(_qw(), bf(M, K), bf(r, K), bf(N, r))      # shapes fine, not on a GPU


BWD_BAD = [
    dict(dY=bf(M, N + 1), X=bf(M, K)),
    dict(dY=bf(M, N), X=bf(M + 1, K), A=bf(r, K), B=bf(N, r)),
    dict(dY=bf(M, N), X=None, A=bf(r, K), B=bf(N, r)),
    dict(dY=bf(M, N), X=bf(M, K), A=bf(r, K), B=bf(N, r), U=bf(M, r + 1)),
    dict(dY=bf(M, N), X=bf(M, K), A=bf(r, K), B=bf(N, r), dX=bf(M, K - 1)),
    dict(dY=bf(M, N), X=bf(M, K), A=bf(r, K), B=bf(N, r), dA=bf(r, K + 1)),
    dict(dY=bf(M, N), X=bf(M, K), A=bf(r, K), B=bf(N, r), dB=bf(N + 1, r)),
]


@pytest.mark.parametrize("kw", BWD_BAD)
def test_linear_bwd_rejects_mismatch(kw):
    kw = dict(kw)
    dY, X = kw.pop("dY"), kw.pop("X")
    with pytest.raises(ValueError):
        q.linear_bwd(_qw(), dY, X, **kw)


def test_fused_rejects_mismatch():
    with pytest.raises(ValueError):
        q.linear_fwd_fused(_qw(), 2, bf(M, K), bf(3, K), bf(N, 1))           # 3 ranks, 2 parts
    with pytest.raises(ValueError):
        q.linear_fwd_fused(_qw(), 2, bf(M, K), bf(2 * r, K), bf(N, 2 * r))   # B has the stacked rank
    with pytest.raises(ValueError):
        q.linear_bwd_fused(_qw(), 2, bf(M, N), bf(M, K), bf(2 * r, K), bf(N, r), dA=bf(r, K))


def test_dequantize_out_checked():
    with pytest.raises(ValueError):
        q.dequantize(_qw(), out=bf(N, K - 64))
    with pytest.raises(TypeError):
        q.dequantize(_qw(), dtype=torch.float16)
