"""qlora_linear_fwd_noalloc (the forward that allocates nothing and keeps its
intermediate sums in the library's fixed per-GPU scratch) against qlora_linear_fwd
with a caller workspace: both calls go through the C ABI on the same inputs and must
agree bit for bit (the same kernels run), and both within the 2e-2 oracle tolerance.
Two calls in a row, the second on a smaller input, for the GEMM path (M > 16) and the
small-M path; a shape whose workspace exceeds the scratch is refused before launching."""

import ctypes

import numpy as np
import pytest

import synth
from oracle import linear, nf4
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


def _call_both(q, qw, d, M, r, alpha):
    import torch
    from bit_quantized_lora_nf4_amd import _lib
    N, K = qw.n_rows, qw.n_cols
    X = gc.dev_bf16(d["X"][:M])
    A = gc.dev_bf16(d["A"]) if r else None
    B = gc.dev_bf16(d["B"]) if r else None
    st = torch.cuda.current_stream().cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    # reference: the workspace entry point
    Yw = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Uw = torch.empty(M, max(r, 1), dtype=torch.bfloat16, device="cuda")
    nb = _lib.qlora_workspace_bytes(0, M, K, N, r)
    ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
    _lib.check(_lib.qlora_linear_fwd(qw.descriptor(), X.data_ptr(), M, ptr(A), ptr(B), r, alpha, Yw.data_ptr(),
                                     Uw.data_ptr() if r else None, ws.data_ptr(), ws.numel(), st), "fwd")
    # the entry point without a workspace, U_s saved and not saved
    Yn = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    Un = torch.full((M, max(r, 1)), 7.0, dtype=torch.bfloat16, device="cuda")
    _lib.check(_lib.qlora_linear_fwd_noalloc(qw.descriptor(), X.data_ptr(), M, ptr(A), ptr(B), r, alpha,
                                             Yn.data_ptr(), Un.data_ptr() if r else None, st), "fwd_noalloc")
    Yn2 = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    _lib.check(_lib.qlora_linear_fwd_noalloc(qw.descriptor(), X.data_ptr(), M, ptr(A), ptr(B), r, alpha,
                                             Yn2.data_ptr(), None, st), "fwd_noalloc (no U)")
    torch.cuda.synchronize()
    assert torch.equal(Yn.view(torch.int16), Yw.view(torch.int16))
    assert torch.equal(Yn2.view(torch.int16), Yw.view(torch.int16))
    if r:
        assert torch.equal(Un.view(torch.int16), Uw.view(torch.int16))
    return Yn


@pytest.mark.parametrize("M1,M2", [(300, 40), (16, 3)])
def test_noalloc_matches_workspace_entry(q, M1, M2):
    K, N, r, alpha = 1024, 768, 16, 16.0
    print(f"no-alloc case M1={M1} M2={M2} K={K} N={N} r={r}", flush=True)
    d = synth.case(M1, K, N, r, seed=31 + M1)
    qw = q.quantize(gc.dev_weight(d))
    Wd = nf4.dequantize_bf16(nf4.quantize_nf4(gc.weight_f32(d))).astype(np.float64)
    for M in (M1, M2):  # two calls in a row, the second smaller
        Y = _call_both(q, qw, d, M, r, alpha)
        Xf, Af, Bf = gc.f64(d["X"][:M]), gc.f64(d["A"]), gc.f64(d["B"])
        e = gc.rel_err(gc.host_f32_from_bf16(Y), linear.forward(Xf, Wd, Af, Bf, alpha, r))
        print(f"  M={M}: rel err {e:.3e}", flush=True)
        assert e <= TOL


def test_noalloc_without_adapter(q):
    d = synth.case(64, 512, 320, 0, seed=5)
    qw = q.quantize(gc.dev_weight(d))
    for M in (64, 8):
        _call_both(q, qw, d, M, 0, 16.0)


def test_noalloc_refuses_oversized_scratch(q):
    """A forward whose workspace exceeds the fixed scratch is refused host-side, with a
    message, before anything is launched."""
    from bit_quantized_lora_nf4_amd import _lib
    N, K, M, r = 256, 4096, 65536, 256  # U_s alone is 32 MiB when the caller does not keep it
    need = _lib.qlora_workspace_bytes(0, M, K, N, r)
    assert need > _lib.QLORA_NOALLOC_SCRATCH_BYTES
    w = _lib.qlora_nf4_weight(0x10000, 0x10000, 0x10000, 0x10000, N, K, None, 0, 0)
    st = _lib.qlora_linear_fwd_noalloc(w, 0x10000, M, 0x10000, 0x10000, r, 16.0, 0x10000, None, None)
    assert st == _lib.QLORA_ERR_WORKSPACE
    assert b"scratch" in _lib.load().qlora_last_error()
