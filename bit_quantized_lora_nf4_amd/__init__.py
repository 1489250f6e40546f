"""QLoRA linear layer (NF4 weight + double-quantized constants + LoRA) for MI355X.

The compute happens in the HIP library ``libqlora_nf4.so`` (C ABI in
``include/qlora_nf4.h``).  This module only marshals torch tensors into that ABI:
torch provides device memory and the current stream.  There is no CPU or PyTorch
fallback; every call fails loudly if the library is missing or the device is not
a gfx950.

    qw = quantize(W)                                   # W [N, K] fp32 or bf16, on the GPU
    Y, U = linear_fwd(qw, X, A, B, alpha)              # Y = X W'^T + (alpha/r) X A^T B^T
    dX, dA, dB = linear_bwd(qw, dY, X, A, B, alpha, U)
    Wm = lora_merge(qw, A, B, alpha)                   # bf16(W' + (alpha/r) B A)
"""

from dataclasses import dataclass

from . import _lib
from ._lib import (QLORA_BF16, QLORA_CONST_DQ_FP8, QLORA_CONST_DQ_INT8, QLORA_CONST_FP32,  # noqa: F401
                   QLORA_F32, QLORA_QUANT_FP4, QLORA_QUANT_NF4, QloraError, qlora_adamw_step,
                   qlora_codebook, qlora_dequantize, qlora_linear_bwd, qlora_linear_bwd_fused,
                   qlora_linear_fwd, qlora_linear_fwd_fused, qlora_linear_fwd_noalloc, qlora_lora_merge,
                   qlora_lora_unmerge,
                   qlora_nf4_codebook, qlora_nf4_concat_rows, qlora_nf4_sizes, qlora_quantize,
                   qlora_quantize_nf4, qlora_workspace_bytes, qlora_workspace_bytes_fused)

__all__ = ["NF4Weight", "quantize", "dequantize", "linear_fwd", "linear_bwd", "workspace",
           "adamw_step", "lora_merge", "lora_unmerge", "concat_rows", "linear_fwd_fused",
           "linear_bwd_fused", "QloraError", "qlora_quantize_nf4", "qlora_dequantize", "qlora_linear_fwd",
           "qlora_linear_bwd", "qlora_nf4_sizes", "qlora_nf4_codebook", "qlora_workspace_bytes",
           "qlora_adamw_step", "qlora_lora_merge", "qlora_lora_unmerge", "qlora_linear_fwd_fused",
           "qlora_linear_bwd_fused", "qlora_workspace_bytes_fused", "qlora_nf4_concat_rows",
           "qlora_quantize", "qlora_codebook", "qlora_linear_fwd_noalloc", "linear_fwd_noalloc", "QLORA_QUANT_NF4", "QLORA_QUANT_FP4", "QLORA_CONST_DQ_INT8",
           "QLORA_CONST_DQ_FP8", "QLORA_CONST_FP32"]


def _torch():
    import torch
    return torch


@dataclass
class NF4Weight:
    """Device arrays of a quantized weight W[n_rows = d_out, n_cols = d_in].  The
    double-quantized constant types use absmax_q / dq_scale / dq_offset; the fp32
    constant type uses absmax (the others are None)."""
    codes: "object"      # uint8 [n_rows * n_cols / 2]
    absmax_q: "object"   # int8 [n_blocks] (int8 codes, or E4M3 bytes for QLORA_CONST_DQ_FP8)
    dq_scale: "object"   # float32 [n_groups]
    dq_offset: "object"  # float32 [n_groups]
    n_rows: int
    n_cols: int
    absmax: "object" = None   # float32 [n_blocks] (QLORA_CONST_FP32)
    quant_type: int = QLORA_QUANT_NF4
    const_type: int = QLORA_CONST_DQ_INT8

    def descriptor(self):
        return _lib.qlora_nf4_weight(self.codes.data_ptr(), _ptr(self.absmax_q), _ptr(self.dq_scale),
                                     _ptr(self.dq_offset), self.n_rows, self.n_cols, _ptr(self.absmax),
                                     self.quant_type, self.const_type)

    @property
    def shape(self):
        return (self.n_rows, self.n_cols)


def _stream(t):
    return _torch().cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _meta(t, dtype, name, shape=None):
    """A torch tensor of ``dtype``, contiguous, of ``shape`` when given."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on(t, name, device=None):
    """On a GPU, and on ``device`` when given."""
    if not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need(t, dtype, name, shape=None, device=None):
    _meta(t, dtype, name, shape)
    _on(t, name, device)


class _Args:
    """Argument checks of one call, done before anything is launched.  The C ABI takes
    bare pointers and sizes its accesses from the weight's shape, M and r, so a tensor
    that does not match would be read or written past its end.  Dtypes, shapes and
    contiguity are checked first for every argument, then the devices."""

    def __init__(self, device):
        self.device = device
        self.seen = []

    def need(self, t, dtype, name, shape=None):
        _meta(t, dtype, name, shape)
        self.seen.append((t, name))
        return t

    def adapter(self, A, B, N, K, R=None, r=None):
        """(A, B) for a weight [N, K]: A [R, K], B [N, r] (R = r for one linear, parts r
        for fused linears).  Returns R, 0 without an adapter."""
        if A is None and B is None:
            return 0
        if A is None or B is None:
            raise ValueError("A and B must both be given or both be None")
        R = A.shape[0] if R is None else R
        r = R if r is None else r
        self.need(A, _torch().bfloat16, "A", (R, K))
        self.need(B, _torch().bfloat16, "B", (N, r))
        return R

    def workspace(self, ws, nbytes):
        if ws is None:
            return
        self.need(ws, _torch().uint8, "ws")
        if ws.numel() < nbytes:
            raise ValueError(f"ws has {ws.numel()} bytes, {nbytes} needed")

    def devices(self):
        for t, name in self.seen:
            _on(t, name, self.device)


def _alloc_weight(n_rows, n_cols, quant_type, const_type, device):
    torch = _torch()
    code_bytes, n_blocks, n_groups = qlora_nf4_sizes(n_rows, n_cols)
    codes = torch.empty(code_bytes, dtype=torch.uint8, device=device)
    if const_type == QLORA_CONST_FP32:
        return NF4Weight(codes, None, None, None, n_rows, n_cols,
                         torch.empty(n_blocks, dtype=torch.float32, device=device), quant_type, const_type)
    return NF4Weight(codes, torch.empty(n_blocks, dtype=torch.int8, device=device),
                     torch.empty(n_groups, dtype=torch.float32, device=device),
                     torch.empty(n_groups, dtype=torch.float32, device=device), n_rows, n_cols,
                     None, quant_type, const_type)


def quantize(W, return_absmax=False, quant_type=QLORA_QUANT_NF4, const_type=QLORA_CONST_DQ_INT8):
    """Blockwise 4-bit quantization of W [n_rows, n_cols] (fp32 or bf16, on the GPU):
    NF4 (or FP4) codes with int8 double-quantized constants by default, FP8-coded
    (QLORA_CONST_DQ_FP8) or plain fp32 constants (QLORA_CONST_FP32) on request."""
    torch = _torch()
    if W.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("W must be float32 or bfloat16")
    if W.dim() != 2:
        raise ValueError(f"W must be 2-D, got shape {tuple(W.shape)}")
    _need(W, W.dtype, "W")
    n_rows, n_cols = W.shape
    qw = _alloc_weight(n_rows, n_cols, quant_type, const_type, W.device)
    c = qw.absmax
    if c is None and return_absmax:
        c = torch.empty(qw.absmax_q.numel(), dtype=torch.float32, device=W.device)
    dt = QLORA_BF16 if W.dtype == torch.bfloat16 else QLORA_F32
    _lib.check(qlora_quantize(W.data_ptr(), dt, n_rows, n_cols, quant_type, const_type, qw.codes.data_ptr(),
                              _ptr(qw.absmax_q), _ptr(qw.dq_scale), _ptr(qw.dq_offset), _ptr(c),
                              _stream(W)), "qlora_quantize")
    return (qw, c) if return_absmax else qw


def dequantize(qw, dtype=None, out=None):
    """W' [n_rows, n_cols]: bf16 (default) or the fp32 product before bf16 rounding."""
    torch = _torch()
    dtype = dtype or torch.bfloat16
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty(qw.shape, dtype=dtype, device=qw.codes.device)
    _meta(out, dtype, "out", qw.shape)
    _on(out, "out", qw.codes.device)
    dt = QLORA_BF16 if dtype == torch.bfloat16 else QLORA_F32
    _lib.check(qlora_dequantize(qw.descriptor(), out.data_ptr(), dt, _stream(out)), "qlora_dequantize")
    return out


def workspace(op, M, K, N, r, device):
    """Allocate the caller workspace for op 0 (forward) or 1 (backward), zeroed: its
    first QLORA_WORKSPACE_HEADER_BYTES bytes are counters and flags of the small-M
    forward that must start at zero (every call leaves them zero)."""
    torch = _torch()
    n = qlora_workspace_bytes(op, M, K, N, r)
    return torch.zeros(max(n, _lib.QLORA_WORKSPACE_HEADER_BYTES), dtype=torch.uint8, device=device)


def linear_fwd(qw, X, A=None, B=None, alpha=16.0, save_u=True, Y=None, U=None, ws=None):
    """Y = bf16(X W'^T + U_s B^T) with U_s = bf16((alpha/r) X A^T).  Returns (Y, U_s or None)."""
    torch = _torch()
    chk = _Args(qw.codes.device)
    K, N = qw.n_cols, qw.n_rows
    if X.dim() != 2:
        raise ValueError(f"X must be 2-D [M, {K}], got shape {tuple(X.shape)}")
    M = X.shape[0]
    chk.need(X, torch.bfloat16, "X", (M, K))
    r = chk.adapter(A, B, N, K)
    if Y is not None:
        chk.need(Y, torch.bfloat16, "Y", (M, N))
    if r and save_u and U is not None:
        chk.need(U, torch.bfloat16, "U", (M, r))
    nbytes = qlora_workspace_bytes(0, M, K, N, r)
    chk.workspace(ws, nbytes)
    chk.devices()
    dev = chk.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if r and save_u and U is None:
        U = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    if ws is None and nbytes > 0:
        ws = workspace(0, M, K, N, r, dev)
    _lib.check(qlora_linear_fwd(qw.descriptor(), X.data_ptr(), M, _ptr(A), _ptr(B), r, float(alpha),
                                Y.data_ptr(), _ptr(U) if save_u else None, _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(X)), "qlora_linear_fwd")
    return Y, (U if save_u else None)


def linear_fwd_noalloc(qw, X, Y, A=None, B=None, alpha=16.0, U=None):
    """linear_fwd into caller-given Y (and U, optional) with no workspace and no allocation:
    the library's fixed per-GPU scratch holds the intermediate sums.  Calls that overlap on
    one GPU race on that scratch."""
    torch = _torch()
    chk = _Args(qw.codes.device)
    K, N = qw.n_cols, qw.n_rows
    if X.dim() != 2:
        raise ValueError(f"X must be 2-D [M, {K}], got shape {tuple(X.shape)}")
    M = X.shape[0]
    chk.need(X, torch.bfloat16, "X", (M, K))
    r = chk.adapter(A, B, N, K)
    chk.need(Y, torch.bfloat16, "Y", (M, N))
    if U is not None:
        chk.need(U, torch.bfloat16, "U", (M, r))
    chk.devices()
    _lib.check(qlora_linear_fwd_noalloc(qw.descriptor(), X.data_ptr(), M, _ptr(A), _ptr(B), r, float(alpha),
                                        Y.data_ptr(), _ptr(U), _stream(X)), "qlora_linear_fwd_noalloc")
    return Y, U


def linear_bwd(qw, dY, X, A=None, B=None, alpha=16.0, U=None, need_dx=True, dX=None, dA=None,
               dB=None, ws=None):
    """(dX, dA, dB) of the QLoRA linear; no gradient for the frozen weight."""
    return _bwd(qw, 1, dY, X, A, B, alpha, U, need_dx, dX, dA, dB, ws)


def _bwd(qw, parts, dY, X, A, B, alpha, U, need_dx, dX, dA, dB, ws):
    torch = _torch()
    chk = _Args(qw.codes.device)
    K, N = qw.n_cols, qw.n_rows
    if dY.dim() != 2:
        raise ValueError(f"dY must be 2-D [M, {N}], got shape {tuple(dY.shape)}")
    M = dY.shape[0]
    chk.need(dY, torch.bfloat16, "dY", (M, N))
    R = 0 if A is None else A.shape[0]
    if R % parts:
        raise ValueError(f"A has {R} rows, not a multiple of n_parts = {parts}")
    r = R // parts
    chk.adapter(A, B, N, K, R=R, r=r)
    if R or X is not None:
        if X is None:
            raise ValueError("X is required when the layer has an adapter")
        chk.need(X, torch.bfloat16, "X", (M, K))
    if U is not None:
        chk.need(U, torch.bfloat16, "U", (M, R))
    if need_dx and dX is not None:
        chk.need(dX, torch.bfloat16, "dX", (M, K))
    nbytes = qlora_workspace_bytes_fused(1, M, K, N, r, parts) if R else 0
    if R:
        if dA is not None:
            chk.need(dA, torch.bfloat16, "dA", (R, K))
        if dB is not None:
            chk.need(dB, torch.bfloat16, "dB", (N, r))
        chk.workspace(ws, nbytes)
    chk.devices()
    dev = chk.device
    if need_dx and dX is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    if R:
        if dA is None:
            dA = torch.empty((R, K), dtype=torch.bfloat16, device=dev)
        if dB is None:
            dB = torch.empty((N, r), dtype=torch.bfloat16, device=dev)
        if ws is None:
            ws = torch.zeros(max(nbytes, _lib.QLORA_WORKSPACE_HEADER_BYTES), dtype=torch.uint8, device=dev)
    fn = qlora_linear_bwd_fused if parts > 1 else None
    dxp = _ptr(dX) if need_dx else None
    wsn = 0 if ws is None else ws.numel()
    if fn is None:
        st = qlora_linear_bwd(qw.descriptor(), dY.data_ptr(), _ptr(X), M, _ptr(A), _ptr(B), r, float(alpha),
                              _ptr(U), dxp, _ptr(dA), _ptr(dB), _ptr(ws), wsn, _stream(dY))
        _lib.check(st, "qlora_linear_bwd")
    else:
        st = fn(qw.descriptor(), parts, dY.data_ptr(), _ptr(X), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(U),
                dxp, _ptr(dA), _ptr(dB), _ptr(ws), wsn, _stream(dY))
        _lib.check(st, "qlora_linear_bwd_fused")
    return (dX if need_dx else None), dA, dB


def adamw_step(param, grad, exp_avg, exp_avg_sq, step, lr, betas=(0.9, 0.999), eps=1e-8,
               weight_decay=0.0, param_bf16=None):
    """In-place AdamW step on an fp32 adapter parameter (any shape, contiguous) with its
    bf16 gradient; optionally writes the bf16 copy the layer reads into ``param_bf16``."""
    torch = _torch()
    _need(param, torch.float32, "param")
    _need(exp_avg, torch.float32, "exp_avg")
    _need(exp_avg_sq, torch.float32, "exp_avg_sq")
    _need(grad, torch.bfloat16, "grad")
    n = param.numel()
    for t, name in ((grad, "grad"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, param has {n}")
    if param_bf16 is not None:
        _need(param_bf16, torch.bfloat16, "param_bf16")
        if param_bf16.numel() != n:
            raise ValueError("param_bf16 size mismatch")
    _lib.check(qlora_adamw_step(param.data_ptr(), _ptr(param_bf16), grad.data_ptr(), exp_avg.data_ptr(),
                                exp_avg_sq.data_ptr(), n, float(lr), float(betas[0]), float(betas[1]),
                                float(eps), float(weight_decay), int(step), _stream(param)),
               "qlora_adamw_step")
    return param


def _adapter(A, B, N, K):
    chk = _Args(None)
    r = chk.adapter(A, B, N, K)
    chk.devices()
    return r


def lora_merge(qw, A, B, alpha=16.0, out=None):
    """bf16 [n_rows, n_cols] weight with the adapter folded in: bf16(W' + (alpha/r) B A)."""
    torch = _torch()
    N, K = qw.shape
    r = _adapter(A, B, N, K)
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=qw.codes.device)
    _need(out, torch.bfloat16, "out", (N, K))
    _lib.check(qlora_lora_merge(qw.descriptor(), _ptr(A), _ptr(B), r, float(alpha), out.data_ptr(),
                                _stream(out)), "qlora_lora_merge")
    return out


def lora_unmerge(Wm, A, B, alpha=16.0, out=None):
    """bf16(Wm - (alpha/r) B A); ``out=Wm`` works in place."""
    torch = _torch()
    _need(Wm, torch.bfloat16, "Wm")
    N, K = Wm.shape
    r = _adapter(A, B, N, K)
    if out is None:
        out = torch.empty_like(Wm)
    _need(out, torch.bfloat16, "out", (N, K))
    _lib.check(qlora_lora_unmerge(Wm.data_ptr(), N, K, _ptr(A), _ptr(B), r, float(alpha), out.data_ptr(),
                                  _stream(Wm)), "qlora_lora_unmerge")
    return out


# ---- horizontally fused linears (shared X; stacked weights and adapters) -------------

def concat_rows(qws):
    """One NF4Weight holding the given weights stacked along rows (every part but the
    last must hold a multiple of 16384 weights so that its DQ groups end with it)."""
    K = qws[0].n_cols
    N = sum(q.n_rows for q in qws)
    out = _alloc_weight(N, K, qws[0].quant_type, qws[0].const_type, qws[0].codes.device)
    _lib.check(qlora_nf4_concat_rows([q.descriptor() for q in qws], out.descriptor(), _stream(out.codes)),
               "qlora_nf4_concat_rows")
    return out


def linear_fwd_fused(qw, n_parts, X, A=None, B=None, alpha=16.0, save_u=True, Y=None, U=None, ws=None):
    """Fused forward of n_parts linears sharing X: A [n_parts r, K] and B [N, r] stack the
    parts' adapters; Y [M, N] holds the parts' outputs side by side."""
    torch = _torch()
    chk = _Args(qw.codes.device)
    K, N = qw.n_cols, qw.n_rows
    if X.dim() != 2:
        raise ValueError(f"X must be 2-D [M, {K}], got shape {tuple(X.shape)}")
    M = X.shape[0]
    chk.need(X, torch.bfloat16, "X", (M, K))
    R = 0 if A is None else A.shape[0]
    if R % n_parts:
        raise ValueError(f"A has {R} rows, not a multiple of n_parts = {n_parts}")
    r = R // n_parts
    chk.adapter(A, B, N, K, R=R, r=r)
    if Y is not None:
        chk.need(Y, torch.bfloat16, "Y", (M, N))
    if r and save_u and U is not None:
        chk.need(U, torch.bfloat16, "U", (M, R))
    nbytes = qlora_workspace_bytes_fused(0, M, K, N, r, n_parts)
    chk.workspace(ws, nbytes)
    chk.devices()
    dev = chk.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if r and save_u and U is None:
        U = torch.empty((M, R), dtype=torch.bfloat16, device=dev)
    if ws is None and nbytes > 0:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    _lib.check(qlora_linear_fwd_fused(qw.descriptor(), n_parts, X.data_ptr(), M, _ptr(A), _ptr(B), r,
                                      float(alpha), Y.data_ptr(), _ptr(U) if save_u else None, _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(X)),
               "qlora_linear_fwd_fused")
    return Y, (U if save_u else None)


def linear_bwd_fused(qw, n_parts, dY, X, A=None, B=None, alpha=16.0, U=None, need_dx=True, dX=None,
                     dA=None, dB=None, ws=None):
    """(dX, dA, dB) of the fused linears; dA and dB are stacked like A and B."""
    return _bwd(qw, n_parts, dY, X, A, B, alpha, U, need_dx, dX, dA, dB, ws)
