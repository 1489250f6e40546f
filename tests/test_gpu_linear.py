"""GPU parity of the QLoRA linear forward and backward against the float64 oracle.

Tolerance (stated for the forward, dX, dA and dB): max|G - R| / max|R| <= 2e-2 with
R the oracle in float64 on the same bf16 operands; the measured error is printed.
Exact checks: Y(B = 0) == Y(r = 0) bitwise; X = I gives Y = W'^T bitwise (one
nonzero term per output); B = 0 gives dA == 0; repeated runs are bitwise equal.
Full-size workloads compare every output element with the oracle.
"""

import numpy as np
import pytest

import synth
from oracle import linear, nf4
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_lora_nf4_amd as q
    return q


def _oracle_w(d):
    return nf4.dequantize_bf16(nf4.quantize_nf4(gc.weight_f32(d))).astype(np.float64)


def _dev(d, r):
    X = gc.dev_bf16(d["X"])
    A = gc.dev_bf16(d["A"]) if r else None
    B = gc.dev_bf16(d["B"]) if r else None
    return X, A, B


def _check(name, G, R, tol=TOL):
    e = gc.rel_err(G, R)
    print(f"  {name}: rel err {e:.3e}", flush=True)
    assert e <= tol, f"{name}: {e}"
    return e


SMALL = [  # (M, K, N, r)
    (77, 320, 200, 8),
    (300, 1088, 520, 16),
    (257, 256, 257, 64),
    (33, 64, 1, 4),
    (600, 640, 96, 0),
    (300, 128, 300, 24),
    (5, 192, 77, 3),       # M <= 16: the GEMV path, odd rank
    (16, 4096, 300, 16),
    (1, 1024, 1000, 8),
    (17, 512, 260, 32),    # just above the GEMV bound
    (513, 768, 640, 128),  # rank 128
    (130, 256, 136, 256),  # the largest rank
    (2100, 1024, 512, 64), # several M-splits in the token reductions
    (7, 512, 300, 256),    # M <= 16 with the largest rank: 16 LoRA workgroups in the launch
    (260, 512, 392, 96),   # 96 ranks: LoRA tiles of 12 chunks per row (no swizzle), B read untransposed
    (200, 384, 264, 40),   # 40 ranks: a partly filled second rank tile
    (1000, 128, 20380, 16),  # 320 output tiles in two rounds, ragged both ways
    (1, 64, 33, 5),        # M <= 16 with one 64-block of contraction
    (12, 4096, 40, 16),    # M <= 16, X too large to stage in LDS: X fragments from memory
    (1, 64, 65552, 4),     # M = 1 past 4096 tiles of 16 rows: the fused GEMM takes it
    (3, 256, 48, 256),     # more LoRA pieces than workgroups: a LoRA wave takes several
    (1, 1024, 48, 64),     # the same with the U_s hand-over through per-workgroup counters
    (16, 1024, 520, 8),    # M = 16 with that hand-over (M r within its bound)
    (16, 4096, 7990, 16),  # X staged once for 2 row groups per workgroup (one per CU), ragged last tile
    (16, 4096, 11008, 16), # 3 row groups per workgroup; the last workgroup holds one
    (12, 4096, 5000, 0),   # row groups without an adapter
    (16, 8256, 200, 16),   # X too large to stage for the workgroup: each weight wave stages its own slices (odd K/64)
    (9, 10240, 72, 0),     # the same with an odd M and no adapter
    (16, 9216, 4096, 24),  # the same at 256 tiles (one workgroup per CU)
]


@pytest.mark.parametrize("M,K,N,r", SMALL)
def test_forward_backward_small(lib, M, K, N, r):
    import torch
    print(f"linear case M={M} K={K} N={N} r={r}", flush=True)
    alpha = 16.0
    d = synth.case(M, K, N, r, seed=M * 7 + N)
    qw = lib.quantize(gc.dev_weight(d))
    X, A, B = _dev(d, r)
    Y, U = lib.linear_fwd(qw, X, A, B, alpha)
    dYt = gc.dev_bf16(d["dY"])
    dX, dA, dB = lib.linear_bwd(qw, dYt, X, A, B, alpha, U)
    torch.cuda.synchronize()
    Wd = _oracle_w(d)
    Xf, Af, Bf, dYf = (gc.f64(d[k]) for k in ("X", "A", "B", "dY"))
    _check("Y", gc.host_f32_from_bf16(Y), linear.forward(Xf, Wd, Af, Bf, alpha, r))
    rdX, rdA, rdB = linear.backward(dYf, Xf, Wd, Af, Bf, alpha, r)
    _check("dX", gc.host_f32_from_bf16(dX), rdX)
    if r:
        _check("U", gc.host_f32_from_bf16(U), linear.lora_down(Xf, Af, alpha, r))
        _check("dA", gc.host_f32_from_bf16(dA), rdA)
        _check("dB", gc.host_f32_from_bf16(dB), rdB)


@pytest.mark.parametrize("M", [40, 3])
def test_zero_B_equals_base_bitwise(lib, M):
    import torch
    K, N, r, alpha = 512, 384, 16, 16.0
    d = synth.case(M, K, N, r, seed=99)
    qw = lib.quantize(gc.dev_weight(d))
    X, A, _ = _dev(d, r)
    B0 = torch.zeros((N, r), dtype=torch.bfloat16, device="cuda")
    Y0, _ = lib.linear_fwd(qw, X, A, B0, alpha)
    Yb, _ = lib.linear_fwd(qw, X)
    dYt = gc.dev_bf16(d["dY"])
    dX0, dA0, dB0 = lib.linear_bwd(qw, dYt, X, A, B0, alpha)
    dXb, _, _ = lib.linear_bwd(qw, dYt, X)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Yb.view(torch.int16))
    assert torch.equal(dX0.view(torch.int16), dXb.view(torch.int16))
    assert torch.count_nonzero(dA0.float()) == 0
    assert torch.count_nonzero(dB0.float()) > 0


@pytest.mark.parametrize("M,K,N", [(256, 256, 200), (320, 320, 77)])
def test_identity_input_gives_weight_bitwise(lib, M, K, N):
    """X = I (M = K): every output is a single product 1 * W'[n, k], so Y = W'^T exactly."""
    import torch
    d = synth.case(1, K, N, 0, seed=K, parts=("W",))
    qw = lib.quantize(gc.dev_weight(d))
    X = torch.eye(K, dtype=torch.bfloat16, device="cuda")
    Y, _ = lib.linear_fwd(qw, X)
    torch.cuda.synchronize()
    ref = nf4.dequantize_bf16_bits(nf4.quantize_nf4(gc.weight_f32(d))).T
    assert np.array_equal(gc.host_bits(Y), ref)
    # the transposed decode of the backward: dY = I (M = N) gives dX = W' exactly
    dY = torch.eye(N, dtype=torch.bfloat16, device="cuda")
    dX, _, _ = lib.linear_bwd(qw, dY, None)
    torch.cuda.synchronize()
    assert np.array_equal(gc.host_bits(dX), ref.T)


@pytest.mark.parametrize("const_type", [0, 1, 2])
@pytest.mark.parametrize("N", [640, 644])
def test_deterministic(lib, N, const_type):
    """Repeated calls are bitwise equal, for every block-constant type and both dX kernels
    (N % 8 == 0 takes the pipelined one, N = 644 the plain one), forward at M > 16 and
    M <= 16 (M = 5 hands U_s over through the ticket path, M = 1 through the per-workgroup
    counters).  A wait that does not cover its loads would show as a run-to-run difference."""
    import torch
    M, K, r = 700, 1024, 64
    d = synth.case(M, K, N, r, seed=3)
    qw = lib.quantize(gc.dev_weight(d), const_type=const_type)
    X5 = gc.dev_bf16(d["X"][:5])
    X1 = gc.dev_bf16(d["X"][:1])
    X, A, B = _dev(d, r)
    dYt = gc.dev_bf16(d["dY"])
    outs = []
    for _ in range(3):
        Y, U = lib.linear_fwd(qw, X, A, B, 16.0)
        g = lib.linear_bwd(qw, dYt, X, A, B, 16.0, U)
        Y5, U5 = lib.linear_fwd(qw, X5, A, B, 16.0)
        Y1, U1 = lib.linear_fwd(qw, X1, A, B, 16.0)
        outs.append([Y.clone(), U.clone(), *[t.clone() for t in g], Y5.clone(), U5.clone(), Y1.clone(), U1.clone()])
    torch.cuda.synchronize()
    for later in outs[1:]:
        for a, b in zip(outs[0], later):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("const_type", [0, 1, 2])
def test_deterministic_per_wave_x_staging(lib, const_type):
    """The small-M forward whose weight waves stage their own X slices (X too large to
    stage for the workgroup): repeated calls are bitwise equal.  A wait that did not cover
    a stage's loads would show as a run-to-run difference."""
    import torch
    M, K, N, r = 16, 8256, 328, 16
    d = synth.case(M, K, N, r, seed=29)
    qw = lib.quantize(gc.dev_weight(d), const_type=const_type)
    X, A, B = _dev(d, r)
    outs = []
    for _ in range(4):
        Y, U = lib.linear_fwd(qw, X, A, B, 16.0)
        outs.append((Y.clone(), U.clone()))
    torch.cuda.synchronize()
    for Y, U in outs[1:]:
        assert torch.equal(Y.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(U.view(torch.int16), outs[0][1].view(torch.int16))


@pytest.mark.parametrize("M", [300, 5])
def test_backward_optional_inputs_and_outputs(lib, M):
    """U_s not passed (the backward recomputes it) and dX not requested (only dA, dB).

    At M > 16 the forward and the backward compute U_s with the same kernel, so the
    recomputed backward is bitwise the saved one; at M <= 16 the forward's U_s comes
    from the weight-stream path (another summation order), so there the results are
    checked against the oracle.  Skipping dX leaves dA and dB bitwise unchanged."""
    import torch
    K, N, r, alpha = 1088, 520, 16, 16.0
    print(f"optional-args case M={M} K={K} N={N} r={r}", flush=True)
    d = synth.case(M, K, N, r, seed=M + 11)
    qw = lib.quantize(gc.dev_weight(d))
    X, A, B = _dev(d, r)
    dYt = gc.dev_bf16(d["dY"])
    _, U = lib.linear_fwd(qw, X, A, B, alpha)
    full = lib.linear_bwd(qw, dYt, X, A, B, alpha, U)
    recomputed = lib.linear_bwd(qw, dYt, X, A, B, alpha)
    dX_none, dA_only, dB_only = lib.linear_bwd(qw, dYt, X, A, B, alpha, U, need_dx=False)
    torch.cuda.synchronize()
    assert dX_none is None
    assert torch.equal(dA_only.view(torch.int16), full[1].view(torch.int16))
    assert torch.equal(dB_only.view(torch.int16), full[2].view(torch.int16))
    if M > 16:
        for a, b in zip(full, recomputed):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    else:
        Wd = _oracle_w(d)
        Xf, Af, Bf, dYf = (gc.f64(d[k]) for k in ("X", "A", "B", "dY"))
        for name, G, R in zip(("dX", "dA", "dB"), recomputed, linear.backward(dYf, Xf, Wd, Af, Bf, alpha, r)):
            _check(name + " (U recomputed)", gc.host_f32_from_bf16(G), R)


def test_workspace_reuse_across_shapes(lib):
    """One zeroed workspace serves small-M forwards (whose workgroups hand U_s to each
    other through counters at the start of the workspace), GEMM forwards and backwards
    in any order: the counters are back at zero after every call and no other call
    writes them, so the small-M results stay bitwise the same and within tolerance."""
    import torch
    K, N, r, alpha = 1024, 520, 16, 16.0
    d = synth.case(300, K, N, r, seed=77)
    qw = lib.quantize(gc.dev_weight(d))
    X, A, B = _dev(d, r)
    X5 = gc.dev_bf16(d["X"][:5])
    dYt = gc.dev_bf16(d["dY"])
    nbytes = max(lib.qlora_workspace_bytes(op, M, K, N, r) for op in (0, 1) for M in (5, 300))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    Wd = _oracle_w(d)
    ref5 = linear.forward(gc.f64(d["X"][:5]), Wd, gc.f64(d["A"]), gc.f64(d["B"]), alpha, r)
    outs = []
    for _ in range(3):
        Y5, _ = lib.linear_fwd(qw, X5, A, B, alpha, ws=ws)
        outs.append(Y5.clone())
        assert int(ws[:lib._lib.QLORA_WORKSPACE_HEADER_BYTES].count_nonzero()) == 0
        Y, U = lib.linear_fwd(qw, X, A, B, alpha, ws=ws)
        lib.linear_bwd(qw, dYt, X, A, B, alpha, U, ws=ws)
        torch.cuda.synchronize()
        assert int(ws[:lib._lib.QLORA_WORKSPACE_HEADER_BYTES].count_nonzero()) == 0
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    _check("Y (M = 5, shared workspace)", gc.host_f32_from_bf16(outs[0]), ref5)


def test_launch_on_a_side_stream(lib):
    """The binding launches on torch's current stream: a forward and backward issued on
    another stream (default priority) give the default stream's results bitwise."""
    import torch
    M, K, N, r = 260, 512, 384, 32
    d = synth.case(M, K, N, r, seed=5)
    qw = lib.quantize(gc.dev_weight(d))
    X, A, B = _dev(d, r)
    dYt = gc.dev_bf16(d["dY"])
    Y0, U0 = lib.linear_fwd(qw, X, A, B, 16.0)
    g0 = lib.linear_bwd(qw, dYt, X, A, B, 16.0, U0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        Y1, U1 = lib.linear_fwd(qw, X, A, B, 16.0)
        g1 = lib.linear_bwd(qw, dYt, X, A, B, 16.0, U1)
    side.synchronize()
    for a, b in zip([Y0, U0, *g0], [Y1, U1, *g1]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("with_B", [False, True])
def test_workload1_full(lib, with_B):
    """1024 -> 1024, M = 64, r = 8, alpha = 16, fp32 weight; B = 0 then B ~ N(0, 0.01^2)."""
    import torch
    wl = synth.WORKLOADS[1]
    d = synth.workload_linear(1, 0)
    if not with_B:
        d["B"] = np.zeros_like(d["B"])
    qw = lib.quantize(gc.dev_weight(d))
    X, A, B = _dev(d, wl.r)
    Y, U = lib.linear_fwd(qw, X, A, B, wl.alpha)
    dX, dA, dB = lib.linear_bwd(qw, gc.dev_bf16(d["dY"]), X, A, B, wl.alpha, U)
    torch.cuda.synchronize()
    Wd = _oracle_w(d)
    Xf, Af, Bf, dYf = (gc.f64(d[k]) for k in ("X", "A", "B", "dY"))
    Yr = linear.forward(Xf, Wd, Af, Bf, wl.alpha, wl.r)
    if not with_B:
        assert np.array_equal(Yr, linear.base_forward(Xf, Wd))
    _check("Y", gc.host_f32_from_bf16(Y), Yr)
    rdX, rdA, rdB = linear.backward(dYf, Xf, Wd, Af, Bf, wl.alpha, wl.r)
    _check("dX", gc.host_f32_from_bf16(dX), rdX)
    _check("dA", gc.host_f32_from_bf16(dA), rdA)
    _check("dB", gc.host_f32_from_bf16(dB), rdB)


def _full_linear(lib, number, i, M=None, bwd=True):
    """One linear of a workload at its full size, every output against the oracle:
    Y and U_s from oracle.linear.forward / lora_down, dX, dA and dB from
    oracle.linear.backward, all on the same seeded inputs (float64)."""
    import torch
    wl = synth.WORKLOADS[number]
    d = synth.workload_linear(number, i, M=M)
    M = d["X"].shape[0]
    K, N = wl.linears[i]
    print(f"workload {number} linear {i}: M={M} K={K} N={N} r={wl.r}", flush=True)
    qw = lib.quantize(gc.dev_weight(d))
    X, A, B = _dev(d, wl.r)
    Y, U = lib.linear_fwd(qw, X, A, B, wl.alpha)
    if bwd:
        dX, dA, dB = lib.linear_bwd(qw, gc.dev_bf16(d["dY"]), X, A, B, wl.alpha, U)
    torch.cuda.synchronize()
    Wd = _oracle_w(d)
    Xf, Af, Bf = (gc.f64(d[k]) for k in ("X", "A", "B"))
    _check("Y", gc.host_f32_from_bf16(Y), linear.forward(Xf, Wd, Af, Bf, wl.alpha, wl.r))
    _check("U", gc.host_f32_from_bf16(U), linear.lora_down(Xf, Af, wl.alpha, wl.r))
    if not bwd:
        return
    rdX, rdA, rdB = linear.backward(gc.f64(d["dY"]), Xf, Wd, Af, Bf, wl.alpha, wl.r)
    _check("dX", gc.host_f32_from_bf16(dX), rdX)
    _check("dA", gc.host_f32_from_bf16(dA), rdA)
    _check("dB", gc.host_f32_from_bf16(dB), rdB)


@pytest.mark.parametrize("i", [0, 1, 2])
def test_workload2_full(lib, i):
    _full_linear(lib, 2, i)


@pytest.mark.parametrize("i", [0, 1])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_workload3_full(lib, i, M):
    import torch
    wl = synth.WORKLOADS[3]
    d = synth.workload_linear(3, i, M=M, parts=("W", "X", "A", "B"))
    K, N = wl.linears[i]
    print(f"workload 3 linear {i}: M={M} K={K} N={N}", flush=True)
    qw = lib.quantize(gc.dev_weight(d))
    X, A, B = _dev(d, wl.r)
    Y, _ = lib.linear_fwd(qw, X, A, B, wl.alpha)
    torch.cuda.synchronize()
    Xf, Af, Bf = (gc.f64(d[k]) for k in ("X", "A", "B"))
    _check("Y", gc.host_f32_from_bf16(Y), linear.forward(Xf, _oracle_w(d), Af, Bf, wl.alpha, wl.r))


@pytest.mark.parametrize("i", [0, 4, 6])
def test_workload4_full(lib, i):
    """LLaMA-65B layer linears at M = 2048, r = 64: q_proj 8192 -> 8192, gate_proj
    8192 -> 22016 and down_proj 22016 -> 8192 (k, v, o share q's shape, up shares gate's)."""
    _full_linear(lib, 4, i)


def test_workload5_forward_sampled_columns(lib):
    """Stress weight 8192 x 22016 (K = 22016 -> N = 8192), M = 512, r = 32: sampled
    output columns against the oracle decode of just those weight rows."""
    import torch
    wl = synth.WORKLOADS[5]
    d = synth.workload_linear(5, 0, parts=("W", "X", "A", "B"))
    qw = lib.quantize(gc.dev_weight(d))
    X, A, B = _dev(d, wl.r)
    Y, _ = lib.linear_fwd(qw, X, A, B, wl.alpha)
    torch.cuda.synchronize()
    rng = np.random.default_rng(55)
    cols = np.sort(rng.choice(8192, 24, replace=False))
    Wrows = gc.oracle_rows(gc.weight_f32(d), cols)
    Xf, Af, Bf = (gc.f64(d[k]) for k in ("X", "A", "B"))
    ref = Xf @ Wrows.T + (wl.alpha / wl.r) * (Xf @ Af.T) @ Bf[cols].T
    _check("Y cols", gc.host_f32_from_bf16(Y)[:, cols], ref)


def test_largest_activation_below_32bit_offsets(lib):
    """X and dX of 131,000 x 16,384 bf16 (4,292,608,000 bytes, just under the 32-bit buffer
    limit of 0xFFFFFFF0) with a 256 x 16,384 weight and r = 16: the last token rows load and
    store at byte offsets near the top of the 32-bit range.  X is drawn on the device from a
    seeded generator and only the sampled rows come back; Y and dX rows against the oracle
    (dA and dB, sums over all 131,000 tokens, are checked at smaller sizes elsewhere)."""
    import torch
    M, K, N, r, alpha = 131000, 16384, 256, 16, 16.0
    assert M * K * 2 <= 0xFFFFFFF0 < (M + 100) * K * 2  # within 100 rows of the limit
    print(f"largest activation: M={M} K={K} N={N} r={r} ({M * K * 2} bytes)", flush=True)
    d = synth.case(1, K, N, r, seed=4242, parts=("W", "X", "A", "B"))
    qw = lib.quantize(gc.dev_weight(d))
    A, B = gc.dev_bf16(d["A"]), gc.dev_bf16(d["B"])
    g = torch.Generator(device="cuda").manual_seed(4242)
    X = torch.randn(M, K, device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
    dY = torch.randn(M, N, device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
    Y, U = lib.linear_fwd(qw, X, A, B, alpha)
    dX, _, _ = lib.linear_bwd(qw, dY, X, A, B, alpha, U)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 255, 256, 65535, 65536, M - 257, M - 256, M - 33, M - 2, M - 1], device="cuda")
    Xs, dYs = gc.host_f32_from_bf16(X[rows]), gc.host_f32_from_bf16(dY[rows])
    Ys, dXs = gc.host_f32_from_bf16(Y[rows]), gc.host_f32_from_bf16(dX[rows])
    del X, dX, Y, U, dY
    torch.cuda.empty_cache()
    Wd = _oracle_w(d)
    Af, Bf = gc.f64(d["A"]), gc.f64(d["B"])
    _check("Y rows", Ys, linear.forward(Xs, Wd, Af, Bf, alpha, r))
    rdX, _, _ = linear.backward(dYs, Xs, Wd, Af, Bf, alpha, r)
    _check("dX rows", dXs, rdX)


def test_largest_weight_below_32bit_offsets(lib):
    """A 262,143 x 32,768 weight (8.59 G weights; 4,294,950,912 bytes of codes, one row under the
    32-bit buffer limit), drawn on the device from a seeded generator and quantized there.
    Each row is exactly two DQ groups, so the oracle quantizes a sampled row on its own: codes,
    constants and the decoded row bit-exact, and the M = 1 GEMV and an M = 32 GEMM forward on
    those output rows against the oracle."""
    import torch
    N, K = 262143, 32768
    assert N * K // 2 <= 0xFFFFFFF0 < (N + 1) * K // 2 and K % 16384 == 0
    print(f"largest weight: N={N} K={K} ({N * K // 2} bytes of codes)", flush=True)
    g = torch.Generator(device="cuda").manual_seed(777)
    W = (torch.randn(N, K, device="cuda", generator=g, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    rows = torch.tensor([0, 1, 4095, N // 2, N - 65, N - 2, N - 1], device="cuda")
    Wrows = gc.host_f32_from_bf16(W[rows]).astype(np.float32)
    qw = lib.quantize(W)
    del W
    torch.cuda.empty_cache()
    X1 = torch.randn(1, K, device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
    X32 = torch.randn(32, K, device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
    Y1, _ = lib.linear_fwd(qw, X1)
    Y32, _ = lib.linear_fwd(qw, X32)
    torch.cuda.synchronize()
    rl = rows.tolist()
    codes = qw.codes.view(N, K // 2)[rows].cpu().numpy()
    c8 = qw.absmax_q.view(N, K // 64)[rows].cpu().numpy()
    s = qw.dq_scale.view(N, 2)[rows].cpu().numpy()
    o = qw.dq_offset.view(N, 2)[rows].cpu().numpy()
    X1f, X32f = gc.host_f32_from_bf16(X1), gc.host_f32_from_bf16(X32)
    Y1r, Y32r = gc.host_f32_from_bf16(Y1)[:, rl], gc.host_f32_from_bf16(Y32)[:, rl]
    del qw, Y1, Y32
    torch.cuda.empty_cache()
    Wd = np.empty((len(rl), K), np.float64)
    for i in range(len(rl)):
        ref = nf4.quantize_nf4(Wrows[i:i + 1])
        assert np.array_equal(codes[i], ref["codes"].reshape(-1))
        assert np.array_equal(c8[i].view(np.uint8), ref["absmax_q"].view(np.uint8))
        assert np.array_equal(s[i].view(np.uint32), ref["dq_scale"].view(np.uint32))
        assert np.array_equal(o[i].view(np.uint32), ref["dq_offset"].view(np.uint32))
        Wd[i] = nf4.dequantize_bf16(ref).reshape(-1)
    _check("Y (M = 1) sampled rows", Y1r, X1f @ Wd.T)
    _check("Y (M = 32) sampled rows", Y32r, X32f @ Wd.T)
