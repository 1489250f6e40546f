"""The fused GEMMs' LDS pipelines wait at each barrier with a fixed count of memory loads
left in flight (`s_waitcnt vmcnt(N)`).  That count is only right if exactly the loads it
assumes were issued after the activation / dY tile that the barrier publishes, in the
order the source issues them; a load the compiler moves or deletes makes the wait too
weak and lets a wave read a tile before it has landed (a run-to-run race).

This test compiles gemm.hip for gfx950 with the library's flags and reads the assembly
of every instantiation.  The kernels keep every value in registers (no scratch spills,
which would cost them about half their speed), and: at each barrier of the forward kernel, the loads left in flight
must all have been issued after the direct-to-LDS loads of the tile read right after it;
at each barrier of the pipelined dX kernel, every direct-to-LDS (dY) load issued before
the barrier must be retired.  No GPU needed (hipcc cross-compiles)."""

import os
import re
import shutil
import subprocess

import pytest

from bit_quantized_lora_nf4_amd import build as libbuild

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "gemm.s"
    flags = [f for f in libbuild.FLAGS if f not in ("-fPIC",)]
    cmd = [HIPCC] + flags + ["--cuda-device-only", "-S", os.path.join(libbuild.CSRC, "gemm.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def _events(asm, kernel):
    m = re.search(r"^" + re.escape(kernel) + r":.*?s_endpgm", asm, re.S | re.M)
    assert m, kernel
    ev = []
    for line in m.group(0).splitlines():
        line = line.strip()
        if line.startswith("buffer_load"):
            ev.append(("D" if line.endswith(" lds") else "R", 0))
        w = re.match(r"s_waitcnt vmcnt\((\d+)\)", line)
        if w:
            ev.append(("W", int(w.group(1))))
        if line.startswith("s_barrier"):
            ev.append(("B", 0))
    return ev


def _barrier_waits(ev):
    """(index, N) of every vmcnt wait directly followed by a barrier."""
    return [(i, e[1]) for i, e in enumerate(ev) if e[0] == "W" and i + 1 < len(ev) and ev[i + 1][0] == "B"]


FWD = "_ZN5qlora12_GLOBAL__N_115gemm_fwd_kernelILi{}EEEvNS0_10GemmParamsE"
DX = "_ZN5qlora12_GLOBAL__N_119gemm_dx_pipe_kernelILi{}EEEvNS0_10GemmParamsE"


@pytest.mark.parametrize("ct", [0, 1, 2])
def test_forward_barrier_waits(gemm_asm, ct):
    ev = _events(gemm_asm, FWD.format(ct))
    waits = _barrier_waits(ev)
    assert len(waits) >= 4
    checked = 0
    for i, n in waits:
        j = i - 1
        while j >= 0 and ev[j][0] != "B":
            j -= 1
        if j < 0 or (j >= 1 and ev[j - 1] == ("W", 0)):
            continue  # the prologue barrier: everything before it was retired
        # the half-tile DMA issued right after the previous barrier must be retired here:
        # the wait may leave in flight only loads issued after it
        k, seen = j + 1, 0
        while k < i and seen < 4:
            seen += ev[k][0] in ("D", "R")
            k += 1
        after = sum(1 for x in ev[k:i] if x[0] in ("D", "R"))
        assert n <= after, f"barrier wait vmcnt({n}) leaves {n - after} loads of the published tile in flight"
        checked += 1
    assert checked >= 3


@pytest.mark.parametrize("ct", [0, 1, 2])
def test_dx_barrier_waits(gemm_asm, ct):
    ev = _events(gemm_asm, DX.format(ct))
    waits = _barrier_waits(ev)
    assert len(waits) >= 4
    for i, n in waits:
        j = i - 1
        while j >= 0 and ev[j][0] != "D":
            j -= 1
        if j < 0:
            continue
        after = sum(1 for x in ev[j + 1:i] if x[0] == "R")
        assert n <= after, f"barrier wait vmcnt({n}) with only {after} register loads after the last dY load"


def test_no_register_spills(gemm_asm):
    """Every fused-GEMM instantiation fits the register file: its private segment stays at
    the few bytes the kernel ABI reserves (a spill adds hundreds)."""
    sizes = dict(re.findall(r"\.name:\s+(\S*gemm_\S*kernel\S*)\s.*?\.private_segment_fixed_size:\s+(\d+)",
                            gemm_asm, re.S))
    assert len(sizes) >= 9, sizes
    for name, size in sizes.items():
        assert int(size) <= 16, f"{name}: {size} bytes of scratch"
