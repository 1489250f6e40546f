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
the barrier must be retired.  The skinny adapter kernels of lora.hip are checked the same
way over their control-flow graph (see the section at the end).  No GPU needed (hipcc
cross-compiles)."""

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


def _all_retired(ev, j):
    """Whether no load is in flight at event j: a vmcnt(0) wait follows the last load before it."""
    k = j - 1
    while k >= 0 and ev[k] != ("W", 0):
        if ev[k][0] in ("D", "R"):
            return False
        k -= 1
    return k >= 0


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
        if j < 0 or _all_retired(ev, j):
            continue  # a prologue barrier: everything issued before it was retired
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


# ---- the skinny adapter kernels (lora.hip) --------------------------------------------
# Each of their staging loops issues the loads of NB - 1 steps before the loop, then one
# step's loads per iteration, and waits at the top of the iteration with vmcnt(N).  Step i
# has landed at that wait iff N <= P - L, where P is the number of direct-to-LDS loads the
# prologue issued and L the number issued per iteration (every load of the prologue and
# the loop body belongs to one step, in issue order).  Any other vector memory operation
# inside the loop would shift the count, so there must be none.

@pytest.fixture(scope="module")
def lora_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "lora.s"
    flags = [f for f in libbuild.FLAGS if f not in ("-fPIC",)]
    cmd = [HIPCC] + flags + ["--cuda-device-only", "-S", os.path.join(libbuild.CSRC, "lora.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


_VMEM = re.compile(r"(buffer|global|flat|scratch)_(load|store|atomic)")
_BR = re.compile(r"s_(c?)branch\S*\s+(\.LBB\S+)")


def _cfg(body):
    """Basic blocks of one function in text order: dicts with the label, its loop-header
    comment, the instructions and the successor block indices."""
    blocks, cur = [], {"label": None, "note": "", "lines": []}
    for raw in body.splitlines()[1:]:
        ln = raw.strip()
        m = re.match(r"(\.LBB\S+):\s*(;.*)?$", ln)
        if m:
            blocks.append(cur)
            cur = {"label": m.group(1), "note": m.group(2) or "", "lines": []}
            continue
        if not ln or ln.startswith((";", ".")):
            continue
        cur["lines"].append(ln)
        if _BR.match(ln) or ln.startswith("s_endpgm"):
            blocks.append(cur)  # a branch ends the block; what follows is a block of its own
            note = cur["note"]
            if cur["label"] and "Loop Header" in note:
                note = f"; in Loop: Header={cur['label'][2:]} Depth=1"
            cur = {"label": None, "note": note, "lines": []}
    blocks.append(cur)
    blocks = [b for b in blocks if b["label"] or b["lines"]]
    index = {b["label"]: i for i, b in enumerate(blocks) if b["label"]}
    for i, b in enumerate(blocks):
        last = b["lines"][-1] if b["lines"] else ""
        m = _BR.match(last)
        succ = []
        if m:
            succ.append(index[m.group(2)])
        if not last.startswith("s_endpgm") and not (m and not m.group(1)) and i + 1 < len(blocks):
            succ.append(i + 1)
        b["succ"] = succ
    return blocks


def _dma(lines):
    return sum(1 for ln in lines if _VMEM.match(ln) and ln.endswith(" lds"))


def _staging_loops(body):
    """(P, L, waits, other) for every innermost loop that waits before a barrier: P the set
    of direct-to-LDS load counts on the paths from the entry to the loop, L the set of
    counts per iteration, waits the vmcnt values before its barriers, other any other
    vector memory operation inside it."""
    blocks = _cfg(body)
    out = []
    for h, hb in enumerate(blocks):
        m = re.match(r"; =>This Inner Loop Header: Depth=1", hb["note"])
        if not m:
            continue
        hid = hb["label"][2:]  # ".LBBx_y" -> "BBx_y"
        members = {i for i, b in enumerate(blocks) if i == h or f"Header={hid} " in b["note"] + " "}
        loop_lines = [ln for i in sorted(members) for ln in blocks[i]["lines"]]
        waits = [int(re.match(r"s_waitcnt vmcnt\((\d+)\)", loop_lines[k]).group(1))
                 for k in range(len(loop_lines) - 1)
                 if re.match(r"s_waitcnt vmcnt\(\d+\)", loop_lines[k]) and loop_lines[k + 1].startswith("s_barrier")]
        if not waits:
            continue
        other = [ln for ln in loop_lines if _VMEM.match(ln) and not ln.endswith(" lds")]
        # loads per iteration: every path from the header back to it
        iters, stack, seen = set(), [(h, 0)], set()
        while stack:
            i, n = stack.pop()
            if (i, n) in seen or n > 4096:
                continue
            seen.add((i, n))
            n += _dma(blocks[i]["lines"])
            for j in blocks[i]["succ"]:
                if j == h:
                    iters.add(n)
                elif j in members:
                    stack.append((j, n))
        # loads on the paths from the entry to the header (earlier loops are walked once,
        # along their exits; a full wait resets the count)
        pro, stack, seen = set(), [(0, 0)], set()
        while stack:
            i, n = stack.pop()
            if (i, n) in seen:
                continue
            seen.add((i, n))
            for ln in blocks[i]["lines"]:
                if ln.startswith("s_waitcnt vmcnt(0)"):
                    n = 0
                n += _VMEM.match(ln) is not None and ln.endswith(" lds")
            for j in blocks[i]["succ"]:
                if j == h:
                    pro.add(n)
                elif j not in members and j > i or (j not in members and j < i and len(seen) < 4096):
                    stack.append((j, n))
        out.append((pro, iters, waits, other))
    return out


def test_lora_staging_waits(lora_asm):
    kernels = re.findall(r"^(_Z\S*(?:lora_down_partial|reduce_m_partial|down_reduce_partial)\S*):", lora_asm, re.M)
    assert len(kernels) >= 24, len(kernels)
    checked = 0
    for name in kernels:
        # the whole function: blocks may follow its first s_endpgm
        body = re.search(r"^" + re.escape(name) + r":.*?^\.Lfunc_end", lora_asm, re.S | re.M).group(0)
        loops = _staging_loops(body)
        assert loops, f"{name}: no staging loop found"
        for P, L, waits, other in loops:
            assert not other, f"{name}: other vector memory operations inside the staging loop: {other[:3]}"
            assert len(L) == 1 and min(L) > 0, (name, L)
            assert P, (name, "the loop is not reached")
            L = min(L)
            for n in waits:
                assert n <= min(P) - L, (f"{name}: vmcnt({n}) at the loop's barrier, but only {min(P) - L} loads "
                                         f"follow a step's on some path ({sorted(P)} before the loop, {L} per step)")
            checked += 1
    assert checked >= 24


def test_lora_no_register_spills(lora_asm):
    sizes = dict(re.findall(r"\.name:\s+(\S*kernel\S*)\s.*?\.private_segment_fixed_size:\s+(\d+)", lora_asm, re.S))
    assert len(sizes) >= 20, sizes
    for name, size in sizes.items():
        assert int(size) <= 16, f"{name}: {size} bytes of scratch"


# The small-M forward's per-wave X stages: each weight wave loads a step's X slice straight
# into one of its two LDS stages (two LDS objects) and reads it back as MFMA fragments two
# ring slots later; the waits before those reads are the compiler's.  In the main loop
# (two steps per iteration, each issuing the same loads), the wait ahead of each step's
# first LDS read must leave in flight at most the other step's loads, so that the step's
# own direct-to-LDS loads have landed.

@pytest.fixture(scope="module")
def gemv_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "gemv.s"
    flags = [f for f in libbuild.FLAGS if f not in ("-fPIC",)]
    cmd = [HIPCC] + flags + ["--cuda-device-only", "-S", os.path.join(libbuild.CSRC, "gemv.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def test_gemv_x_stage_waits(gemv_asm):
    # gemv_kernel<CT, XLDS = false, MULTI, DIRECT, XDMA = true>
    kernels = re.findall(r"^(_Z\S*gemv_kernelILi\dELb0ELb\dELb\dELb1E\S*):", gemv_asm, re.M)
    assert len(kernels) == 12, kernels
    for name in kernels:
        body = re.search(r"^" + re.escape(name) + r":.*?^\.Lfunc_end", gemv_asm, re.S | re.M).group(0)
        lines = [l.strip() for l in body.splitlines()]
        labels = {m.group(1): i for i, l in enumerate(lines) if (m := re.match(r"^(\.LBB\S+):", l))}
        loops = [(labels[m.group(2)], i) for i, l in enumerate(lines)
                 if (m := _BR.search(l)) and m.group(2) in labels and labels[m.group(2)] < i]
        a, b = max(loops, key=lambda x: x[1] - x[0])  # the main loop: the longest back edge
        loop = lines[a:b + 1]
        dma = sum(1 for l in loop if l.startswith("buffer_load") and l.endswith(" lds"))
        vmem = sum(1 for l in loop if _VMEM.match(l))
        assert dma == 16 and vmem % 2 == 0, (name, dma, vmem)
        per_step = vmem // 2
        # the last vmcnt wait before each run of LDS reads that follows vector memory issue
        waits, last, seen_vmem = [], None, True
        for l in loop:
            w = re.match(r"s_waitcnt vmcnt\((\d+)\)", l)
            if w:
                last = int(w.group(1))
            elif _VMEM.match(l):
                seen_vmem, last = True, None
            elif l.startswith("ds_read") and seen_vmem:
                waits.append(last)
                seen_vmem = False
        assert len(waits) == 2, (name, waits)
        for n in waits:
            assert n is not None and n <= per_step, \
                f"{name}: LDS reads of a stage after vmcnt({n}), but a step issues {per_step} loads"
