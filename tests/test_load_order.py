"""Load order of the small-M product kernel (gemm_small_kernel), read from its
gfx950 assembly.

The kernel hands the X slice of each step from the waves that DMA it to the
other column waves with a counted wait (``s_waitcnt vmcnt(n)``) and a bare
barrier.  The count is right only if the compiled code issues, per step, the
slice's DMAs first and then the weight loads, with no load dropped or moved
between steps, and if the steps past the end of a K range issue nothing.  A
wrong order does not fail a parity test reliably (the stale read is a race),
so the order is checked here in the compiled code of every instantiation:

* the prologue is D groups (DMAs, then weight loads);
* every barrier-to-barrier segment of the loop is one such group or nothing;
* every wait in front of a barrier leaves a count that the step schedule
  allows: D - 1 groups plus one step's weight loads in the main loop, fewer in
  the tail, 0 after the loop.

The ring depth, DMA and load counts per step follow the kernel's own rules:
S = 3 slots with a two-way K split, else 2 (fewer if LDS is short), D = S - 1
steps in flight, 1 KB DMAs per 16*RB x 128 bf16 slice shared among the NC
column waves, and two (3, 4 bits) or three (5..7 bits) loads per step for a
lane's packed chunk and its scale.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from dit_dequant_gemm_amd import build as B

BITS = (3, 4, 5, 6, 7)
KERNEL = re.compile(r"^(_ZN3ddg17gemm_small_kernelILi(\d)ELi(\d)ELi(\d)ELi(\d+)EEEvNS_8GemmArgsE):", re.M)
WAIT = re.compile(r"s_waitcnt\s+(.*)$")


def _schedule(bits, rb, nc, nk):
    xslot = rb * 16 * 256
    red = (nk - 1 if nk > 1 else 1) * nc * rb * 64 * 16
    s_fit = (160 * 1024 - red) // (nk * xslot)
    s = min(3 if nk <= 2 else 2, s_fit)
    d = s - 1
    nd = xslot // 1024 // nc
    nwl = 2 if bits in (3, 4) else 3
    return d, nd, nwl


def _vmcnt(wait_args):
    m = re.search(r"vmcnt\((\d+)\)", wait_args)
    return int(m.group(1)) if m else None


def _events(body):
    """Buffer loads ('X' = DMA to LDS, 'W' = to registers), barriers ('|', with
    the vmcnt of the last wait in front of it).  A barrier with no vmcnt wait
    and no load since the previous barrier is not listed: the compiler drops a
    wait that an earlier, stricter one already covers."""
    ev, waits, last_vm, loaded = [], [], None, False
    for line in body.split("\n"):
        line = line.strip()
        if line.startswith("buffer_load"):
            ev.append("X" if line.endswith(" lds") or " lds " in line else "W")
            last_vm, loaded = None, True
        elif line.startswith("s_waitcnt"):
            v = _vmcnt(WAIT.match(line).group(1))
            if v is not None:
                last_vm = v if last_vm is None else min(last_vm, v)
        elif line.startswith("s_barrier"):
            ev.append("|")
            if last_vm is not None or loaded:
                waits.append(last_vm)
            last_vm, loaded = None, False
    return "".join(ev), waits


def _asm(tmp, bits):
    out = os.path.join(tmp, f"b{bits}.s")
    cmd = [B.HIPCC, *B.COMMON, f"-DDDG_BITS={bits}", "--cuda-device-only", "-S",
           os.path.join(B.CSRC, "inst_bits.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def asm_by_bits(tmp_path_factory):
    if not (shutil.which(B.HIPCC) or os.path.exists(B.HIPCC)):
        pytest.skip("hipcc not found")
    tmp = str(tmp_path_factory.mktemp("asm"))
    with cf.ThreadPoolExecutor(max_workers=len(BITS)) as ex:
        texts = list(ex.map(lambda b: _asm(tmp, b), BITS))
    return dict(zip(BITS, texts))


@pytest.mark.parametrize("bits", BITS)
def test_small_kernel_load_order(asm_by_bits, bits):
    text = asm_by_bits[bits]
    kernels = list(KERNEL.finditer(text))
    assert kernels, "no gemm_small_kernel instantiation found"
    for m in kernels:
        b, rb, nc, nk = (int(g) for g in m.groups()[1:])
        assert b == bits
        d, nd, nwl = _schedule(b, rb, nc, nk)
        group = "X" * nd + "W" * nwl
        body = text[m.end(): text.index("s_endpgm", m.end())]
        ev, waits = _events(body)
        segs = ev.split("|")
        where = f"B={b} RB={rb} NC={nc} NK={nk}"
        assert segs[0] == group * d, f"{where}: prologue {segs[0]!r}, want {group * d!r}"
        for seg in segs[1:]:
            assert seg in ("", group), f"{where}: loop segment {seg!r}"
        allowed = {nwl + u * (nd + nwl) for u in range(d)} | {0}
        for w in waits:
            assert w in allowed, f"{where}: barrier after vmcnt({w}), allowed {sorted(allowed)}"
        # the steady-state count appears (main loop) unless the ring is one step deep
        assert nwl + (d - 1) * (nd + nwl) in waits, f"{where}: no steady-state wait"


GROUPED_SMALL = re.compile(r"^(_ZN3ddg25gemm_grouped_small_kernelILi(\d)EEEvNS_9GroupArgsE):", re.M)


@pytest.fixture(scope="module")
def grouped_asm(tmp_path_factory):
    if not (shutil.which(B.HIPCC) or os.path.exists(B.HIPCC)):
        pytest.skip("hipcc not found")
    tmp = str(tmp_path_factory.mktemp("asm_grouped"))
    out = os.path.join(tmp, "grouped.s")
    cmd = [B.HIPCC, *B.COMMON, "--cuda-device-only", "-S", os.path.join(B.CSRC, "grouped.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.mark.parametrize("rb", (2, 4))
def test_grouped_small_kernel_load_order(grouped_asm, rb):
    """The grouped kernel inlines the same body once per bit width, one after
    the other: every barrier-to-barrier segment is a prologue (D groups), one
    group or nothing, for a width of two (3, 4 bits) or three (5..7 bits)
    weight loads, and every wait is one the schedule allows."""
    text = grouped_asm
    ms = [m for m in GROUPED_SMALL.finditer(text) if int(m.group(2)) == rb]
    assert ms, f"no gemm_grouped_small_kernel<{rb}> found"
    m = ms[0]
    body = text[m.end(): text.index("s_endpgm", m.end())]
    ev, waits = _events(body)
    segs = ev.split("|")
    allowed_segs, allowed_waits = {""}, {0}
    for bits in (3, 5):
        d, nd, nwl = _schedule(bits, rb, 2, 2)
        group = "X" * nd + "W" * nwl
        allowed_segs |= {group, group * d}
        allowed_waits |= {nwl + u * (nd + nwl) for u in range(d)}
    for sg in segs:
        assert sg in allowed_segs, f"RB={rb}: segment {sg!r}"
    for w in waits:
        assert w in allowed_waits, f"RB={rb}: barrier after vmcnt({w}), allowed {sorted(allowed_waits)}"
