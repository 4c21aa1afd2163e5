"""The X hand-over of the small-M product kernels, read from their gfx950
assembly (CPU only).

Each wave loads its share of a step's X slice into registers, writes it to an
LDS slot, and one LDS barrier hands the slot to the other column waves.  The
waits in front of the LDS writes are the compiler's own (register
dependences), so no wait depends on the order the loads were issued in.  This
checks, in every instantiation of gemm_small_kernel and in the grouped
small-M kernel, that no X slice goes to LDS by DMA (buffer_load ... lds: its
completion would need a counted vmcnt wait) and that every barrier is preceded
by a wait for the wave's LDS writes (lgkmcnt(0)) since the previous one.
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
GROUPED_SMALL = re.compile(r"^(_ZN3ddg25gemm_grouped_small_kernelILi(\d)EEEvNS_9GroupArgsE):", re.M)


def _compile(tmp, src, defs, name):
    out = os.path.join(tmp, name)
    cmd = [B.HIPCC, *B.COMMON, *defs, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not (shutil.which(B.HIPCC) or os.path.exists(B.HIPCC)):
        pytest.skip("hipcc not found")
    tmp = str(tmp_path_factory.mktemp("asm"))
    jobs = [("inst_bits.hip", [f"-DDDG_BITS={b}"], f"b{b}.s") for b in BITS]
    jobs.append(("grouped.hip", [], "grouped.s"))
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        texts = list(ex.map(lambda j: _compile(tmp, *j), jobs))
    return texts


def _check_body(body, where):
    assert " lds" not in "\n".join(l for l in body.split("\n") if l.strip().startswith("buffer_load")), \
        f"{where}: an X slice goes to LDS by DMA"
    barriers = 0
    lgkm_done = False
    for line in body.split("\n"):
        line = line.strip()
        if line.startswith("s_waitcnt") and "lgkmcnt(0)" in line:
            lgkm_done = True
        elif line.startswith("ds_write") or line.startswith("ds_store"):
            lgkm_done = False
        elif line.startswith("s_barrier"):
            barriers += 1
            assert lgkm_done, f"{where}: barrier {barriers} without a wait for the LDS writes before it"
    assert barriers > 0, f"{where}: no barrier found"


def test_small_kernels_hand_over_x_through_lds_writes(asm):
    seen = 0
    for text in asm[:-1]:
        for m in KERNEL.finditer(text):
            b, rb, nc, nk = (int(g) for g in m.groups()[1:])
            body = text[m.end(): text.index("s_endpgm", m.end())]
            _check_body(body, f"gemm_small_kernel B={b} RB={rb} NC={nc} NK={nk}")
            seen += 1
    assert seen >= len(BITS) * 9


@pytest.mark.parametrize("rb", (2, 4))
def test_grouped_small_kernel_hands_over_x_through_lds_writes(asm, rb):
    text = asm[-1]
    ms = [m for m in GROUPED_SMALL.finditer(text) if int(m.group(2)) == rb]
    assert ms, f"no gemm_grouped_small_kernel<{rb}> found"
    body = text[ms[0].end(): text.index("s_endpgm", ms[0].end())]
    _check_body(body, f"gemm_grouped_small_kernel<{rb}>")
