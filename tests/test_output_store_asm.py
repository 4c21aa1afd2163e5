"""The output stores that write through the L2, read from the gfx950
assembly of the 4-bit product kernels (CPU only).

The large-M epilogues store Y with global_store_dwordx4 ... sc1, written in
assembly because the global-store builtins take no cache-policy operand.  A
vector ALU instruction that overwrites the data registers of a store of more
than 8 bytes right after it needs a wait state the compiler cannot insert for
an instruction it did not generate, so each such store carries its own
s_nop.  This checks that every write-through store in the kernels is followed
at once by an s_nop, and that the kernels that should use it (256 x 256 and
256 x 192 tiles, stream-K) do.
"""
import os
import re
import shutil
import subprocess

import pytest

from dit_dequant_gemm_amd import build as B

STORE = re.compile(r"^\s*global_store_dwordx4\s+v\[\d+:\d+\],\s*v\[\d+:\d+\],\s*off\s+sc1\s*$")
NOP = re.compile(r"^\s*s_nop\s+(\d+)\s*$")


def _kernels(text):
    for m in re.finditer(r"^(_Z\S+):\s*;.*?$(.*?)s_endpgm", text, re.S | re.M):
        yield m.group(1), m.group(2).split("\n")


def test_write_through_stores_carry_their_wait_state(tmp_path):
    if not (shutil.which(B.HIPCC) or os.path.exists(B.HIPCC)):
        pytest.skip("hipcc not found")
    out = str(tmp_path / "inst_b4.s")
    cmd = [B.HIPCC, *B.COMMON, "-DDDG_BITS=4", "--cuda-device-only", "-S",
           os.path.join(B.CSRC, "inst_bits.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=str(tmp_path))
    assert r.returncode == 0, r.stderr[-2000:]
    users = {}
    for name, lines in _kernels(open(out).read()):
        code = [l for l in lines if l.strip() and not l.strip().startswith(";")]
        n = 0
        for i, line in enumerate(code):
            if STORE.match(line):
                n += 1
                nxt = NOP.match(code[i + 1]) if i + 1 < len(code) else None
                # s_nop N waits N + 1 states; one is enough
                assert nxt is not None, (name, line, code[i + 1] if i + 1 < len(code) else None)
        users[name] = n
    for kernel in ("gemm_large_kernel", "gemm_n192_kernel", "gemm_streamk_kernel"):
        assert any(kernel in k and v > 0 for k, v in users.items()), (kernel, users)
