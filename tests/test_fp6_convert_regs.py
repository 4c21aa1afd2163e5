"""Register assignment of the packed FP6 conversions, read from the gfx950
assembly of w4a8.hip (CPU only).

v_cvt_scalef32_2xpk16_{fp6,bf6}_f32 turns two 16-float sources into six
result dwords and writes early result dwords before it has read all of its
first source.  Given a result range inside a source that ends at the
instruction, code 8 of each 32-value unit came out wrong.  Both quantizers
(FP6 activations, FP6 weights) keep the sources live past the result; this
checks that no such instruction's result registers overlap either source.
"""
import os
import re
import shutil
import subprocess

import pytest

from dit_dequant_gemm_amd import build as B

CVT = re.compile(r"v_cvt_scalef32_2xpk16_(?:fp6|bf6)_f32\s+v\[(\d+):(\d+)\],\s*v\[(\d+):(\d+)\],\s*v\[(\d+):(\d+)\]")


def test_fp6_conversions_do_not_overwrite_their_sources(tmp_path):
    if not (shutil.which(B.HIPCC) or os.path.exists(B.HIPCC)):
        pytest.skip("hipcc not found")
    out = str(tmp_path / "w4a8.s")
    cmd = [B.HIPCC, *B.COMMON, "--cuda-device-only", "-S", os.path.join(B.CSRC, "w4a8.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=str(tmp_path))
    assert r.returncode == 0, r.stderr[-2000:]
    text = open(out).read()
    found = CVT.findall(text)
    # two quantizers x two formats, the weight quantizer also x dtype x pow2
    assert len(found) >= 12, len(found)
    for d0, d1, a0, a1, b0, b1 in found:
        dst = set(range(int(d0), int(d1) + 1))
        assert int(d1) - int(d0) == 5 and int(a1) - int(a0) == 15 and int(b1) - int(b0) == 15
        assert not dst & set(range(int(a0), int(a1) + 1)), (d0, d1, a0, a1)
        assert not dst & set(range(int(b0), int(b1) + 1)), (d0, d1, b0, b1)
