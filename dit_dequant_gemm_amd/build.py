"""Build libddg.so (HIP, gfx950) in-tree with hipcc.

    python -m dit_dequant_gemm_amd.build          # compile + link
    python -m dit_dequant_gemm_amd.build --asm    # also keep gfx950 assembly

Objects go to ``_build/`` at the repository root; the library to
``dit_dequant_gemm_amd/libddg.so``.  Every call rebuilds everything.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libddg.so")
ARCH = "gfx950"
BITS = (3, 4, 5, 6, 7)

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    # IEEE float32 for the bit-exact quantizer: correctly rounded division,
    # subnormals kept, no contraction into fused multiply-adds.
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=off",
    # no packed-FP32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _units():
    units = [(os.path.join(CSRC, "inst_bits.hip"), f"inst_b{b}", [f"-DDDG_BITS={b}"]) for b in BITS]
    units.append((os.path.join(CSRC, "lowrank.hip"), "lowrank", []))
    units.append((os.path.join(CSRC, "grouped.hip"), "grouped", []))
    units.append((os.path.join(CSRC, "pd.hip"), "pd", []))
    units.append((os.path.join(CSRC, "rotate.hip"), "rotate", []))
    units.append((os.path.join(CSRC, "w4a8.hip"), "w4a8", []))
    units.append((os.path.join(CSRC, "api.hip"), "api", []))
    return units


def _compile(unit, asm: bool):
    src, name, defs = unit
    udir = os.path.join(BUILD, name)          # one folder per unit: temps do not collide
    os.makedirs(udir, exist_ok=True)
    obj = os.path.join(udir, name + ".o")
    cmd = [HIPCC, *COMMON, *defs, "-c", src, "-o", obj]
    if asm:
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=udir)
    if r.returncode != 0 and asm:
        # keeping intermediates can trip the compiler on some template
        # instantiations; the object itself builds without them
        r = subprocess.run(cmd[:-1], capture_output=True, text=True, cwd=udir)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(asm: bool = False, jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every HIP unit for gfx950 and link libddg.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda u: _compile(u, asm), _units()))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true", help="keep the gfx950 assembly in _build/")
    ap.add_argument("-j", type=int, default=None)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(asm=a.asm, jobs=a.j, verbose=a.v))
