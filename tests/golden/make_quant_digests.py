"""Write tests/golden/quant_digests.json: SHA-256 digests of the oracle's
packed bytes and scale bits for every weight of workloads 3 and 5 at every
width the workload names, in chunks of 1024 weight rows.

It calls only the oracle (oracle/) and the seeded input generators
(dit_dequant_gemm_amd/synth.py); the GPU parity test hashes the library's
record of the same inputs the same way and compares.

    python tests/golden/make_quant_digests.py          # about a minute
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from dit_dequant_gemm_amd import synth  # noqa: E402

CHUNK_ROWS = 1024
OUT = os.path.join(HERE, "quant_digests.json")


def digests(packed_rows, scale_rows):
    """Per chunk of CHUNK_ROWS rows: sha256 of the packed bytes and of the
    little-endian float32 bit patterns of the scales."""
    p, s = [], []
    for r0 in range(0, packed_rows.shape[0], CHUNK_ROWS):
        p.append(hashlib.sha256(np.ascontiguousarray(packed_rows[r0:r0 + CHUNK_ROWS]).tobytes()).hexdigest())
        s.append(hashlib.sha256(np.ascontiguousarray(
            scale_rows[r0:r0 + CHUNK_ROWS], dtype="<f4").view("<u4").tobytes()).hexdigest())
    return p, s


def tensors():
    """(key, weight, widths) of every tensor covered."""
    for which in ("up", "down"):
        c = synth.config3(which, m=1)
        yield f"workload3/{which}", c["w"], c["bits_sweep"]
    for name in ("qkv", "o", "up", "down"):
        yield f"workload5/{name}", synth.config5_weights(name), synth.C5_BIT_CHOICES


def main():
    out = {"chunk_rows": CHUNK_ROWS,
           "about": "oracle quantize_pack of the seeded workload weights; sha256 per 1024-row chunk "
                    "of the packed bytes and of the float32 scale bits",
           "tensors": {}}
    for key, w, widths in tensors():
        n, k = w.shape
        for bits in widths:
            packed, scales, _ = O.quantize_pack(w, bits)
            p, s = digests(packed.reshape(n, k * bits // 8), np.asarray(scales).reshape(n, k // 128))
            out["tensors"][f"{key}/{bits}"] = {"rows": n, "cols": k, "bits": bits, "packed": p, "scales": s}
            print(key, bits, len(p), "chunks", flush=True)
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
