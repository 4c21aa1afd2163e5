"""Bit-exactness of the whole packed record (every row) on the workloads
whose tensors the other parity tests sample: workloads 3 and 5 at every
width against digests the oracle wrote (tests/golden/make_quant_digests.py),
and workload 4's residual against the oracle run here.  A mismatch names the
first 1024-row chunk that differs."""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
from dit_dequant_gemm_amd import synth
from parity_util import dev_bf16, dev_f32, f32_bits, host

DIGESTS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant_digests.json")


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _load():
    with open(DIGESTS) as f:
        return json.load(f)


def _weights(key):
    wl, name = key.split("/")
    if wl == "workload3":
        return synth.config3(name, m=1)["w"]
    return synth.config5_weights(name)


KEYS = ["workload3/up", "workload3/down", "workload5/qkv", "workload5/o", "workload5/up", "workload5/down"]


@pytest.mark.gpu
@pytest.mark.parametrize("key", KEYS)
def test_record_matches_oracle_digests(gpu_lib, key):
    d = _load()
    chunk = d["chunk_rows"]
    w = _weights(key)
    n, k = w.shape
    wd = dev_bf16(w)
    del w
    widths = sorted(v["bits"] for kk, v in d["tensors"].items() if kk.startswith(key + "/"))
    assert widths, key
    for bits in widths:
        _case(f"quantize_pack {key} ({n} x {k}) bits={bits}: every row against the oracle's digests")
        ref = d["tensors"][f"{key}/{bits}"]
        assert (ref["rows"], ref["cols"]) == (n, k)
        qw = gpu_lib.quantize_pack(wd, bits)
        packed = host(qw.packed).reshape(n, k * bits // 8)
        scales = host(qw.scales).reshape(n, k // 128)
        for i, r0 in enumerate(range(0, n, chunk)):
            hp = hashlib.sha256(np.ascontiguousarray(packed[r0:r0 + chunk]).tobytes()).hexdigest()
            hs = hashlib.sha256(np.ascontiguousarray(scales[r0:r0 + chunk], dtype="<f4").view("<u4").tobytes()).hexdigest()
            assert hp == ref["packed"][i], f"{key} bits={bits}: packed bytes differ in rows {r0}..{r0 + chunk - 1}"
            assert hs == ref["scales"][i], f"{key} bits={bits}: scales differ in rows {r0}..{r0 + chunk - 1}"
        del qw, packed, scales


@pytest.mark.gpu
def test_workload4_residual_every_row(gpu_lib):
    """The float32 residual of workload 4 (after the rank-32 branch), 4 bits:
    packed bytes and scales of every row against the oracle."""
    _case("quantize_pack workload 4 residual (3072 x 3072 float32), every row")
    c = synth.config4(m=1)
    _, _, res = O.svd_split(c["w"], c["rank"])
    qw = gpu_lib.quantize_pack(dev_f32(res), 4)
    p_ref, s_ref, _ = O.quantize_pack(res, 4)
    assert np.array_equal(host(qw.packed).reshape(-1), p_ref)
    assert np.array_equal(f32_bits(host(qw.scales)).reshape(-1), f32_bits(s_ref).reshape(-1))


def test_digest_file_covers_the_workloads():
    """Workload 3 at 3/5/6/7 bits and workload 5 at 3..7 bits, all present."""
    d = _load()["tensors"]
    for key in KEYS:
        want = (3, 5, 6, 7) if key.startswith("workload3") else (3, 4, 5, 6, 7)
        assert sorted(v["bits"] for kk, v in d.items() if kk.startswith(key + "/")) == list(want)
