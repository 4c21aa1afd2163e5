"""The fused low-rank product without a workspace (for callers that cannot
allocate): through the C ABI, against the entry point that takes a
workspace, given one of T's bytes alone (same kernels: equal bit for bit) and against the oracle (the
product's tolerance), on consecutive calls that share the library's device
array, the second one smaller."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from dit_dequant_gemm_amd import synth
from parity_util import check_product, dev_bf16, host

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _prepare(api, seed, m, n, k, r, bits):
    c = synth.random_case(seed, m, n, k, wstd=0.05)
    l1, l2, res = O.svd_split(c["w"], r)
    qr = api.quantize_pack(torch.from_numpy(res).to("cuda"), bits)
    w16 = O.dequant_bf16(*O.quantize_groups(res, bits), bits)
    ld = dev_bf16(np.ascontiguousarray(l1.T))
    lu = dev_bf16(np.ascontiguousarray(l2.T))
    return c["x"], dev_bf16(c["x"]), qr, ld, lu, (w16, l1, l2)


def _noalloc(lib, x, qr, ld, lu, y):
    dt = 1 if y.dtype == torch.float32 else 0
    st = lib.ddg_lowrank_fused_gemm_noalloc(x.data_ptr(), x.shape[0], qr.k, qr.packed.data_ptr(),
                                            qr.scales.data_ptr(), qr.bits, qr.n, ld.data_ptr(),
                                            lu.data_ptr(), ld.shape[0], y.data_ptr(), dt,
                                            torch.cuda.current_stream().cuda_stream)
    assert st == 0, st


@pytest.mark.parametrize("first,second", [
    # (m, n, k, r, bits, y dtype): the large-M kernel, then the small-M one
    ((300, 512, 768, 32, 5, torch.float32), (16, 256, 384, 16, 4, torch.bfloat16)),
    # the largest T the array holds (32768 x 128 bf16 = 8 MiB), then a tiny one
    ((32768, 256, 256, 128, 6, torch.bfloat16), (3, 48, 256, 8, 3, torch.float32)),
])
def test_noalloc_matches_workspace_call(gpu_lib, first, second):
    lib = gpu_lib.load_library()
    cases = []
    for i, (m, n, k, r, bits, dt) in enumerate((first, second)):
        _case(f"lowrank_fused_gemm_noalloc call {i}: m={m} n={n} k={k} r={r} bits={bits}")
        xh, x, qr, ld, lu, ref = _prepare(gpu_lib, 900 + 17 * i + m, m, n, k, r, bits)
        # a workspace of T's bytes alone: whole tiles, as the call without one
        t_ws = torch.empty(max(256, -(-m * r * 2 // 256) * 256), dtype=torch.uint8, device="cuda")
        y_ws = gpu_lib.lowrank_fused_gemm(x, qr, ld, lu, out_dtype=dt, workspace=t_ws)
        y_na = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
        cases.append((xh, x, qr, ld, lu, ref, y_ws, y_na, dt))
    torch.cuda.synchronize()
    # the two calls back to back on one stream: the second overwrites the
    # array the first used
    for xh, x, qr, ld, lu, ref, y_ws, y_na, dt in cases:
        _noalloc(lib, x, qr, ld, lu, y_na)
    for xh, x, qr, ld, lu, (w16, l1, l2), y_ws, y_na, dt in cases:
        a, b = host(y_na), host(y_ws)                # float32 (bf16 values exactly)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        rows = np.unique(np.concatenate([np.arange(min(64, xh.shape[0])),
                                         np.arange(max(0, xh.shape[0] - 64), xh.shape[0])]))
        y_ref, _ = O.lowrank_fused_ref(xh[rows], w16, l1, l2)
        check_product(a[rows], y_ref, dt == torch.bfloat16, "noalloc")
