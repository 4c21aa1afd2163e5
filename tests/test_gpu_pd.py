"""GPU parity of the quantization-error tables ([WDQ] §3.2 inputs): the
library's per-row and total sums of (w - w_hat32)^2 at widths 3..7 against
the oracle (float64 sums in another order: relative 1e-12), and the whole
allocation (GPU tables + library search) against the oracle's."""
import numpy as np
import pytest
import torch

import oracle as O
from dit_dequant_gemm_amd import synth
from parity_util import dev_bf16, dev_f32

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _check_sse(api, w, f32):
    rows, total = api.quant_sse(dev_f32(w) if f32 else dev_bf16(w))
    torch.cuda.synchronize()
    rows = rows.cpu().numpy()
    total = total.cpu().numpy()
    for j, b in enumerate(O.PD_CANDIDATES):
        ref = O.quant_sse_rows(w, b)
        assert np.allclose(rows[:, j], ref, rtol=1e-12, atol=0.0), (b, np.max(np.abs(rows[:, j] - ref)))
        assert total[j] == pytest.approx(ref.sum(), rel=1e-12, abs=0.0)


@pytest.mark.parametrize("n,k", [(1, 128), (33, 384), (7, 4096), (64, 5120), (5, 13824), (3, 40960)])
def test_quant_sse_random(gpu_lib, n, k):
    _case(f"quant_sse n={n} k={k}")
    w = synth.random_case(n * 7 + k, 1, n, k, wstd=0.03)["w"]
    _check_sse(gpu_lib, w, False)


def test_quant_sse_edge_groups(gpu_lib):
    _case("quant_sse zero, constant, tiny and f32 groups")
    rng = np.random.default_rng(3)
    w = rng.standard_t(3, size=(8, 640)).astype(np.float32) * 0.02
    w[0] = 0.0                                  # all-zero row
    w[1, :128] = 0.0                            # one zero group
    w[2, 128:256] = np.float32(0.25)            # constant group
    w[3, 256:384] = -np.float32(0.25)
    w[4] *= np.float32(1e-30)                   # tiny (subnormal steps at 7 bits)
    _check_sse(gpu_lib, w, True)
    _check_sse(gpu_lib, synth.to_bf16(w), False)


def test_quant_sse_empty(gpu_lib):
    _case("quant_sse n=0")
    rows, total = gpu_lib.quant_sse(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert rows.shape == (0, 5) and np.all(total.cpu().numpy() == 0.0)


def test_allocation_end_to_end(gpu_lib):
    _case("sse_table on the GPU + library search against the oracle")
    rng = np.random.default_rng(11)
    ws = []
    for i in range(10):
        if i % 2:
            w = rng.standard_t(3 + i, size=(64, 1024)) * 0.02
        else:
            w = rng.normal(0, 0.02 * (1 + i / 5), size=(64, 1024))
        ws.append(synth.to_bf16(w))
    sse_gpu, n_gpu = gpu_lib.sse_table([dev_bf16(w) for w in ws])
    sse_ref, n_ref = O.sse_table(ws)
    mse_ref = sse_ref / n_ref[:, None]
    assert np.array_equal(n_gpu, n_ref)
    assert np.allclose(sse_gpu, sse_ref, rtol=1e-12, atol=0.0)
    t_init = 0.5 * np.random.default_rng(12).standard_normal((8, len(ws)))
    for target in (4.0, 4.7, 5.0):
        bits, info = gpu_lib.pd_allocate(sse_gpu, n_gpu, target, t_init, iters=300)
        ro = O.pd_search(mse_ref, n_ref, target, t_init, iters=300)
        assert np.array_equal(bits, ro["bits"]), (target, bits, ro["bits"])
        assert info["bpw"] <= target + 1e-9


def test_allocation_drives_a_grouped_block(gpu_lib):
    """The search's widths drive the block's products: every tensor packed at
    its allocated width (bytes and scales as the oracle's), then one grouped
    launch of the block's products at 16 tokens against the oracle product."""
    _case("allocation -> quantize_pack at the chosen widths -> grouped products")
    from parity_util import check_product, host
    rng = np.random.default_rng(31)
    shapes = [(256, 512), (256, 512), (256, 512), (256, 512), (704, 512), (512, 768)]
    ws = [synth.to_bf16(rng.normal(0, 0.01 * (1 + i), size=s)) for i, s in enumerate(shapes)]
    ws[3] = synth.to_bf16(rng.standard_t(3, size=shapes[3]) * 0.02)
    sse, nparams = gpu_lib.sse_table([dev_bf16(w) for w in ws])
    t_init = 0.5 * np.random.default_rng(32).standard_normal((6, len(ws)))
    bits, info = gpu_lib.pd_allocate(sse, nparams, 5.0, t_init, iters=300)
    assert info["bpw"] <= 5.0 + 1e-9 and len(set(bits.tolist())) > 1
    items, refs = [], []
    for i, (w, b) in enumerate(zip(ws, bits)):
        qw = gpu_lib.quantize_pack(dev_bf16(w), int(b))
        packed_ref, scales_ref, _ = O.quantize_pack(w, int(b))
        assert np.array_equal(host(qw.packed).reshape(-1), np.asarray(packed_ref).reshape(-1))
        assert np.array_equal(host(qw.scales).view(np.uint32).reshape(-1),
                              np.asarray(scales_ref, dtype=np.float32).view(np.uint32).reshape(-1))
        x = synth.to_bf16(rng.normal(0, 1, size=(16, w.shape[1])))
        items.append((dev_bf16(x), qw, torch.empty((16, w.shape[0]), dtype=torch.float32, device="cuda")))
        q_u, s = O.quantize_groups(w, int(b))
        refs.append(O.gemm_ref(x, O.dequant_bf16(q_u, s, int(b))))
    outs = gpu_lib.dequant_gemm_grouped(items)
    for b, y, ref in zip(bits, outs, refs):
        check_product(host(y), ref, False, f"allocated width {b}")
