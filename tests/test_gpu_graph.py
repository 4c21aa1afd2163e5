"""The binding's calls captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed with new inputs.

Called eagerly these shapes split K across workgroups (the 16-token 8-part
split, large-M split-K) or split the low-rank pre-pass, exchanging partial
sums tagged with a per-call epoch.  Under capture the binding hands over no
split-K workspace, so each replay computes whole tiles afresh.  Every replay
(three inputs, eager work and synchronizations between them) is checked
against the oracle, and two replays of one input must agree bit for bit.
"""
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


def _replays(g, x_static, y_static, xs, ref_of, bf):
    """Replay g once per input (copied into x_static between replays) and
    check each output; the first input again at the end, bit for bit."""
    outs = []
    for i, xh in enumerate(xs + xs[:1]):
        x_static.copy_(dev_bf16(xh))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y = host(y_static)
        outs.append(y)
        if i < len(xs):
            check_product(y, ref_of(xh), bf, f"replay {i}")
    assert np.array_equal(outs[0].view(np.uint32), outs[-1].view(np.uint32)), "replays of one input differ"


@pytest.mark.parametrize("m,n,k,bits", [(16, 1040, 8192, 4),     # 16 tokens, K split in 8 parts eagerly
                                        (1041, 2320, 1536, 5)])  # split-K over 50 tiles eagerly
def test_graph_replay_of_split_k_shapes(gpu_lib, m, n, k, bits):
    _case(f"graph capture: dequant_gemm m={m} n={n} k={k} bits={bits}")
    assert gpu_lib.workspace_bytes(m, n, k, 0) > 0, "an eager call of this shape splits K"
    c = synth.random_case(31 * m + n, m, n, k)
    qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
    w16 = O.dequant_bf16(*O.quantize_groups(c["w"], bits), bits)
    rng = np.random.default_rng(m + k)
    xs = [O.bf16_rne(rng.standard_normal((m, k)).astype(np.float32)) for _ in range(3)]
    x_static = dev_bf16(xs[0])
    y_static = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                       # warm-up on the capture's kind of stream
        gpu_lib.dequant_gemm(x_static, qw, out=y_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_lib.dequant_gemm(x_static, qw, out=y_static)
    # eager calls of the same product between replays use the split form
    eager = host(gpu_lib.dequant_gemm(dev_bf16(xs[1]), qw))
    check_product(eager, O.gemm_ref(xs[1], w16), True, "eager split call")
    _replays(g, x_static, y_static, xs, lambda xh: O.gemm_ref(xh, w16), True)


def test_graph_replay_of_lowrank_calls(gpu_lib):
    """The fused product at 16 tokens (eagerly: the pre-pass split over K) and
    the workspace-free entry point, each captured and replayed."""
    m, n, k, r, bits = 16, 272, 5120, 32, 4
    _case(f"graph capture: lowrank_fused_gemm and its workspace-free variant m={m} n={n} k={k} r={r}")
    c = synth.random_case(4711, m, n, k, wstd=0.05)
    l1, l2, res = O.svd_split(c["w"], r)
    qr = gpu_lib.quantize_pack(torch.from_numpy(res).to("cuda"), bits)
    w16 = O.dequant_bf16(*O.quantize_groups(res, bits), bits)
    ld = dev_bf16(np.ascontiguousarray(l1.T))
    lu = dev_bf16(np.ascontiguousarray(l2.T))
    rng = np.random.default_rng(99)
    xs = [O.bf16_rne(rng.standard_normal((m, k)).astype(np.float32)) for _ in range(3)]

    def ref_of(xh):
        return O.lowrank_fused_ref(xh, w16, l1, l2)[0]

    lib = gpu_lib.load_library()

    def noalloc(x, y):
        st = lib.ddg_lowrank_fused_gemm_noalloc(x.data_ptr(), m, k, qr.packed.data_ptr(), qr.scales.data_ptr(),
                                                bits, n, ld.data_ptr(), lu.data_ptr(), r, y.data_ptr(), 0,
                                                torch.cuda.current_stream().cuda_stream)
        assert st == 0, st

    for name, call in (("fused", lambda x, y: gpu_lib.lowrank_fused_gemm(x, qr, ld, lu, out=y)),
                       ("workspace-free", noalloc)):
        x_static = dev_bf16(xs[0])
        y_static = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(x_static, y_static)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(x_static, y_static)
        print(f"[case] {name}: captured", flush=True)
        _replays(g, x_static, y_static, xs, ref_of, True)
