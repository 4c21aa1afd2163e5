"""Guard bands around every output (stores outside an output buffer): each
output lives inside a larger allocation whose bytes before and after it hold
a seeded pattern, and the output itself starts as NaN (or a byte pattern).
After ragged-shape calls of every kernel the pattern must be intact, every
output element written, and the result equal to (or within the product bound
of) the oracle's."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from dit_dequant_gemm_amd import synth
from oracle import fp4 as F
from parity_util import check_product, dev_bf16, dev_f32, f32_bits, host

pytestmark = pytest.mark.gpu

PAD = 4096          # guard bytes on each side (keeps 16-byte alignment)


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


class Guarded:
    """A tensor of `shape`/`dtype` at byte offset PAD of a larger buffer."""

    def __init__(self, shape, dtype, seed):
        self.nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.empty(2 * PAD + self.nbytes, dtype=torch.uint8, device="cuda")
        rng = np.random.default_rng([1234, seed])
        self.head = rng.integers(0, 256, PAD, dtype=np.uint8)
        self.tail = rng.integers(0, 256, PAD, dtype=np.uint8)
        self.raw[:PAD] = torch.from_numpy(self.head).cuda()
        self.raw[PAD + self.nbytes:] = torch.from_numpy(self.tail).cuda()
        self.t = self.raw[PAD:PAD + self.nbytes].view(dtype).view(shape)
        if dtype.is_floating_point:
            self.t.fill_(float("nan"))
        else:
            self.raw[PAD:PAD + self.nbytes] = 0xA5

    def check(self, what):
        torch.cuda.synchronize()
        raw = self.raw.cpu().numpy()
        assert np.array_equal(raw[:PAD], self.head), f"{what}: bytes before the output changed"
        assert np.array_equal(raw[PAD + self.nbytes:], self.tail), f"{what}: bytes after the output changed"
        if self.t.dtype.is_floating_point:
            assert not torch.isnan(self.t).any().item(), f"{what}: output elements left unwritten"


def _w16(w, bits):
    q_u, s = O.quantize_groups(w, bits)
    return O.dequant_bf16(q_u, s, bits)


@pytest.mark.parametrize("bits", (3, 4, 5, 6, 7))
def test_quantize_pack_and_dequantize(gpu_lib, bits):
    n, k = 17, 384
    _case(f"guards: quantize_pack + dequantize n={n} k={k} bits={bits}")
    w = synth.random_case(bits, 1, n, k)["w"]
    lib = gpu_lib.load_library()
    gp = Guarded((n * k * bits // 8,), torch.uint8, 1)
    gs = Guarded((n, k // 128), torch.float32, 2)
    wd = dev_bf16(w)
    st = lib.ddg_quantize_pack(wd.data_ptr(), 0, n, k, bits, gp.t.data_ptr(), gs.t.data_ptr(), None)
    assert st == 0
    gp.check("packed")
    gs.check("scales")
    p_ref, s_ref, q_ref = O.quantize_pack(w, bits)
    assert np.array_equal(host(gp.t), p_ref)
    assert np.array_equal(f32_bits(host(gs.t)), f32_bits(s_ref))
    gw = Guarded((n, k), torch.bfloat16, 3)
    st = lib.ddg_dequantize(gp.t.data_ptr(), gs.t.data_ptr(), bits, n, k, gw.t.data_ptr(), None)
    assert st == 0
    gw.check("dense w_hat")
    assert np.array_equal(host(gw.t), O.dequant_bf16(q_ref, s_ref, bits))


# (m, n, k): the large-M tiles with ragged M and N; the small-M kernel at
# each row-block size; the weight-streaming kernel with a ragged last block
PRODUCTS = [(257, 272, 384), (65, 48, 256), (15, 272, 384), (17, 272, 384), (33, 80, 512),
            (64, 272, 256), (16, 12816, 384), (5, 12816, 256), (1, 16, 128),
            (1041, 2320, 1536), (2100, 528, 6144),          # split-K: 50 tiles x 2, 27 x 8
            (4160, 4080, 1280),                             # stream-K: 272 tiles
            (4160, 5136, 1280),                             # 459 tiles of 256 x 192
            (3800, 4112, 256),                              # 255 tiles of 256 x 256
            (16, 1040, 8192), (3, 272, 8320)]               # 16 tokens, K split in 8 parts


@pytest.mark.parametrize("m,n,k", PRODUCTS)
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16])
def test_dequant_gemm(gpu_lib, m, n, k, y_dtype):
    bits = 3 + (m + n) % 5
    _case(f"guards: dequant_gemm m={m} n={n} k={k} bits={bits} {y_dtype}")
    c = synth.random_case(m * 7 + n, m, n, k)
    qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
    g = Guarded((m, n), y_dtype, m + n)
    need = gpu_lib.workspace_bytes(m, n, k, 0)
    ws = Guarded((max(need, 16),), torch.uint8, m + n + 1)
    gpu_lib.dequant_gemm(dev_bf16(c["x"]), qw, out=g.t, workspace=ws.t)
    g.check("y")
    torch.cuda.synchronize()
    raw = ws.raw.cpu().numpy()
    assert np.array_equal(raw[:PAD], ws.head) and np.array_equal(raw[PAD + ws.nbytes:], ws.tail), "workspace guards"
    check_product(host(g.t), O.gemm_ref(c["x"], _w16(c["w"], bits)), y_dtype == torch.bfloat16)


def test_dequant_gemm_grouped(gpu_lib):
    _case("guards: dequant_gemm_grouped across its four launch classes")
    items, refs, guards = [], [], []
    for i, (m, n, k) in enumerate(PRODUCTS):
        bits = 3 + i % 5
        c = synth.random_case(500 + i, m, n, k)
        qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
        dt = torch.bfloat16 if i % 2 else torch.float32
        g = Guarded((m, n), dt, 600 + i)
        items.append((dev_bf16(c["x"]), qw, g.t))
        refs.append((O.gemm_ref(c["x"], _w16(c["w"], bits)), dt == torch.bfloat16))
        guards.append(g)
    gpu_lib.dequant_gemm_grouped(items)
    for i, (g, (ref, bf)) in enumerate(zip(guards, refs)):
        g.check(f"grouped product {i}")
        check_product(host(g.t), ref, bf, f"grouped product {i}")


@pytest.mark.parametrize("m,n,k", [(257, 272, 384), (17, 272, 384), (15, 272, 256), (5, 12816, 256),
                                   (3800, 4112, 256), (7, 272, 8192)])
def test_lowrank_fused_gemm(gpu_lib, m, n, k):
    r = 24
    _case(f"guards: lowrank_fused_gemm (workspace and no-allocation) m={m} n={n} k={k} r={r}")
    c = synth.random_case(m + 3 * n, m, n, k, wstd=0.05)
    l1, l2, res = O.svd_split(c["w"], r)
    qr = gpu_lib.quantize_pack(dev_f32(res), 4)
    ld = dev_bf16(np.ascontiguousarray(l1.T))
    lu = dev_bf16(np.ascontiguousarray(l2.T))
    y_ref, _ = O.lowrank_fused_ref(c["x"], _w16(res, 4), l1, l2)
    xd = dev_bf16(c["x"])
    need = gpu_lib.workspace_bytes(m, n, k, r)
    ws = Guarded((need,), torch.uint8, 77)
    g = Guarded((m, n), torch.float32, 78)
    gpu_lib.lowrank_fused_gemm(xd, qr, ld, lu, out=g.t, workspace=ws.t)
    g.check("y")
    torch.cuda.synchronize()
    raw = ws.raw.cpu().numpy()
    assert np.array_equal(raw[:PAD], ws.head) and np.array_equal(raw[PAD + ws.nbytes:], ws.tail), "workspace guards"
    check_product(host(g.t), y_ref, False, "lowrank")
    g2 = Guarded((m, n), torch.bfloat16, 79)
    gpu_lib.lowrank_fused_gemm_noalloc(xd, qr, ld, lu, g2.t)
    g2.check("y (no allocation)")
    check_product(host(g2.t), y_ref, True, "lowrank no-alloc")


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("m,n,k", [(300, 272, 384), (17, 48, 256)])
def test_w4a8_chain(gpu_lib, m, n, k, tiled):
    _case(f"guards: fp8_quantize_rows + w4a8_gemm m={m} n={n} k={k} tiled={tiled}")
    rng = np.random.default_rng(m + n + k)
    w = synth.to_bf16(rng.standard_t(4, size=(n, k)) * 0.02)
    x = synth.to_bf16(rng.normal(0, 1, size=(m, k)))
    lib = gpu_lib.load_library()
    gq = Guarded((m, k), torch.uint8, 11)
    gs = Guarded((m,), torch.float32, 12)
    st = lib.ddg_fp8_quantize_rows(dev_bf16(x).data_ptr(), m, k, gq.t.data_ptr(), gs.t.data_ptr(), None)
    assert st == 0
    gq.check("E4M3 codes")
    gs.check("row scales")
    cq, cs = F.quantize_rows_e4m3(x)
    assert np.array_equal(host(gq.t), cq) and np.array_equal(f32_bits(host(gs.t)), f32_bits(cs))
    qw = gpu_lib.fp4_quantize_pack(dev_bf16(w), "e2m1", tiled=tiled)
    wc, wsc = F.quantize_fp4_groups(w, "e2m1")
    g = Guarded((m, n), torch.bfloat16, 13)
    gpu_lib.w4a8_gemm(gq.t, gs.t, qw, out=g.t)
    g.check("y")
    check_product(host(g.t), F.w4a8_ref(cq, cs, wc, wsc, "e2m1"), True, "w4a8")


def test_w4a6_chain(gpu_lib):
    m, n, k = 33, 272, 384
    _case(f"guards: fp6_quantize_rows + w4a6_gemm m={m} n={n} k={k}")
    rng = np.random.default_rng(66)
    w = synth.to_bf16(rng.standard_t(4, size=(n, k)) * 0.02)
    x = synth.to_bf16(rng.normal(0, 1, size=(m, k)))
    lib = gpu_lib.load_library()
    size = -(-m // 32) * (k // 128) * 3072
    gq = Guarded((size,), torch.uint8, 21)
    gs = Guarded((m,), torch.float32, 22)
    st = lib.ddg_fp6_quantize_rows(dev_bf16(x).data_ptr(), m, k, 0, gq.t.data_ptr(), gs.t.data_ptr(), None)
    assert st == 0
    gq.check("FP6 storage")
    gs.check("row scales")
    cq, cs = F.quantize_rows_fp6(x, "e2m3")
    assert np.array_equal(host(gq.t), F.pack_fp6_tiled(cq))
    qw = gpu_lib.fp4_quantize_pack(dev_bf16(w), "e2m1", tiled=True)
    wc, wsc = F.quantize_fp4_groups(w, "e2m1")
    g = Guarded((m, n), torch.float32, 23)
    gpu_lib.w4a6_gemm(gq.t, gs.t, "e2m3", qw, out=g.t)
    g.check("y")
    check_product(host(g.t), F.w4a6_ref(cq, cs, wc, wsc, "e2m1", "e2m3"), False, "w4a6")


def test_fp4_quantize_pack(gpu_lib):
    n, k = 33, 384
    _case(f"guards: fp4_quantize_pack rows and tiled n={n} k={k}")
    w = synth.to_bf16(np.random.default_rng(5).standard_t(4, size=(n, k)) * 0.02)
    lib = gpu_lib.load_library()
    wc, wsc = F.quantize_fp4_groups(w, "e2m1")
    for tiled in (False, True):
        nb = -(-n // 32)
        pshape = (nb * (k // 128) * 2048,) if tiled else (n, k // 2)
        sshape = (nb * (k // 128) * 32,) if tiled else (n, k // 128)
        gp = Guarded(pshape, torch.uint8, 31 + tiled)
        gs = Guarded(sshape, torch.float32, 33 + tiled)
        st = lib.ddg_fp4_quantize_pack(dev_bf16(w).data_ptr(), 0, n, k, 0 | (0x200 if tiled else 0),
                                       gp.t.data_ptr(), gs.t.data_ptr(), None)
        assert st == 0
        gp.check("FP4 codes")
        gs.check("FP4 scales")
        if tiled:
            tp, ts = F.tile_fp4(F.pack_fp4(wc), wsc)
            assert np.array_equal(host(gp.t), tp) and np.array_equal(f32_bits(host(gs.t)), f32_bits(ts))
        else:
            assert np.array_equal(host(gp.t), F.pack_fp4(wc))
            assert np.array_equal(f32_bits(host(gs.t)), f32_bits(wsc))


def test_rpbh_rotate(gpu_lib):
    n, d, h = 5, 384, 128
    _case(f"guards: rpbh_rotate n={n} d={d} h={h}")
    x = np.random.default_rng(8).normal(0, 1, size=(n, d)).astype(np.float32)
    perm, signs = synth.rpbh_draw(d, 9)
    g = Guarded((n, d), torch.float32, 41)
    gpu_lib.rpbh_rotate(dev_f32(x), torch.from_numpy(perm).cuda(), torch.from_numpy(signs).cuda(), h, out=g.t)
    g.check("rotated rows")
    ref = O.rpbh_rotate(x, perm, signs, h)
    assert np.max(np.abs(host(g.t) - ref)) <= 1e-5 * np.max(np.abs(ref))
