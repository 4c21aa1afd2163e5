"""GPU parity of the FP4-weight / FP8-activation path ([FP4] §3.2, §4.1):
both quantizers bit for bit against the oracle, and the W4A8 product against
the oracle's float64 sum on the oracle's own codes and scales, to the usual
product bounds (relative Frobenius 1e-3, per-row 2e-2 of the row's largest).
Tighter, for float32 outputs: every element within 2^-14 times the same sum
over absolute values.  A chain of float32 additions would stay within
(130 + G) 2^-24 of it; the matrix instruction's own accumulation measured up
to 1.15x that, so the envelope sits well above it and far below what any
mis-paired operand produces (about 1/sqrt(k) of the absolute sum)."""
import numpy as np
import pytest
import torch

from dit_dequant_gemm_amd import synth
from oracle import fp4 as F
from parity_util import check_product, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _cuda_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _cuda_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("fmt", list(F.FP4_FORMATS))
@pytest.mark.parametrize("n,k,f32", [(16, 128, False), (33, 384, True), (64, 5120, False), (7, 1024, True)])
def test_fp4_quantize_bit_exact(gpu_lib, fmt, n, k, f32):
    _case(f"fp4_quantize_pack {fmt} n={n} k={k} f32={f32}")
    rng = np.random.default_rng(n * k)
    w = (rng.standard_t(4, size=(n, k)) * 0.02).astype(np.float32)
    if not f32:
        w = synth.to_bf16(w)
    qw = gpu_lib.fp4_quantize_pack(dev_f32(w) if f32 else dev_bf16(w), fmt)
    codes, s = F.quantize_fp4_groups(w, fmt)
    assert np.array_equal(host(qw.packed), F.pack_fp4(codes))
    assert np.array_equal(host(qw.scales).view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("fmt", list(F.FP4_FORMATS))
def test_fp4_quantize_ties_zero_and_tiny_groups(gpu_lib, fmt):
    _case(f"fp4_quantize_pack {fmt}: ties, zero, constant and tiny groups")
    lv = F.fp4_values(fmt)
    w = np.zeros((4, 256), dtype=np.float32)
    # group 0 of row 0: scale 1 (amax = vmax), values on every midpoint, both signs
    mids = (lv[1:] + lv[:-1]) / 2
    w[0, :128] = np.resize(np.concatenate([mids, -mids, [lv[-1]]]), 128)
    w[0, 0] = lv[-1]
    w[1, 128:] = np.float32(0.37)                      # constant group
    w[2, :128] = np.random.default_rng(1).normal(0, 1, 128).astype(np.float32) * np.float32(1e-41)
    # row 3 stays zero
    qw = gpu_lib.fp4_quantize_pack(dev_f32(w), fmt)
    codes, s = F.quantize_fp4_groups(w, fmt)
    assert np.array_equal(host(qw.packed), F.pack_fp4(codes))
    assert np.array_equal(host(qw.scales).view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("m,k", [(1, 128), (5, 384), (64, 3072), (3, 13824), (2, 20480)])
def test_fp8_rows_bit_exact(gpu_lib, m, k):
    _case(f"fp8_quantize_rows m={m} k={k}")
    x = synth.to_bf16(np.random.default_rng(m + k).normal(0, 1, size=(m, k)))
    xq, xs = gpu_lib.fp8_quantize_rows(dev_bf16(x))
    cq, cs = F.quantize_rows_e4m3(x)
    assert np.array_equal(host(xq), cq)
    assert np.array_equal(host(xs).view(np.uint32), cs.view(np.uint32))


def test_fp8_rows_ties_subnormals_and_zero_rows(gpu_lib):
    _case("fp8_quantize_rows: ties, subnormal range, zero row")
    lv = F.e4m3_values()
    x = np.zeros((3, 384), dtype=np.float64)
    mids = (lv[1:] + lv[:-1]) / 2                      # scale 1: amax = 448
    x[0, :len(mids)] = mids
    x[0, 200:200 + 100] = -mids[:100]
    x[0, 383] = 448.0
    x[1, :] = np.random.default_rng(2).normal(0, 1, 384)
    x[1, 0] = 4096.0                                   # most of the row lands in the subnormal range
    x = synth.to_bf16(x)
    xq, xs = gpu_lib.fp8_quantize_rows(dev_bf16(x))
    cq, cs = F.quantize_rows_e4m3(x)
    assert np.array_equal(host(xq), cq)
    assert np.array_equal(host(xs).view(np.uint32), cs.view(np.uint32))


def _check_f32_product(y, xc, xs, wc, ws, ref, fmt="e2m1"):
    absref = F.w4a8_ref(xc & 0x7F, xs, wc & 7, ws, fmt)           # the same sum over magnitudes
    assert np.all(np.abs(y - ref) <= 2.0 ** -14 * absref + 1e-37), \
        float(np.max(np.abs(y - ref) / (absref + 1e-37)))
    check_product(y, ref, False, f"w4a8 f32 k={xc.shape[1]}")


def _product_case(gpu_lib, m, n, k, seed, out_dtype, fmt="e2m1"):
    rng = np.random.default_rng(seed)
    w = synth.to_bf16(rng.standard_t(4, size=(n, k)) * 0.02)
    x = synth.to_bf16(rng.normal(0, 1, size=(m, k)))
    wc, ws = F.quantize_fp4_groups(w, fmt)
    xc, xs = F.quantize_rows_e4m3(x)
    qw = gpu_lib.QWeightFP4(_cuda_u8(F.pack_fp4(wc)), _cuda_f32(ws), fmt, n, k)
    y = host(gpu_lib.w4a8_gemm(_cuda_u8(xc), _cuda_f32(xs), qw, out_dtype))
    return y, F.w4a8_ref(xc, xs, wc, ws, fmt), (xc, xs, wc, ws)


@pytest.mark.parametrize("fmt", list(F.FP4_FORMATS))
@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (17, 48, 384), (256, 256, 1024), (300, 272, 640),
                                   (513, 300, 2048), (64, 1000, 128)])
def test_w4a8_gemm(gpu_lib, m, n, k, fmt):
    _case(f"w4a8_gemm {fmt} m={m} n={n} k={k}")
    y, ref, codes = _product_case(gpu_lib, m, n, k, m * n + k, torch.float32, fmt)
    _check_f32_product(y, *codes, ref, fmt)
    yb, _, _ = _product_case(gpu_lib, m, n, k, m * n + k, torch.bfloat16, fmt)
    check_product(yb, ref, True, f"w4a8 bf16 {fmt} m={m} n={n} k={k}")


def test_w4a8_attention_projection_sampled(gpu_lib):
    """The bench shape (4096 x 3072 x 3072) on sampled rows."""
    _case("w4a8_gemm 4096 x 3072 x 3072 (sampled rows)")
    c = synth.config2()
    wc, ws = F.quantize_fp4_groups(c["w"], "e2m1")
    xc, xs = F.quantize_rows_e4m3(c["x"])
    qw = gpu_lib.QWeightFP4(_cuda_u8(F.pack_fp4(wc)), _cuda_f32(ws), "e2m1", 3072, 3072)
    y = host(gpu_lib.w4a8_gemm(_cuda_u8(xc), _cuda_f32(xs), qw, torch.float32))
    rows = np.r_[0:32, 2040:2072, 4064:4096]
    ref = F.w4a8_ref(xc[rows], xs[rows], wc, ws, "e2m1")
    _check_f32_product(y[rows], xc[rows], xs[rows], wc, ws, ref)


@pytest.mark.parametrize("fmt", list(F.FP4_FORMATS))
def test_w4a8_chain(gpu_lib, fmt):
    """The GPU quantizers feed the product; m = 0 is a no-op."""
    _case(f"w4a8 chain {fmt}: GPU quantizers -> product")
    rng = np.random.default_rng(9)
    w = synth.to_bf16(rng.normal(0, 0.02, size=(64, 256)))
    x = synth.to_bf16(rng.normal(0, 1, size=(40, 256)))
    qw = gpu_lib.fp4_quantize_pack(dev_bf16(w), fmt)
    xq, xs = gpu_lib.fp8_quantize_rows(dev_bf16(x))
    y = host(gpu_lib.w4a8_gemm(xq, xs, qw, torch.float32))
    wc, wsc = F.quantize_fp4_groups(w, fmt)
    xc, xsc = F.quantize_rows_e4m3(x)
    ref = F.w4a8_ref(xc, xsc, wc, wsc, fmt)
    _check_f32_product(y, xc, xsc, wc, wsc, ref, fmt)
    assert gpu_lib.w4a8_gemm(xq[:0], xs[:0], qw, torch.float32).shape == (0, 64)


@pytest.mark.parametrize("fmt", list(F.FP4_FORMATS))
@pytest.mark.parametrize("n,k,f32", [(16, 128, False), (33, 384, True), (64, 5120, False)])
def test_fp4_quantize_pow2_bit_exact(gpu_lib, fmt, n, k, f32):
    _case(f"fp4_quantize_pack {fmt} power-of-two scales n={n} k={k} f32={f32}")
    rng = np.random.default_rng(n * k + 1)
    w = (rng.standard_t(4, size=(n, k)) * 0.02).astype(np.float32)
    w[0, :128] = 0.0
    w[-1, -128:] *= np.float32(1e-39)                    # scale below 2^-126
    if not f32:
        w = synth.to_bf16(w)
    qw = gpu_lib.fp4_quantize_pack(dev_f32(w) if f32 else dev_bf16(w), fmt, pow2=True)
    codes, s = F.quantize_fp4_groups(w, fmt, pow2=True)
    assert qw.pow2
    assert np.array_equal(host(qw.packed), F.pack_fp4(codes))
    assert np.array_equal(host(qw.scales).view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("fmt", list(F.FP4_FORMATS))
@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (300, 272, 640), (513, 300, 2048)])
def test_w4a8_gemm_pow2(gpu_lib, m, n, k, fmt):
    """Power-of-two group scales, applied by the matrix instruction."""
    _case(f"w4a8_gemm power-of-two scales {fmt} m={m} n={n} k={k}")
    rng = np.random.default_rng(m + n + k)
    w = synth.to_bf16(rng.standard_t(4, size=(n, k)) * 0.02)
    w[1, :128] = 0.0                                     # a zero group: scale 0
    x = synth.to_bf16(rng.normal(0, 1, size=(m, k)))
    wc, ws = F.quantize_fp4_groups(w, fmt, pow2=True)
    xc, xs = F.quantize_rows_e4m3(x)
    ref = F.w4a8_ref(xc, xs, wc, ws, fmt)
    for dt in (torch.float32, torch.bfloat16):
        qw = gpu_lib.QWeightFP4(_cuda_u8(F.pack_fp4(wc)), _cuda_f32(ws), fmt, n, k, pow2=True)
        y = host(gpu_lib.w4a8_gemm(_cuda_u8(xc), _cuda_f32(xs), qw, dt))
        if dt == torch.float32:
            _check_f32_product(y, xc, xs, wc, ws, ref, fmt)
        else:
            check_product(y, ref, True, f"w4a8 pow2 bf16 {fmt} m={m} n={n} k={k}")


def test_w4a8_pow2_chain_attention_projection_sampled(gpu_lib):
    """GPU quantizers (power-of-two scales) feeding the product at 4096 x 3072 x 3072."""
    _case("w4a8 pow2 chain 4096 x 3072 x 3072 (sampled rows)")
    c = synth.config2()
    qw = gpu_lib.fp4_quantize_pack(dev_bf16(c["w"]), "e2m1", pow2=True)
    xq, xs = gpu_lib.fp8_quantize_rows(dev_bf16(c["x"]))
    y = host(gpu_lib.w4a8_gemm(xq, xs, qw, torch.float32))
    wc, ws = F.quantize_fp4_groups(c["w"], "e2m1", pow2=True)
    rows = np.r_[0:32, 4064:4096]
    xc, xsc = F.quantize_rows_e4m3(c["x"][rows])
    assert np.array_equal(host(qw.scales).view(np.uint32), ws.view(np.uint32))
    _check_f32_product(y[rows], xc, xsc, wc, ws, F.w4a8_ref(xc, xsc, wc, ws, "e2m1"))


@pytest.mark.parametrize("fmt", list(F.FP4_FORMATS))
@pytest.mark.parametrize("n,k,f32,pow2", [(16, 128, False, False), (33, 384, True, True), (100, 5120, False, False),
                                          (64, 256, True, False), (7, 1024, False, True)])
def test_fp4_quantize_tiled_bit_exact(gpu_lib, fmt, n, k, f32, pow2):
    _case(f"fp4_quantize_pack tiled {fmt} n={n} k={k} f32={f32} pow2={pow2}")
    rng = np.random.default_rng(n * k + 2)
    w = (rng.standard_t(4, size=(n, k)) * 0.02).astype(np.float32)
    w[n // 2, :128] = 0.0
    if not f32:
        w = synth.to_bf16(w)
    qw = gpu_lib.fp4_quantize_pack(dev_f32(w) if f32 else dev_bf16(w), fmt, pow2=pow2, tiled=True)
    codes, s = F.quantize_fp4_groups(w, fmt, pow2=pow2)
    t, ts = F.tile_fp4(F.pack_fp4(codes), s)
    assert qw.tiled and qw.packed.shape == t.shape and qw.scales.shape == ts.shape
    assert np.array_equal(host(qw.packed), t)                  # padding columns included: zero codes
    assert np.array_equal(host(qw.scales).view(np.uint32), ts.view(np.uint32))
    # layout-free: back in row order, the codes and scales are the oracle's
    back, bs = F.untile_fp4(host(qw.packed), host(qw.scales), n, k)
    assert np.array_equal(F.unpack_fp4(back), codes)
    assert np.array_equal(np.asarray(bs, dtype=np.float32).view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("fmt", list(F.FP4_FORMATS))
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (300, 272, 640), (513, 300, 2048), (64, 1000, 128),
                                   (257, 33, 384)])
def test_w4a8_gemm_tiled(gpu_lib, m, n, k, fmt, pow2):
    """The product on tiled weights (oracle codes, tiled by the oracle)."""
    _case(f"w4a8_gemm tiled {fmt} pow2={pow2} m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 7 + n + k)
    w = synth.to_bf16(rng.standard_t(4, size=(n, k)) * 0.02)
    x = synth.to_bf16(rng.normal(0, 1, size=(m, k)))
    wc, ws = F.quantize_fp4_groups(w, fmt, pow2=pow2)
    xc, xs = F.quantize_rows_e4m3(x)
    t, ts = F.tile_fp4(F.pack_fp4(wc), ws)
    qw = gpu_lib.QWeightFP4(_cuda_u8(t), _cuda_f32(ts), fmt, n, k, pow2=pow2, tiled=True)
    ref = F.w4a8_ref(xc, xs, wc, ws, fmt)
    y = host(gpu_lib.w4a8_gemm(_cuda_u8(xc), _cuda_f32(xs), qw, torch.float32))
    _check_f32_product(y, xc, xs, wc, ws, ref, fmt)
    yb = host(gpu_lib.w4a8_gemm(_cuda_u8(xc), _cuda_f32(xs), qw, torch.bfloat16))
    check_product(yb, ref, True, f"w4a8 tiled bf16 {fmt} m={m} n={n} k={k}")


def test_w4a8_tiled_chain_attention_projection_sampled(gpu_lib):
    """GPU quantizers (tiled, float32 scales) feeding the product at 4096 x 3072 x 3072."""
    _case("w4a8 tiled chain 4096 x 3072 x 3072 (sampled rows)")
    c = synth.config2()
    qw = gpu_lib.fp4_quantize_pack(dev_bf16(c["w"]), "e2m1", tiled=True)
    xq, xs = gpu_lib.fp8_quantize_rows(dev_bf16(c["x"]))
    y = host(gpu_lib.w4a8_gemm(xq, xs, qw, torch.float32))
    wc, ws = F.quantize_fp4_groups(c["w"], "e2m1")
    rows = np.r_[0:32, 2048:2080, 4064:4096]
    xc, xsc = F.quantize_rows_e4m3(c["x"][rows])
    _check_f32_product(y[rows], xc, xsc, wc, ws, F.w4a8_ref(xc, xsc, wc, ws, "e2m1"))


# ---- W4A6: 6-bit activations ----

@pytest.mark.parametrize("fmt", list(F.FP6_FORMATS))
@pytest.mark.parametrize("m,k", [(1, 128), (5, 384), (33, 256), (100, 3072), (64, 13824), (3, 20480)])
def test_fp6_rows_bit_exact(gpu_lib, fmt, m, k):
    _case(f"fp6_quantize_rows {fmt} m={m} k={k}")
    x = synth.to_bf16(np.random.default_rng(m * 3 + k).normal(0, 1, size=(m, k)))
    if m > 4:
        x[3] = 0.0                                         # a zero row
    xq, xs = gpu_lib.fp6_quantize_rows(dev_bf16(x), fmt)
    cq, cs = F.quantize_rows_fp6(x, fmt)
    assert np.array_equal(host(xq), F.pack_fp6_tiled(cq))  # padding rows included: zero codes
    assert np.array_equal(F.unpack_fp6_tiled(host(xq), m, k), cq)   # layout-free: row order
    assert np.array_equal(host(xs).view(np.uint32), cs.view(np.uint32))


@pytest.mark.parametrize("fmt", list(F.FP6_FORMATS))
def test_fp6_rows_ties_and_subnormals(gpu_lib, fmt):
    _case(f"fp6_quantize_rows {fmt}: midpoints, subnormal range")
    lv = F.fp6_values(fmt)
    x = np.zeros((3, 128), dtype=np.float64)
    mids = (lv[1:] + lv[:-1]) / 2                          # scale 1: the row's amax is the top level
    x[0, :31] = mids
    x[0, 40:71] = -mids
    x[0, 127] = lv[-1]
    x[1] = np.random.default_rng(4).normal(0, 1, 128)
    x[1, 0] = 1000.0                                       # most of the row in the subnormal range
    x = synth.to_bf16(x)
    xq, xs = gpu_lib.fp6_quantize_rows(dev_bf16(x), fmt)
    cq, cs = F.quantize_rows_fp6(x, fmt)
    assert np.array_equal(host(xq), F.pack_fp6_tiled(cq))
    assert np.array_equal(host(xs).view(np.uint32), cs.view(np.uint32))


def _check_w4a6_f32(y, xc, xs, wc, ws, ref, afmt, wfmt="e2m1"):
    absref = F.w4a6_ref(xc & 31, xs, wc & 7, ws, wfmt, afmt)
    assert np.all(np.abs(y - ref) <= 2.0 ** -14 * absref + 1e-37), \
        float(np.max(np.abs(y - ref) / (absref + 1e-37)))
    check_product(y, ref, False, f"w4a6 f32 {afmt} k={xc.shape[1]}")


@pytest.mark.parametrize("wfmt", list(F.FP4_FORMATS))
@pytest.mark.parametrize("afmt", list(F.FP6_FORMATS))
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (300, 272, 640), (513, 300, 2048), (64, 1000, 128),
                                   (257, 33, 384)])
def test_w4a6_gemm(gpu_lib, m, n, k, afmt, pow2, wfmt):
    """The product on the oracle's FP6 codes (tiled by the oracle) and tiled
    FP4 weights of every format (E3M0 and E1M2 as FP8 operands)."""
    _case(f"w4a6_gemm {wfmt} x {afmt} pow2={pow2} m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 11 + n + k)
    w = synth.to_bf16(rng.standard_t(4, size=(n, k)) * 0.02)
    x = synth.to_bf16(rng.normal(0, 1, size=(m, k)))
    wc, ws = F.quantize_fp4_groups(w, wfmt, pow2=pow2)
    xc, xs = F.quantize_rows_fp6(x, afmt)
    t, ts = F.tile_fp4(F.pack_fp4(wc), ws)
    qw = gpu_lib.QWeightFP4(_cuda_u8(t), _cuda_f32(ts), wfmt, n, k, pow2=pow2, tiled=True)
    ref = F.w4a6_ref(xc, xs, wc, ws, wfmt, afmt)
    xq = _cuda_u8(F.pack_fp6_tiled(xc))
    y = host(gpu_lib.w4a6_gemm(xq, _cuda_f32(xs), afmt, qw, torch.float32))
    _check_w4a6_f32(y, xc, xs, wc, ws, ref, afmt, wfmt)
    yb = host(gpu_lib.w4a6_gemm(xq, _cuda_f32(xs), afmt, qw, torch.bfloat16))
    check_product(yb, ref, True, f"w4a6 bf16 {wfmt} x {afmt} m={m} n={n} k={k}")


@pytest.mark.parametrize("afmt", list(F.FP6_FORMATS))
def test_w4a6_chain_attention_projection_sampled(gpu_lib, afmt):
    """GPU quantizers feeding the W4A6 product at 4096 x 3072 x 3072; m = 0 is a no-op."""
    _case(f"w4a6 chain {afmt} 4096 x 3072 x 3072 (sampled rows)")
    c = synth.config2()
    qw = gpu_lib.fp4_quantize_pack(dev_bf16(c["w"]), "e2m1", tiled=True)
    xq, xs = gpu_lib.fp6_quantize_rows(dev_bf16(c["x"]), afmt)
    y = host(gpu_lib.w4a6_gemm(xq, xs, afmt, qw, torch.float32))
    wc, ws = F.quantize_fp4_groups(c["w"], "e2m1")
    rows = np.r_[0:32, 2048:2080, 4064:4096]
    xc, xsc = F.quantize_rows_fp6(c["x"][rows], afmt)
    _check_w4a6_f32(y[rows], xc, xsc, wc, ws, F.w4a6_ref(xc, xsc, wc, ws, "e2m1", afmt), afmt)
    empty = gpu_lib.w4a6_gemm(xq[:0], xs[:0], afmt, qw, torch.float32)
    assert empty.shape == (0, 3072)


@pytest.mark.parametrize("fmt", ["e4m3"] + list(F.FP6_FORMATS))
def test_rows_quantizers_extreme_scales(gpu_lib, fmt):
    """Rows whose scale falls below 2^-60 (the quantizers' exact-division
    path), just above it (the multiply-and-correct path with the tiniest
    elements), and far above 1: bit for bit against the oracle."""
    _case(f"row quantizer {fmt}: extreme row scales")
    rng = np.random.default_rng(12)
    x = rng.normal(0, 1, size=(6, 384))
    for r, e in enumerate((-80, -68, -52, -40, 40, 100)):
        x[r] *= 2.0 ** e
    x = synth.to_bf16(x)
    if fmt == "e4m3":
        xq, xs = gpu_lib.fp8_quantize_rows(dev_bf16(x))
        cq, cs = F.quantize_rows_e4m3(x)
        assert np.array_equal(host(xq), cq)
    else:
        xq, xs = gpu_lib.fp6_quantize_rows(dev_bf16(x), fmt)
        cq, cs = F.quantize_rows_fp6(x, fmt)
        assert np.array_equal(host(xq), F.pack_fp6_tiled(cq))
    assert np.array_equal(host(xs).view(np.uint32), cs.view(np.uint32))


# ---- W6A8: FP6 weights ----

@pytest.mark.parametrize("fmt", list(F.FP6_FORMATS))
@pytest.mark.parametrize("n,k,f32,pow2", [(16, 128, False, False), (33, 384, True, True), (100, 5120, False, False),
                                          (64, 256, True, False), (7, 1024, False, True), (300, 640, False, True)])
def test_fp6_weight_quantize_bit_exact(gpu_lib, fmt, n, k, f32, pow2):
    _case(f"fp6_quantize_pack {fmt} n={n} k={k} f32={f32} pow2={pow2}")
    rng = np.random.default_rng(n * k + 5)
    w = (rng.standard_t(4, size=(n, k)) * 0.02).astype(np.float32)
    w[n // 2, :128] = 0.0                                      # a zero group
    if not f32:
        w = synth.to_bf16(w)
    qw = gpu_lib.fp6_quantize_pack(dev_f32(w) if f32 else dev_bf16(w), fmt, pow2=pow2)
    codes, s = F.quantize_fp6_groups(w, fmt, pow2=pow2)
    # layout-free: back in row order, the codes and scales are the oracle's
    assert np.array_equal(F.unpack_fp6_tiled(host(qw.packed), n, k), codes)
    bs = F.untile_group_scales(host(qw.scales), n, k)
    assert np.array_equal(bs.view(np.uint32), s.view(np.uint32))
    # the stored bytes, padding rows included (zero codes and scales)
    assert np.array_equal(host(qw.packed), F.pack_fp6_tiled(codes))
    assert np.array_equal(host(qw.scales).view(np.uint32), F.tile_group_scales(s).view(np.uint32))


@pytest.mark.parametrize("fmt", list(F.FP6_FORMATS))
def test_fp6_weight_quantize_ties_and_tiny_groups(gpu_lib, fmt):
    """Hand-made groups with power-of-two scales whose quotients land on every
    midpoint between levels (ties to the even code) and on the levels, a
    group of subnormal weights and a zero group."""
    _case(f"fp6_quantize_pack ties {fmt}")
    lv = F.fp6_values(fmt).astype(np.float32)
    mids = np.concatenate([(lv[1:] + lv[:-1]) / 2, lv, -(lv[1:] + lv[:-1]) / 2]).astype(np.float32)
    w = np.zeros((4, 256), dtype=np.float32)
    w[0, :mids.size] = mids * np.float32(0.125)                # group amax = top level -> s = 0.125
    w[1, :128] = np.linspace(-1, 1, 128, dtype=np.float32) * np.float32(1e-39)
    w[2, 128:] = rng_vals = np.random.default_rng(14).normal(0, 3, 128).astype(np.float32)
    qw = gpu_lib.fp6_quantize_pack(dev_f32(w), fmt)
    codes, s = F.quantize_fp6_groups(w, fmt)
    assert s[0, 0] == np.float32(0.125) and s[3, 0] == 0 and s[3, 1] == 0 and rng_vals.size == 128
    assert np.array_equal(F.unpack_fp6_tiled(host(qw.packed), 4, 256), codes)
    assert np.array_equal(F.untile_group_scales(host(qw.scales), 4, 256).view(np.uint32), s.view(np.uint32))


def _check_w6a8_f32(y, xc, xs, wc, ws, ref, wfmt):
    absref = F.w6a8_ref(xc & 0x7F, xs, wc & 31, ws, wfmt)       # the same sum over magnitudes
    assert np.all(np.abs(y - ref) <= 2.0 ** -14 * absref + 1e-37), \
        float(np.max(np.abs(y - ref) / (absref + 1e-37)))
    check_product(y, ref, False, f"w6a8 f32 {wfmt} k={xc.shape[1]}")


@pytest.mark.parametrize("wfmt", list(F.FP6_FORMATS))
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (300, 272, 640), (513, 300, 2048), (64, 1000, 128),
                                   (257, 33, 384)])
def test_w6a8_gemm(gpu_lib, m, n, k, wfmt, pow2):
    """The product on the oracle's FP6 weight codes (stored by the oracle) and
    E4M3 activation codes."""
    _case(f"w6a8_gemm {wfmt} pow2={pow2} m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 13 + n + k)
    w = synth.to_bf16(rng.standard_t(4, size=(n, k)) * 0.02)
    x = synth.to_bf16(rng.normal(0, 1, size=(m, k)))
    wc, ws = F.quantize_fp6_groups(w, wfmt, pow2=pow2)
    xc, xs = F.quantize_rows_e4m3(x)
    qw = gpu_lib.QWeightFP6(_cuda_u8(F.pack_fp6_tiled(wc)), _cuda_f32(F.tile_group_scales(ws)), wfmt, n, k, pow2=pow2)
    ref = F.w6a8_ref(xc, xs, wc, ws, wfmt)
    y = host(gpu_lib.w6a8_gemm(_cuda_u8(xc), _cuda_f32(xs), qw, torch.float32))
    _check_w6a8_f32(y, xc, xs, wc, ws, ref, wfmt)
    yb = host(gpu_lib.w6a8_gemm(_cuda_u8(xc), _cuda_f32(xs), qw, torch.bfloat16))
    check_product(yb, ref, True, f"w6a8 bf16 {wfmt} m={m} n={n} k={k}")


@pytest.mark.parametrize("wfmt", list(F.FP6_FORMATS))
def test_w6a8_chain_attention_projection_sampled(gpu_lib, wfmt):
    """GPU quantizers feeding the W6A8 product at 4096 x 3072 x 3072; m = 0 is a no-op."""
    _case(f"w6a8 chain {wfmt} 4096 x 3072 x 3072 (sampled rows)")
    c = synth.config2()
    qw = gpu_lib.fp6_quantize_pack(dev_bf16(c["w"]), wfmt)
    xq, xs = gpu_lib.fp8_quantize_rows(dev_bf16(c["x"]))
    y = host(gpu_lib.w6a8_gemm(xq, xs, qw, torch.float32))
    wc, ws = F.quantize_fp6_groups(c["w"], wfmt)
    rows = np.r_[0:32, 2048:2080, 4064:4096]
    xc, xsc = F.quantize_rows_e4m3(c["x"][rows])
    _check_w6a8_f32(y[rows], xc, xsc, wc, ws, F.w6a8_ref(xc, xsc, wc, ws, wfmt), wfmt)
    empty = gpu_lib.w6a8_gemm(xq[:0], xs[:0], qw, torch.float32)
    assert empty.shape == (0, 3072)
