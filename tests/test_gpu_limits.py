"""GPU parity at the limits of the C ABI: the largest K it accepts (2^20), and
buffers past 4 GiB (an input, a packed weight and an output), so that every
byte offset a kernel forms above 2^32 is exercised.

Large inputs are built on the GPU by repeating a seeded block from the input
generators; the rows that are checked are overwritten with rows of their own
(another seeded draw), so an offset that wrapped at 32 bits would read other
data and fail the comparison.  The oracle quantizes and multiplies only the
checked rows.  Same bars as the other parity tests: packed bytes and scales
bit for bit, products within a relative Frobenius error of 1e-3 and a per-row
max error of 2e-2 * max |row|.
"""
import numpy as np
import pytest
import torch

import oracle as O
from dit_dequant_gemm_amd import synth
from parity_util import check_product, dev_bf16, dev_f32, f32_bits, host

pytestmark = pytest.mark.gpu

K_MAX = 1 << 20          # the largest K the C ABI accepts
GIB4 = 1 << 32


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _rows_to_host(t, rows):
    idx = torch.as_tensor(rows, device=t.device, dtype=torch.long)
    return t.index_select(0, idx).float().cpu().numpy()


def _w16(w, bits):
    q_u, s = O.quantize_groups(w, bits)
    return O.dequant_bf16(q_u, s, bits)


@pytest.mark.parametrize("bits", (3, 7))
def test_quantize_and_gemm_at_k_max(gpu_lib, bits):
    """K = 2^20 (8192 groups per row) with N = 32: M = 4 (the small-M kernel
    with one row block), 20 (two row blocks), 80 (large tiles).  The
    weight-streaming kernel (M <= 16 with N >= 12800), the grouped kernels,
    the low-rank pre-pass and the W4A8 product at this K follow."""
    c = synth.random_case(31 + bits, 80, 32, K_MAX)
    _case(f"quantize_pack 32 x 2^20 bits={bits}")
    qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
    p_ref, s_ref, q_ref = O.quantize_pack(c["w"], bits)
    assert np.array_equal(host(qw.packed).reshape(-1), p_ref), "packed bytes differ"
    assert np.array_equal(f32_bits(host(qw.scales).reshape(-1)), f32_bits(s_ref.reshape(-1))), "scales differ"
    w16 = O.dequant_bf16(q_ref, s_ref, bits)
    xd = dev_bf16(c["x"])
    for m in (4, 20, 80):
        _case(f"dequant_gemm M={m} N=32 K=2^20 bits={bits}")
        y_ref = O.gemm_ref(c["x"][:m], w16)
        check_product(host(gpu_lib.dequant_gemm(xd[:m], qw, torch.float32)), y_ref, False, f"M={m} f32")
        check_product(host(gpu_lib.dequant_gemm(xd[:m], qw, torch.bfloat16)), y_ref, True, f"M={m} bf16")


def test_gemm_input_past_4gib(gpu_lib):
    """X of 2176 x 2^20 bf16 (4.56 GB, large tiles): rows from 2048 on start
    past 4 GiB."""
    api = gpu_lib
    m, n, bits = 2176, 32, 5
    assert m * K_MAX * 2 > GIB4
    c = synth.random_case(41, 64, n, K_MAX)
    rows = np.array([0, 1, 63, 1000, 2047, 2048, 2049, 2100, 2111, 2112, 2150, 2175])
    own = synth.random_case(42, len(rows), 16, K_MAX)["x"]
    _case(f"dequant_gemm X past 4 GiB: M={m} N={n} K=2^20 bits={bits}")
    xd = dev_bf16(c["x"]).repeat(m // 64, 1)
    xd[torch.as_tensor(rows, device="cuda")] = dev_bf16(own)
    x_rows = _rows_to_host(xd, rows)
    assert np.array_equal(x_rows, own)
    qw = api.quantize_pack(dev_bf16(c["w"]), bits)
    w16 = _w16(c["w"], bits)
    y_ref = O.gemm_ref(x_rows, w16)
    for dt, bf in ((torch.float32, False), (torch.bfloat16, True)):
        y = api.dequant_gemm(xd, qw, dt)
        check_product(_rows_to_host(y, rows), y_ref, bf, f"X past 4 GiB {dt}")
        del y
    del xd
    torch.cuda.empty_cache()


def test_quantize_and_gemm_weight_past_4gib(gpu_lib):
    """W of 3,842,048 x 1280 at 7 bits: the packed weight is 4.30 GB and the
    bf16 input 9.8 GB.  The checked rows include the last ones, whose packed
    bytes start past 4 GiB; products at M = 4, 24 and 100 compare those
    columns."""
    api = gpu_lib
    k, bits, block = 1280, 7, 4096
    n = 938 * block
    row_bytes = k * bits // 8
    assert n * row_bytes > GIB4 and n % 16 == 0
    base = synth.random_case(51, 100, block, k)
    cols = np.unique(np.concatenate([[0, 1, 4095, 4096, 2_000_000],
                                     np.arange(GIB4 // row_bytes - 2, GIB4 // row_bytes + 3),
                                     np.arange(n - 40, n)]))
    own = synth.random_case(52, 0, len(cols), k)["w"]
    _case(f"quantize_pack W past 4 GiB: N={n} K={k} bits={bits}")
    wd = dev_bf16(base["w"]).repeat(n // block, 1)
    wd[torch.as_tensor(cols, device="cuda")] = dev_bf16(own)
    assert np.array_equal(_rows_to_host(wd, cols), own)
    qw = api.quantize_pack(wd, bits)
    del wd
    torch.cuda.empty_cache()
    p_ref, s_ref, q_ref = O.quantize_pack(own, bits)
    packed = qw.packed.view(n, row_bytes)
    got = _rows_to_host(packed, cols).astype(np.uint8)
    assert np.array_equal(got.reshape(-1), p_ref), "packed bytes differ"
    sc = _rows_to_host(qw.scales.view(n, k // 128), cols)
    assert np.array_equal(f32_bits(sc), f32_bits(s_ref.reshape(len(cols), -1))), "scales differ"
    w16 = O.dequant_bf16(q_ref, s_ref, bits)
    xd = dev_bf16(base["x"])
    colt = torch.as_tensor(cols, device="cuda")
    for m in (4, 24, 100):
        _case(f"dequant_gemm W past 4 GiB: M={m} N={n} K={k} bits={bits}")
        y_ref = O.gemm_ref(base["x"][:m], w16)
        y = api.dequant_gemm(xd[:m], qw, torch.bfloat16)
        check_product(y.index_select(1, colt).float().cpu().numpy(), y_ref, True, f"M={m}")
        del y
    del qw, packed
    torch.cuda.empty_cache()


def test_gemm_output_past_4gib(gpu_lib):
    """Y of 32800 x 65536 (bf16 4.30 GB, float32 8.6 GB; large tiles): the
    last rows are stored past 4 GiB."""
    api = gpu_lib
    m, n, k, bits = 32800, 65536, 128, 4
    assert m * n * 2 > GIB4
    c = synth.random_case(61, m, n, k)
    rows = np.unique(np.concatenate([[0, 1, 16383, 16384, 32767, 32768], np.arange(m - 40, m)]))
    _case(f"dequant_gemm Y past 4 GiB: M={m} N={n} K={k} bits={bits}")
    qw = api.quantize_pack(dev_bf16(c["w"]), bits)
    w16 = _w16(c["w"], bits)
    y_ref = O.gemm_ref(c["x"][rows], w16)
    xd = dev_bf16(c["x"])
    for dt, bf in ((torch.bfloat16, True), (torch.float32, False)):
        y = api.dequant_gemm(xd, qw, dt)
        check_product(_rows_to_host(y, rows), y_ref, bf, f"Y past 4 GiB {dt}")
        del y
        torch.cuda.empty_cache()


def _w4a8_check(y, xc, xs, wc, ws, out_bf16, what):
    from oracle import fp4 as F
    ref = F.w4a8_ref(xc, xs, wc, ws, "e2m1")
    if not out_bf16:
        absref = F.w4a8_ref(xc & 0x7F, xs, wc & 7, ws, "e2m1")     # the same sum over magnitudes
        assert np.all(np.abs(y - ref) <= 2.0 ** -14 * absref + 1e-37), what
    check_product(y, ref, out_bf16, what)


def test_w4a8_chain_activation_codes_past_4gib(gpu_lib):
    """E4M3 codes of X (1,048,832 x 4096, 4.30 GB; bf16 input 8.6 GB) from the
    row quantizer, then the tiled FP4 product: the last rows' codes start past
    4 GiB.  Codes and scales of the checked rows bit for bit, then the
    product's rows."""
    from oracle import fp4 as F
    api = gpu_lib
    k, n, block = 4096, 64, 256
    m = 4097 * block
    assert m * k > GIB4
    base = synth.random_case(71, block, n, k)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 500_000], np.arange(GIB4 // k - 2, GIB4 // k + 3),
                                     np.arange(m - 40, m)]))
    own = synth.random_case(72, len(rows), 16, k)["x"]
    _case(f"fp8_quantize_rows + w4a8_gemm X codes past 4 GiB: M={m} N={n} K={k}")
    xd = dev_bf16(base["x"]).repeat(m // block, 1)
    rt = torch.as_tensor(rows, device="cuda")
    xd[rt] = dev_bf16(own)
    xq, xs = api.fp8_quantize_rows(xd)
    del xd
    torch.cuda.empty_cache()
    xc, xsc = F.quantize_rows_e4m3(own)
    assert np.array_equal(_rows_to_host(xq, rows).astype(np.uint8), xc), "E4M3 codes differ"
    assert np.array_equal(f32_bits(xs.index_select(0, rt).cpu().numpy()), f32_bits(xsc)), "row scales differ"
    qw = api.fp4_quantize_pack(dev_bf16(base["w"]), "e2m1", tiled=True)
    wc, ws = F.quantize_fp4_groups(base["w"], "e2m1")
    for dt, bf in ((torch.float32, False), (torch.bfloat16, True)):
        y = api.w4a8_gemm(xq, xs, qw, dt)
        _w4a8_check(_rows_to_host(y, rows).astype(np.float64), xc, xsc, wc, ws, bf, f"w4a8 X past 4 GiB {dt}")
        del y
    del xq, xs
    torch.cuda.empty_cache()


def test_w4a8_output_past_4gib(gpu_lib):
    """The tiled FP4 x E4M3 product into a 32800 x 65536 bf16 output
    (4.30 GB): the last rows are stored past 4 GiB."""
    from oracle import fp4 as F
    api = gpu_lib
    m, n, k = 32800, 65536, 128
    assert m * n * 2 > GIB4
    c = synth.random_case(81, m, n, k)
    rows = np.unique(np.concatenate([[0, 1, 16383, 16384, 32767, 32768], np.arange(m - 40, m)]))
    _case(f"w4a8_gemm Y past 4 GiB: M={m} N={n} K={k}")
    qw = api.fp4_quantize_pack(dev_bf16(c["w"]), "e2m1", tiled=True)
    xq, xs = api.fp8_quantize_rows(dev_bf16(c["x"]))
    wc, ws = F.quantize_fp4_groups(c["w"], "e2m1")
    xc, xsc = F.quantize_rows_e4m3(c["x"][rows])
    y = api.w4a8_gemm(xq, xs, qw, torch.bfloat16)
    _w4a8_check(_rows_to_host(y, rows).astype(np.float64), xc, xsc, wc, ws, True, "w4a8 Y past 4 GiB")
    del y
    torch.cuda.empty_cache()


def test_lowrank_output_past_4gib(gpu_lib):
    """The fused low-rank product (r = 32) into a 32800 x 65536 bf16 output
    (4.30 GB): the last rows, with their T . L2 term, are stored past 4 GiB."""
    api = gpu_lib
    m, n, k, r, bits = 32800, 65536, 128, 32, 4
    assert m * n * 2 > GIB4
    c = synth.random_case(91, m, n, k, wstd=0.05)
    rows = np.unique(np.concatenate([[0, 1, 16383, 16384, 32767, 32768], np.arange(m - 40, m)]))
    _case(f"lowrank_fused_gemm Y past 4 GiB: M={m} N={n} K={k} r={r} bits={bits}")
    l1, l2, res = O.svd_split(c["w"], r)
    qr = api.quantize_pack(torch.from_numpy(np.ascontiguousarray(res, dtype=np.float32)).cuda(), bits)
    y_ref, _ = O.lowrank_fused_ref(c["x"][rows], _w16(res, bits), l1, l2)
    ld = dev_bf16(np.ascontiguousarray(l1.T))
    lu = dev_bf16(np.ascontiguousarray(l2.T))
    y = api.lowrank_fused_gemm(dev_bf16(c["x"]), qr, ld, lu, torch.bfloat16)
    check_product(_rows_to_host(y, rows), y_ref, True, "lowrank Y past 4 GiB")
    del y
    torch.cuda.empty_cache()


def test_grouped_past_4gib(gpu_lib):
    """One grouped call: a 32800 x 65536 product (bf16 output past 4 GiB, large
    tiles) beside a 16-token and a 40-token product on a packed weight of
    3,842,048 x 1280 at 7 bits (4.30 GB).  Each is checked on its own rows or
    columns."""
    api = gpu_lib
    big = synth.random_case(101, 32800, 65536, 128)
    rows = np.unique(np.concatenate([[0, 16384, 32767, 32768], np.arange(32800 - 24, 32800)]))
    k, bits, block = 1280, 7, 4096
    n = 938 * block
    row_bytes = k * bits // 8
    base = synth.random_case(102, 40, block, k)
    cols = np.unique(np.concatenate([[0, 4096], np.arange(GIB4 // row_bytes - 1, GIB4 // row_bytes + 2),
                                     np.arange(n - 20, n)]))
    own = synth.random_case(103, 0, len(cols), k)["w"]
    _case(f"grouped: 32800 x 65536 x 128 (4 bits) + 16/40 x {n} x {k} (7 bits)")
    qb = api.quantize_pack(dev_bf16(big["w"]), 4)
    wd = dev_bf16(base["w"]).repeat(n // block, 1)
    colt = torch.as_tensor(cols, device="cuda")
    wd[colt] = dev_bf16(own)
    qw = api.quantize_pack(wd, bits)
    del wd
    torch.cuda.empty_cache()
    xb, xs = dev_bf16(big["x"]), dev_bf16(base["x"])
    yb, y16, y40 = api.dequant_gemm_grouped([(xb, qb), (xs[:16], qw), (xs, qw)], torch.bfloat16)
    check_product(_rows_to_host(yb, rows), O.gemm_ref(big["x"][rows], _w16(big["w"], 4)), True, "grouped big")
    w16 = _w16(own, bits)
    for y, m in ((y16, 16), (y40, 40)):
        check_product(y.index_select(1, colt).float().cpu().numpy(), O.gemm_ref(base["x"][:m], w16), True,
                      f"grouped M={m}")
    del yb, y16, y40, qw
    torch.cuda.empty_cache()


def test_w4a6_chain_activation_codes_past_4gib(gpu_lib):
    """E2M3 codes of X (1,398,272 x 4096, 4.30 GB in the tiled 32-row records;
    bf16 input 11.5 GB), then the W4A6 product.  Whole 32-row blocks are
    checked (the first, the two around the 4 GiB byte, the last): their
    records bit for bit, then the product's rows."""
    from oracle import fp4 as F
    api = gpu_lib
    k, n, block = 4096, 64, 256
    m = 5462 * block
    blk_bytes = 32 * k * 3 // 4                      # one 32-row record block
    assert m * k * 3 // 4 > GIB4 and blk_bytes == (k // 128) * 3072
    blocks = np.array([0, GIB4 // blk_bytes, GIB4 // blk_bytes + 1, m // 32 - 1])
    rows = (blocks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    base = synth.random_case(111, block, n, k)
    own = synth.random_case(112, len(rows), 16, k)["x"]
    _case(f"fp6_quantize_rows + w4a6_gemm X codes past 4 GiB: M={m} N={n} K={k}")
    xd = dev_bf16(base["x"]).repeat(m // block, 1)
    rt = torch.as_tensor(rows, device="cuda")
    xd[rt] = dev_bf16(own)
    xq, xs = api.fp6_quantize_rows(xd, "e2m3")
    del xd
    torch.cuda.empty_cache()
    xc, xsc = F.quantize_rows_fp6(own, "e2m3")
    for i, b in enumerate(blocks):
        got = xq[int(b) * blk_bytes:(int(b) + 1) * blk_bytes].cpu().numpy()
        assert np.array_equal(got, F.pack_fp6_tiled(xc[32 * i:32 * (i + 1)])), f"records of block {b} differ"
    assert np.array_equal(f32_bits(xs.index_select(0, rt).cpu().numpy()), f32_bits(xsc)), "row scales differ"
    qw = api.fp4_quantize_pack(dev_bf16(base["w"]), "e2m1", tiled=True)
    wc, ws = F.quantize_fp4_groups(base["w"], "e2m1")
    ref = F.w4a6_ref(xc, xsc, wc, ws, "e2m1", "e2m3")
    y = api.w4a6_gemm(xq, xs, "e2m3", qw, torch.float32)
    yr = _rows_to_host(y, rows).astype(np.float64)
    absref = F.w4a6_ref(xc & 31, xsc, wc & 7, ws, "e2m1", "e2m3")
    assert np.all(np.abs(yr - ref) <= 2.0 ** -14 * absref + 1e-37)
    check_product(yr, ref, False, "w4a6 X past 4 GiB")
    del y, xq, xs
    torch.cuda.empty_cache()


def test_rotate_past_4gib(gpu_lib):
    """The rotation pre-pass on 699,136 x 3072 bf16 rows (4.30 GB in; float32
    out, 8.6 GB): rows from 699,051 on start past 4 GiB in the input.  Checked
    rows within the float32 butterfly bound of the float64 oracle."""
    import math
    api = gpu_lib
    d, h, block = 3072, 128, 256
    n = 2731 * block
    assert n * d * 2 > GIB4
    base = synth.random_case(121, block, 16, d)["x"]
    rows = np.unique(np.concatenate([[0, 1, 255, 256], np.arange(GIB4 // (2 * d) - 2, GIB4 // (2 * d) + 3),
                                     np.arange(n - 40, n)]))
    own = synth.random_case(122, len(rows), 16, d)["x"]
    perm, signs = synth.rpbh_draw(d, 12)
    _case(f"rpbh_rotate past 4 GiB: n={n} d={d} h={h}")
    xd = dev_bf16(base).repeat(n // block, 1)
    rt = torch.as_tensor(rows, device="cuda")
    xd[rt] = dev_bf16(own)
    y = api.rpbh_rotate(xd, torch.from_numpy(perm).cuda(), torch.from_numpy(signs).cuda(), h, torch.float32)
    got = _rows_to_host(y, rows).astype(np.float64)
    del y, xd
    torch.cuda.empty_cache()
    import oracle.rpbh_oracle as R
    ref = R.rpbh_rotate(own, perm, signs, h)
    t = np.abs(np.asarray(own, dtype=np.float64)[:, perm])
    blk = t.reshape(len(rows), d // h, h).sum(axis=2, keepdims=True)
    bound = np.broadcast_to((math.log2(h) + 1) * 2.0 ** -24 * blk / math.sqrt(h),
                            (len(rows), d // h, h)).reshape(len(rows), d) * 1.01 + 1e-37
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) / bound))


def _wide_k_max_weight(n, bits, cols):
    """An n x 2^20 weight on the GPU: a seeded 32-row block repeated, with
    seeded rows of their own at `cols`.  Returns (device bf16, own rows)."""
    base = synth.random_case(61 + bits, 0, 32, K_MAX)["w"]
    own = synth.random_case(62 + bits, 0, len(cols), K_MAX)["w"]
    wd = dev_bf16(base).repeat(n // 32, 1)
    wd[torch.as_tensor(cols, device="cuda")] = dev_bf16(own)
    return wd, own


@pytest.mark.parametrize("bits", (3, 6))
def test_weight_streaming_and_grouped_at_k_max(gpu_lib, bits):
    """K = 2^20 through the weight-streaming kernel (M = 16 and 5 with
    N = 12800: 200 workgroups of 64 columns) and through one grouped call that
    holds that product beside a 20-token and an 80-token one on a 32-column
    weight (the grouped kernels of each class)."""
    api = gpu_lib
    n = 12800
    cols = np.array([0, 1, 63, 64, 6399, 6400, 12735, 12736, 12798, 12799])
    _case(f"quantize_pack {n} x 2^20 bits={bits} (repeated block, own rows at the checked columns)")
    wd, own = _wide_k_max_weight(n, bits, cols)
    qw = api.quantize_pack(wd, bits)
    del wd
    torch.cuda.empty_cache()
    p_ref, s_ref, q_ref = O.quantize_pack(own, bits)
    colt = torch.as_tensor(cols, device="cuda")
    got = qw.packed.view(n, -1).index_select(0, colt).cpu().numpy()
    assert np.array_equal(got.reshape(-1), p_ref), "packed bytes differ"
    w16 = O.dequant_bf16(q_ref, s_ref, bits)
    xs = synth.random_case(63 + bits, 80, 32, K_MAX)
    xd = dev_bf16(xs["x"])
    for m in (16, 5):
        _case(f"dequant_gemm weight streaming M={m} N={n} K=2^20 bits={bits}")
        y = api.dequant_gemm(xd[:m], qw, torch.float32)
        check_product(y.index_select(1, colt).cpu().numpy(), O.gemm_ref(xs["x"][:m], w16), False, f"M={m}")
        del y
    _case(f"dequant_gemm_grouped at K=2^20 bits={bits}: M=16 x N={n}, M=20 and M=80 x N=32")
    qs = api.quantize_pack(dev_bf16(xs["w"]), bits)
    ws16 = _w16(xs["w"], bits)
    outs = api.dequant_gemm_grouped([(xd[:16], qw), (xd[:20], qs), (xd[:80], qs)], out_dtype=torch.float32)
    check_product(outs[0].index_select(1, colt).cpu().numpy(), O.gemm_ref(xs["x"][:16], w16), False, "grouped M=16")
    check_product(outs[1].cpu().numpy(), O.gemm_ref(xs["x"][:20], ws16), False, "grouped M=20")
    check_product(outs[2].cpu().numpy(), O.gemm_ref(xs["x"][:80], ws16), False, "grouped M=80")
    del outs, qw
    torch.cuda.empty_cache()


def test_lowrank_at_k_max(gpu_lib):
    """The low-rank pre-pass and the fused product at K = 2^20, r = 32, for
    M = 16 (small-M kernel) and 80 (large tiles)."""
    api = gpu_lib
    c = synth.random_case(71, 80, 64, K_MAX, wstd=0.05)
    _case("lowrank_fused_gemm K=2^20 r=32 (SVD split of a 64 x 2^20 weight)")
    l1, l2, res = O.svd_split(c["w"], 32)
    qr = api.quantize_pack(dev_f32(res), 4)
    ld = dev_bf16(np.ascontiguousarray(l1.T))
    lu = dev_bf16(np.ascontiguousarray(l2.T))
    w16 = _w16(res, 4)
    xd = dev_bf16(c["x"])
    for m in (16, 80):
        _case(f"lowrank_fused_gemm M={m} N=64 K=2^20 r=32")
        y_ref, _ = O.lowrank_fused_ref(c["x"][:m], w16, l1, l2)
        check_product(host(api.lowrank_fused_gemm(xd[:m], qr, ld, lu, torch.float32)), y_ref, False, f"M={m}")


def test_w4a8_tiled_at_k_max(gpu_lib):
    """The E4M3 row quantizer, the tiled E2M1 quantizer and their product at
    K = 2^20 (M = 20, N = 48)."""
    from oracle import fp4 as F
    api = gpu_lib
    rng = np.random.default_rng(81)
    w = synth.to_bf16(rng.standard_t(4, size=(48, K_MAX)) * 0.02)
    x = synth.to_bf16(rng.normal(0, 1, size=(20, K_MAX)))
    _case("fp8_quantize_rows + fp4_quantize_pack (tiled) + w4a8_gemm at K=2^20")
    xq, xs = api.fp8_quantize_rows(dev_bf16(x))
    cq, cs = F.quantize_rows_e4m3(x)
    assert np.array_equal(host(xq), cq) and np.array_equal(f32_bits(host(xs)), f32_bits(cs))
    qw = api.fp4_quantize_pack(dev_bf16(w), "e2m1", tiled=True)
    wc, wsc = F.quantize_fp4_groups(w, "e2m1")
    tp, ts = F.tile_fp4(F.pack_fp4(wc), wsc)
    assert np.array_equal(host(qw.packed), tp)
    y = host(api.w4a8_gemm(xq, xs, qw, torch.float32))
    check_product(y, F.w4a8_ref(cq, cs, wc, wsc, "e2m1"), False, "w4a8 K=2^20")
