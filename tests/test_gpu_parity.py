"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: packed bytes, scales, dense dequantized bf16 weights.
Tolerance (products): relative Frobenius <= 1e-3 and per-row max-abs
<= 2e-2 * max|row| of the oracle on the same dequantized weights.
Full-size workloads compare sampled rows that the oracle computes one by one
(first rows, random rows, the ragged last rows); small shapes compare every
element.
"""
import functools

import numpy as np
import pytest
import torch

import oracle as O
from dit_dequant_gemm_amd import synth
from parity_util import (check_product, dev_bf16, dev_f32, f32_bits, host, sample_rows,
                         sample_weight_rows)

pytestmark = pytest.mark.gpu
BITS = (3, 4, 5, 6, 7)


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _quant_exact(api, w, bits, rows=None, f32_input=False):
    """GPU quantize_pack of the whole tensor; oracle on `rows` (all if None)."""
    wt = dev_f32(w) if f32_input else dev_bf16(w)
    qw = api.quantize_pack(wt, bits)
    n, k = w.shape
    packed = host(qw.packed).reshape(n, k * bits // 8)
    scales = host(qw.scales)
    rows = np.arange(n) if rows is None else rows
    p_ref, s_ref, q_ref = O.quantize_pack(w[rows], bits)
    assert np.array_equal(packed[rows].reshape(-1), p_ref), "packed bytes differ"
    assert np.array_equal(f32_bits(scales[rows]), f32_bits(s_ref)), "scales differ"
    return qw, q_ref, s_ref


# ------------------------------------------------------------------ quantize + pack
@pytest.mark.parametrize("bits", BITS)
def test_quantize_pack_small_edge_cases(gpu_lib, bits):
    _case(f"quantize_pack edge cases bits={bits}")
    rng = np.random.default_rng(bits)
    w = rng.normal(0, 0.02, (24, 384)).astype(np.float32)
    w[1, :128] = 0.0                                   # all-zero group
    w[2, 128:256] = rng.normal(0, 1e-39, 128)          # subnormal group (f32 input)
    w[3, :] = rng.standard_t(2, 384) * 3.0             # heavy tails
    w[4, 5] = 100.0                                    # single outlier
    w[5, :] = np.round(rng.normal(0, 3, 384))          # many exact ties
    w[6, 256:] = -w[6, 256:]
    w[7, :128] = 1e30
    wb = synth.to_bf16(w)
    _quant_exact(gpu_lib, wb, bits)                    # bf16 input
    _quant_exact(gpu_lib, w, bits, f32_input=True)     # float32 input


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("n,k", [(1, 128), (3, 256), (17, 1152), (64, 512)])
def test_quantize_pack_random_shapes(gpu_lib, bits, n, k):
    _case(f"quantize_pack n={n} k={k} bits={bits}")
    w = synth.random_case(n * 1000 + k + bits, 1, n, k)["w"]
    _quant_exact(gpu_lib, w, bits)


def test_quantize_pack_config1(gpu_lib):
    _case("quantize_pack workload 1")
    c = synth.config1()
    _quant_exact(gpu_lib, c["w"], c["bits"])


def test_quantize_pack_config2_full(gpu_lib):
    _case("quantize_pack workload 2 (3072x3072, every row)")
    c = synth.config2(m=1)
    _quant_exact(gpu_lib, c["w"], 4)


@pytest.mark.parametrize("which", ["up", "down"])
@pytest.mark.parametrize("bits", (3, 5, 6, 7))
def test_quantize_pack_config3(gpu_lib, which, bits):
    _case(f"quantize_pack workload 3 {which} bits={bits}")
    c = synth.config3(which, m=1)
    rows = sample_weight_rows(c["w"].shape[0], bits)
    _quant_exact(gpu_lib, c["w"], bits, rows)


@pytest.mark.parametrize("name", ["qkv", "o", "up", "down"])
def test_quantize_pack_config5_all_bits(gpu_lib, name):
    w = synth.config5_weights(name)
    for bits in BITS:
        _case(f"quantize_pack workload 5 {name} bits={bits}")
        _quant_exact(gpu_lib, w, bits, sample_weight_rows(w.shape[0], bits))


# ------------------------------------------------------------------ dense dequantize
@pytest.mark.parametrize("bits", BITS)
def test_dequantize_bit_exact(gpu_lib, bits):
    _case(f"dequantize bits={bits}")
    w = synth.random_case(7 + bits, 1, 48, 640, wstd=0.05)["w"]
    qw = gpu_lib.quantize_pack(dev_bf16(w), bits)
    d = host(gpu_lib.dequantize(qw))
    q_u, s = O.quantize_groups(w, bits)
    assert np.array_equal(f32_bits(d), f32_bits(O.dequant_bf16(q_u, s, bits)))


# ------------------------------------------------------------------ products
def _oracle_w16(w, bits):
    q_u, s = O.quantize_groups(w, bits)
    return O.dequant_bf16(q_u, s, bits)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("m", [1, 15, 16, 17, 33, 64, 65, 130, 257])
def test_gemm_ragged_shapes(gpu_lib, bits, m):
    for n, k in ((16, 128), (48, 384), (272, 256)):
        _case(f"dequant_gemm m={m} n={n} k={k} bits={bits}")
        c = synth.random_case(m * 7 + n + k + bits, m, n, k)
        qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
        y_ref = O.gemm_ref(c["x"], _oracle_w16(c["w"], bits))
        xd = dev_bf16(c["x"])
        check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.float32)), y_ref, False, "f32")
        check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.bfloat16)), y_ref, True, "bf16")


# M <= 16 with a wide output (N >= 12800) runs the weight-streaming kernel:
# K from one group (7 of 8 K-split waves idle) to 108 groups (several chunks
# per wave, a short last chunk), N with a partial last workgroup, M < 16.
# (the 108-group case runs at the narrowest and widest code only)
@pytest.mark.parametrize("bits,m,n,k", [(b, m, n, k) for (m, n, k) in [(16, 12800, 128), (1, 12816, 640),
                                                                       (7, 12816, 3328), (16, 12864, 5120)]
                                        for b in BITS] + [(3, 16, 12816, 13824), (7, 16, 12816, 13824)])
def test_gemm_wide_small_m(gpu_lib, bits, m, n, k):
    _case(f"dequant_gemm wide small-M m={m} n={n} k={k} bits={bits}")
    c = synth.random_case(m * 131 + n + k + bits, m, n, k)
    qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
    y_ref = O.gemm_ref(c["x"], _oracle_w16(c["w"], bits))
    xd = dev_bf16(c["x"])
    check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.float32)), y_ref, False, "f32")
    check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.bfloat16)), y_ref, True, "bf16")


# The small-M kernel's launch shapes (column waves x K-split waves): (1, 8) at
# M <= 16 and (1, 4) above for narrow outputs, (2, 2) from 4096 columns.  Each
# K is chosen so that the K ranges end part-way through the ring of X slots:
# 2560 (20 groups: 3 steps with an 8-way split, 5 with a 4-way one, ring of
# 2), 1280 (10 groups: 5 steps, ring of 3) and 512 (4 groups: 2 steps, shorter
# than the ring, so only the prologue issues loads).  Ragged M included.
_SMALL_SHAPES = [(3072, 2560), (5120, 1280), (4096, 512)]


@functools.lru_cache(maxsize=None)
def _small_shape_case(n, k, bits):
    c = synth.random_case(n + k + bits, 64, n, k)
    return c["x"], c["w"], _oracle_w16(c["w"], bits)


@pytest.mark.parametrize("bits", (3, 4, 7))
@pytest.mark.parametrize("n,k", _SMALL_SHAPES)
@pytest.mark.parametrize("m", [16, 23, 32, 50, 64])
def test_gemm_small_m_launch_shapes(gpu_lib, m, n, k, bits):
    _case(f"dequant_gemm small-M launch shape m={m} n={n} k={k} bits={bits}")
    x, w, w16 = _small_shape_case(n, k, bits)
    qw = gpu_lib.quantize_pack(dev_bf16(w), bits)
    xd = dev_bf16(np.ascontiguousarray(x[:m]))
    y_ref = O.gemm_ref(x[:m], w16)
    check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.float32)), y_ref, False, "f32")
    check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.bfloat16)), y_ref, True, "bf16")


# Grouped products: mixed widths, shapes and output dtypes in one call.  Each
# output is checked against the oracle on its own weight.
_GROUP_CASES = [
    # (m, n, k, bits, out dtype)
    (16, 5120, 640, 5, torch.bfloat16),
    (16, 272, 640, 6, torch.float32),       # a partial last workgroup
    (7, 1024, 3328, 4, torch.bfloat16),     # 26 groups: short chunks
    (1, 64, 128, 3, torch.float32),         # one group: 7 of 8 K-split waves idle
    (16, 512, 13824, 7, torch.bfloat16),    # 108 groups: several chunks per wave
    (48, 256, 384, 5, torch.float32),       # M > 16: its own launch
]


def _run_group(api, cases, seed):
    items, refs = [], []
    for i, (m, n, k, bits, dt) in enumerate(cases):
        c = synth.random_case(seed * 97 + i, m, n, k)
        qw = api.quantize_pack(dev_bf16(c["w"]), bits)
        items.append((dev_bf16(c["x"]), qw, torch.empty((m, n), dtype=dt, device="cuda")))
        refs.append((O.gemm_ref(c["x"], _oracle_w16(c["w"], bits)), dt))
    outs = api.dequant_gemm_grouped(items)
    for (m, n, k, bits, dt), y, (ref, _) in zip(cases, outs, refs):
        check_product(host(y), ref, dt == torch.bfloat16, f"grouped m={m} n={n} k={k} bits={bits}")


def test_gemm_grouped_mixed(gpu_lib):
    _case("dequant_gemm_grouped mixed widths and shapes")
    _run_group(gpu_lib, _GROUP_CASES, 1)


def test_gemm_grouped_more_than_one_launch(gpu_lib):
    _case("dequant_gemm_grouped 19 small products (two launches)")
    cases = [(1 + (i % 16), 64 * (1 + i % 5), 128 * (1 + i % 7), 3 + i % 5,
              torch.float32 if i % 2 else torch.bfloat16) for i in range(19)]
    _run_group(gpu_lib, cases, 2)


# Products with M > 64 share launches of the large-M kernel's tiles: mixed
# widths, one and several tiles, ragged M and N, K from one to ten groups,
# beside small products of the same call.
_GROUP_LARGE_CASES = [
    (65, 192, 128, 3, torch.float32),        # one tile, one group
    (300, 528, 384, 4, torch.bfloat16),      # 2 x 3 tiles, ragged M and N
    (257, 256, 1280, 5, torch.float32),      # ten groups, a 1-row last row tile
    (130, 1024, 640, 6, torch.bfloat16),
    (96, 304, 896, 7, torch.float32),
    (16, 272, 640, 6, torch.float32),        # a small product in the same call
]


# Products with 16 < M <= 32 and 32 < M <= 64 share launches of the small-M
# kernel's body (two column waves, a two-way K split): mixed widths, ragged
# N (a half-filled last workgroup), one group to 108 groups of K (ring tails).
_GROUP_MID_CASES = [
    (17, 5120, 1280, 4, torch.bfloat16),
    (32, 272, 384, 6, torch.float32),        # N = 8.5 workgroups of 32 columns
    (24, 1024, 13824, 3, torch.bfloat16),    # 108 groups
    (33, 3072, 128, 7, torch.float32),       # one group: one K half idle
    (64, 528, 2560, 5, torch.bfloat16),
    (50, 4096, 512, 4, torch.float32),
    (16, 272, 640, 6, torch.float32),        # a 16-token product in the same call
    (80, 192, 384, 3, torch.float32),        # and a large-M one
]


def test_gemm_grouped_mid(gpu_lib):
    _case("dequant_gemm_grouped products with 16 < M <= 64 (grouped small-M body)")
    _run_group(gpu_lib, _GROUP_MID_CASES, 5)


def test_gemm_grouped_mid_more_than_one_launch(gpu_lib):
    _case("dequant_gemm_grouped 18 products with 16 < M <= 32 (two launches)")
    cases = [(17 + (i % 16), 64 * (1 + i % 5), 128 * (1 + i % 7), 3 + i % 5,
              torch.float32 if i % 2 else torch.bfloat16) for i in range(18)]
    _run_group(gpu_lib, cases, 6)


def test_gemm_grouped_large(gpu_lib):
    _case("dequant_gemm_grouped products with M > 64 (grouped large tiles)")
    _run_group(gpu_lib, _GROUP_LARGE_CASES, 3)


def test_gemm_grouped_large_more_than_one_launch(gpu_lib):
    _case("dequant_gemm_grouped 18 products with M > 64 (two launches)")
    cases = [(65 + 37 * (i % 4), 64 * (1 + i % 5), 128 * (1 + i % 3), 3 + i % 5,
              torch.float32 if i % 2 else torch.bfloat16) for i in range(18)]
    _run_group(gpu_lib, cases, 4)


@pytest.mark.parametrize("m,n,k,exact", [(3800, 4112, 256, True), (300, 528, 1280, False)])
def test_gemm_grouped_large_equals_single_calls(gpu_lib, m, n, k, exact):
    """The grouped launch runs 256 x 256 tiles.  A single call of 3800 x 4112
    (255 such tiles) takes the same tiles and must match bit for bit; one of
    300 x 528 takes 256 x 192 tiles (another float32 summation order)."""
    _case(f"dequant_gemm_grouped M > 64 against separate dequant_gemm calls m={m} n={n} k={k} exact={exact}")
    c = synth.random_case(6, m, n, k)
    outs_single, items = [], []
    for bits in (3, 4, 7):
        qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
        x = dev_bf16(c["x"])
        outs_single.append(host(gpu_lib.dequant_gemm(x, qw, torch.float32)))
        items.append((x, qw))
    outs = gpu_lib.dequant_gemm_grouped(items, out_dtype=torch.float32)
    for a, b in zip(outs, outs_single):
        if exact:
            assert np.array_equal(host(a), b), "grouped large tiles differ from the single call"
        else:
            assert np.max(np.abs(host(a) - b)) <= 1e-5 * np.max(np.abs(b)) + 1e-6


def test_gemm_grouped_matches_single_calls(gpu_lib):
    _case("dequant_gemm_grouped against separate dequant_gemm calls")
    c = synth.random_case(5, 16, 1024, 1280)
    outs_single, items = [], []
    for bits in (4, 5, 6):
        qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
        x = dev_bf16(c["x"])
        outs_single.append(host(gpu_lib.dequant_gemm(x, qw, torch.float32)))
        items.append((x, qw))
    outs = gpu_lib.dequant_gemm_grouped(items, out_dtype=torch.float32)
    for a, b in zip(outs, outs_single):
        check_product(host(a), b.astype(np.float64), False, "grouped vs single")


# The grouped 16-token launch takes 4, 2 or 1 column blocks of 16 per
# workgroup, whichever has the least estimated time: the larger of the
# costliest workgroup and the total cost per compute unit, a workgroup costing
# its packed and scale bytes plus half its X bytes.  _grouped_ncb restates that
# choice so that each set below is known to run the form it is meant to cover
# (mixed widths and dtypes, ragged N: partial last workgroups).
_GROUP_NCB_CASES = {
    1: [(16, 1952, 384, 4, torch.bfloat16), (5, 1040, 256, 6, torch.float32),
        (16, 272, 640, 3, torch.bfloat16), (1, 64, 128, 7, torch.float32)],
    2: [(16, 4112, 256, 5, torch.float32), (16, 3088, 128, 4, torch.bfloat16),
        (7, 2064, 256, 6, torch.float32), (16, 1008, 384, 3, torch.bfloat16)],
    4: [(16, 12304, 128, 4, torch.bfloat16), (11, 8208, 128, 5, torch.float32),
        (16, 4096, 256, 3, torch.bfloat16), (2, 1040, 128, 7, torch.float32)],
}


def _grouped_ncb(cases, cus):
    est = {}
    for ncb in (4, 2, 1):
        worst = total = 0.0
        for _m, n, k, bits, _dt in cases:
            wg = 16.0 * ncb * k * (bits / 8.0 + 4.0 / 128) + 0.5 * 32.0 * k
            worst = max(worst, wg)
            total += -(-n // (16 * ncb)) * wg
        est[ncb] = max(worst, total / cus)
    best = 4
    for ncb in (2, 1):
        if est[ncb] < est[best]:
            best = ncb
    return best


@pytest.mark.parametrize("ncb", sorted(_GROUP_NCB_CASES))
def test_gemm_grouped_column_blocks(gpu_lib, ncb):
    _case(f"dequant_gemm_grouped 16-token launch with {ncb} column blocks per workgroup")
    cases = _GROUP_NCB_CASES[ncb]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert _grouped_ncb(cases, cus) == ncb, "the set no longer selects the form it covers"
    _run_group(gpu_lib, cases, 11 + ncb)


def test_gemm_empty_batch_leaves_output(gpu_lib):
    _case("dequant_gemm m=0")
    c = synth.random_case(1, 4, 32, 128)
    qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), 4)
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    y = gpu_lib.dequant_gemm(x, qw, torch.float32)
    assert y.shape == (0, 32)


def test_gemm_config1(gpu_lib):
    _case("dequant_gemm workload 1 (M=64)")
    c = synth.config1()
    qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), 4)
    y_ref = O.gemm_ref(c["x"], _oracle_w16(c["w"], 4))
    xd = dev_bf16(c["x"])
    check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.float32)), y_ref, False)
    check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.bfloat16)), y_ref, True)


@pytest.mark.parametrize("m", [16, 4096])
def test_gemm_config2(gpu_lib, m):
    _case(f"dequant_gemm workload 2 M={m}")
    c = synth.config2(m=m)
    qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), 4)
    w16 = _oracle_w16(c["w"], 4)
    rows = sample_rows(m, 2) if m > 64 else np.arange(m)
    y_ref = O.gemm_ref(c["x"][rows], w16)
    xd = dev_bf16(c["x"])
    check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.float32))[rows], y_ref, False)
    check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.bfloat16))[rows], y_ref, True)


@pytest.mark.parametrize("which", ["up", "down"])
def test_gemm_config3(gpu_lib, which):
    c = synth.config3(which)
    xd = dev_bf16(c["x"])
    rows = sample_rows(4096, 3, count=64)
    for bits in c["bits_sweep"]:
        _case(f"dequant_gemm workload 3 {which} bits={bits}")
        qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
        y_ref = O.gemm_ref(c["x"][rows], _oracle_w16(c["w"], bits))
        check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.bfloat16))[rows], y_ref, True)
        check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.float32))[rows], y_ref, False)


@pytest.mark.parametrize("name", ["qkv", "o", "up", "down"])
def test_gemm_config5(gpu_lib, name):
    w = synth.config5_weights(name)
    x16 = synth.config5_x(name, 16)
    xd16 = dev_bf16(x16)
    wd = dev_bf16(w)
    for bits in BITS:                      # every width at M = 16
        _case(f"dequant_gemm workload 5 {name} M=16 bits={bits}")
        qw = gpu_lib.quantize_pack(wd, bits)
        w16 = _oracle_w16(w, bits)
        check_product(host(gpu_lib.dequant_gemm(xd16, qw, torch.bfloat16)), O.gemm_ref(x16, w16), True)


@functools.lru_cache(maxsize=1)
def _c5_large(name):
    """Workload 5 weight and its 32760-token X (one tensor held at a time)."""
    return synth.config5_weights(name), synth.config5_x(name, 32760)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("name", ["qkv", "o", "up", "down"])
def test_gemm_config5_m32760(gpu_lib, name, bits):
    """Every width at 32760 tokens (127 full 256-row tiles and a 248-row
    tail): the first rows, random rows and the whole ragged tail."""
    _case(f"dequant_gemm workload 5 {name} M=32760 bits={bits}")
    w, x = _c5_large(name)
    qw = gpu_lib.quantize_pack(dev_bf16(w), bits)
    rows = sample_rows(32760, 5 + bits, count=48, tail=248)
    y = gpu_lib.dequant_gemm(dev_bf16(x), qw, torch.bfloat16)
    ys = y.index_select(0, torch.as_tensor(rows, device="cuda")).float().cpu().numpy()
    del y
    check_product(ys, O.gemm_ref(x[rows], _oracle_w16(w, bits)), True)


# ------------------------------------------------------------------ stream-K (large M, few tiles)
@pytest.mark.parametrize("m,n,k,bits", [
    (1041, 528, 1536, 3), (2065, 272, 6144, 5), (300, 4096, 3072, 7), (1024, 5120, 5120, 4),   # split-K 2, 8, 4, 3
    (4160, 4080, 1280, 6), (4352, 3856, 2560, 4),                                               # stream-K
    (4096, 5120, 5120, 4), (4160, 5136, 1280, 6), (4096, 3072, 3072, 4), (2065, 272, 384, 5),   # 256 x 192 tiles
    (3800, 4112, 256, 3)])                                                                      # 256 x 256 tiles
def test_gemm_streamk(gpu_lib, m, n, k, bits):
    """Products whose 256 x 256 tiles fill the compute units unevenly split K
    across workgroups when given a workspace (split-K for few tiles, stream-K
    for some more; others take whole tiles of 256 x 192 or 256 x 256):
    against the oracle, equal to themselves on a second call (the partial sums
    are added in a fixed order), and against the same product without a
    workspace (whole tiles) within float32 summation order."""
    _case(f"dequant_gemm stream-K m={m} n={n} k={k} bits={bits}")
    c = synth.random_case(m + n + k, m, n, k)
    qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
    need = gpu_lib.workspace_bytes(m, n, k, 0)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    xd = dev_bf16(c["x"])
    rows = sample_rows(m, 7, count=96) if m > 512 else np.arange(m)
    y_ref = O.gemm_ref(c["x"][rows], _oracle_w16(c["w"], bits))
    y1 = host(gpu_lib.dequant_gemm(xd, qw, torch.float32, workspace=ws))
    y2 = host(gpu_lib.dequant_gemm(xd, qw, torch.float32, workspace=ws))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "stream-K results differ between calls"
    check_product(y1[rows], y_ref, False, "stream-K f32")
    yb = host(gpu_lib.dequant_gemm(xd, qw, torch.bfloat16, workspace=ws))
    check_product(yb[rows], y_ref, True, "stream-K bf16")
    y_plain = host(gpu_lib.dequant_gemm(xd, qw, torch.float32, workspace=torch.empty(16, dtype=torch.uint8, device="cuda")))
    check_product(y_plain[rows], y_ref, False, "whole tiles")
    assert np.max(np.abs(y1 - y_plain)) <= 1e-5 * np.max(np.abs(y_plain)) + 1e-6


# ------------------------------------------------------------------ M <= 16: K split across workgroups
@pytest.mark.parametrize("m,n,k,bits", [(16, 5120, 13824, 5), (7, 1040, 8192, 3), (1, 48, 8320, 7),
                                        (16, 2048, 8192, 4), (13, 3184, 8192, 6), (16, 48, 40960, 6)])
def test_gemm_small_m_split_k(gpu_lib, m, n, k, bits):
    """16-token products with long K split K into 8 parts across workgroups
    when given a workspace (odd column-block counts, parts of unequal group
    counts): against the oracle, bit-identical on a second call, and within
    float32 summation order of the call without a workspace."""
    _case(f"dequant_gemm 16-token split K m={m} n={n} k={k} bits={bits}")
    c = synth.random_case(m * 31 + n + k, m, n, k)
    qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
    need = gpu_lib.workspace_bytes(m, n, k, 0)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    xd = dev_bf16(c["x"])
    y_ref = O.gemm_ref(c["x"], _oracle_w16(c["w"], bits))
    y1 = host(gpu_lib.dequant_gemm(xd, qw, torch.float32, workspace=ws))
    y2 = host(gpu_lib.dequant_gemm(xd, qw, torch.float32, workspace=ws))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "split results differ between calls"
    check_product(y1, y_ref, False, "split f32")
    yb = host(gpu_lib.dequant_gemm(xd, qw, torch.bfloat16, workspace=ws))
    check_product(yb, y_ref, True, "split bf16")
    y_plain = host(gpu_lib.dequant_gemm(xd, qw, torch.float32, workspace=torch.empty(16, dtype=torch.uint8, device="cuda")))
    assert np.max(np.abs(y1 - y_plain)) <= 1e-5 * np.max(np.abs(y_plain)) + 1e-6


# ------------------------------------------------------------------ M <= 16: repeatability
@pytest.mark.parametrize("m,n,k,bits", [
    (16, 3072, 3072, 4), (1, 16, 128, 3), (5, 272, 384, 5), (16, 5120, 5120, 4), (11, 5120, 6144, 5),
    (16, 15360, 5120, 6), (3, 1040, 1024, 7), (16, 12800, 40960, 6), (2, 12816, 640, 3)])
def test_gemm_small_m_repeatable(gpu_lib, m, n, k, bits):
    """The M <= 16 kernels that keep K inside a workgroup (K < 8192, or
    12800 columns and more; partial tiles added in wave order) against the
    oracle, equal to themselves bit for bit on a second call, with and
    without a workspace (they use none)."""
    _case(f"dequant_gemm M<=16 repeatability m={m} n={n} k={k} bits={bits}")
    c = synth.random_case(m * 31 + n + k, m, n, k)
    qw = gpu_lib.quantize_pack(dev_bf16(c["w"]), bits)
    assert gpu_lib.workspace_bytes(m, n, k, 0) == 0
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    xd = dev_bf16(c["x"])
    y_ref = O.gemm_ref(c["x"], _oracle_w16(c["w"], bits))
    y1 = host(gpu_lib.dequant_gemm(xd, qw, torch.float32, workspace=ws))
    y2 = host(gpu_lib.dequant_gemm(xd, qw, torch.float32))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "results differ between calls"
    check_product(y1, y_ref, False, "f32")
    check_product(host(gpu_lib.dequant_gemm(xd, qw, torch.bfloat16)), y_ref, True, "bf16")


# ------------------------------------------------------------------ low-rank branch
def _lowrank_case(api, x, w, bits, r, rows=None, out=torch.float32):
    l1, l2, res = O.svd_split(w, r)
    qr, q_ref, s_ref = _quant_exact(api, res, bits, f32_input=True,
                                    rows=None if w.shape[0] <= 512 else sample_weight_rows(w.shape[0], r))
    w16 = O.dequant_bf16(*O.quantize_groups(res, bits), bits)
    rows = np.arange(x.shape[0]) if rows is None else rows
    y_ref, _ = O.lowrank_fused_ref(x[rows], w16, l1, l2)
    ld = dev_bf16(np.ascontiguousarray(l1.T))
    lu = dev_bf16(np.ascontiguousarray(l2.T))
    y = host(api.lowrank_fused_gemm(dev_bf16(x), qr, ld, lu, out))
    return check_product(y[rows], y_ref, out == torch.bfloat16)


def _check_t(api, x, l1, what):
    """T = bf16(X L1) from ddg_lowrank_down against the oracle's
    bf16(fl32(X L1)) summed in float64.  The kernel sums the exact bf16
    products in float32, so its sum is within (K - 1) 2^-24 sum|x l1| of the
    exact one, and the two bf16 roundings can then land one bf16 step apart
    (2^-7 of the value at most).  Every element is held to that bound, and at
    least 99% must be equal bit for bit."""
    t_ref = O.lowrank_t_ref(x, l1)
    t = host(api.lowrank_down(dev_bf16(x), dev_bf16(np.ascontiguousarray(l1.T)))).astype(np.float64)
    tr = t_ref.astype(np.float64)
    absdot = np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(l1, np.float64))
    bound = 2.0 ** -7 * np.maximum(np.abs(t), np.abs(tr)) + (x.shape[1] - 1) * 2.0 ** -24 * absdot
    err = np.abs(t - tr)
    assert np.all(err <= bound), f"{what}: T off by {np.max(err - bound):.3e} beyond the bound"
    same = np.mean(t == tr)
    assert same >= 0.99, f"{what}: only {same:.4f} of T equal to the oracle"
    return same


@pytest.mark.parametrize("m,k,r", [(1, 128, 8), (17, 640, 24), (100, 256, 128), (33, 1024, 40),
                                   (300, 3072, 32),
                                   (16400, 256, 48),     # two row blocks per workgroup
                                   (32790, 128, 32)])    # four, the last workgroup 22 rows
def test_lowrank_down_small_shapes(gpu_lib, m, k, r):
    """The pre-pass alone at ragged row counts (the last 16-row block partly
    filled), every rank class, and the grids that give a workgroup two or
    four row blocks."""
    _case(f"lowrank_down m={m} k={k} r={r}")
    rng = np.random.default_rng(m * 131 + r)
    x = O.bf16_rne(rng.standard_normal((m, k)).astype(np.float32))
    l1 = O.bf16_rne((rng.standard_normal((k, r)) / np.sqrt(k)).astype(np.float32))
    _check_t(gpu_lib, x, l1, f"m={m} k={k} r={r}")


def test_lowrank_down_config4(gpu_lib):
    """Workload 4's T at full size: X 4096 x 3072 with its outlier channels and
    the rank-32 factor of the SVD split of its weight, every element."""
    _case("lowrank_down workload 4 (4096 x 3072, r = 32)")
    c = synth.config4()
    l1, _, _ = O.svd_split(c["w"], 32)
    same = _check_t(gpu_lib, c["x"], l1, "workload 4")
    print(f"[case] workload 4 T equal to the oracle: {same:.5f}", flush=True)


@pytest.mark.parametrize("r", [8, 16, 40, 64, 128])
@pytest.mark.parametrize("m", [5, 16, 48, 100])
def test_lowrank_small_shapes(gpu_lib, r, m):
    _case(f"lowrank_fused_gemm m={m} r={r}")
    c = synth.random_case(r * 100 + m, m, 144, 384, wstd=0.05)
    _lowrank_case(gpu_lib, c["x"], c["w"], 4, r)
    _lowrank_case(gpu_lib, c["x"], c["w"], 5, r, out=torch.bfloat16)


def test_lowrank_wide_small_m(gpu_lib):
    _case("lowrank_fused_gemm wide small-M m=16 n=12816 k=640 r=32")
    c = synth.random_case(4242, 16, 12816, 640, wstd=0.05)
    _lowrank_case(gpu_lib, c["x"], c["w"], 5, 32)
    _lowrank_case(gpu_lib, c["x"][:3], c["w"], 4, 32, out=torch.bfloat16)


@pytest.mark.parametrize("m,n,k,r", [(1, 272, 1024, 8), (16, 272, 5120, 32), (37, 144, 13824, 128),
                                     (64, 272, 3072, 40), (16, 5120, 13824, 32)])
def test_lowrank_split_prepass(gpu_lib, m, n, k, r):
    """At most 64 token rows and at least 8 groups, with the workspace
    ddg_workspace_bytes asks for: the pre-pass splits K over workgroups
    (float32 partials after the product's own split-K area, added in chunk
    order).  T (the workspace's first bytes) against the oracle's T, Y against
    the oracle, and two calls equal bit for bit."""
    _case(f"lowrank_fused_gemm split pre-pass m={m} n={n} k={k} r={r}")
    c = synth.random_case(7000 + m + r, m, n, k, wstd=0.05)
    l1, l2, res = O.svd_split(c["w"], r)
    qr = gpu_lib.quantize_pack(torch.from_numpy(res).to("cuda"), 4)
    w16 = O.dequant_bf16(*O.quantize_groups(res, 4), 4)
    ld = dev_bf16(np.ascontiguousarray(l1.T))
    lu = dev_bf16(np.ascontiguousarray(l2.T))
    ws = torch.empty(gpu_lib.workspace_bytes(m, n, k, r), dtype=torch.uint8, device="cuda")
    x = dev_bf16(c["x"])
    y1 = host(gpu_lib.lowrank_fused_gemm(x, qr, ld, lu, torch.float32, workspace=ws))
    t = ws[:m * r * 2].view(torch.bfloat16).view(m, r).float().cpu().numpy().astype(np.float64)
    t_ref = O.lowrank_t_ref(c["x"], l1).astype(np.float64)
    absdot = np.abs(np.asarray(c["x"], np.float64)) @ np.abs(np.asarray(l1, np.float64))
    bound = 2.0 ** -7 * np.maximum(np.abs(t), np.abs(t_ref)) + (k - 1) * 2.0 ** -24 * absdot
    assert np.all(np.abs(t - t_ref) <= bound), "T beyond the float32 summation bound"
    assert np.mean(t == t_ref) >= 0.99, "T: fewer than 99% equal to the oracle"
    y2 = host(gpu_lib.lowrank_fused_gemm(x, qr, ld, lu, torch.float32, workspace=ws))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "split pre-pass results differ between calls"
    y_ref, _ = O.lowrank_fused_ref(c["x"], w16, l1, l2)
    check_product(y1, y_ref, False, "split pre-pass f32")
    yb = host(gpu_lib.lowrank_fused_gemm(x, qr, ld, lu, torch.bfloat16, workspace=ws))
    check_product(yb, y_ref, True, "split pre-pass bf16")


def test_lowrank_config4(gpu_lib):
    _case("lowrank_fused_gemm workload 4 (M=4096, r=32)")
    c = synth.config4()
    _lowrank_case(gpu_lib, c["x"], c["w"], 4, 32, rows=sample_rows(4096, 4))
    _lowrank_case(gpu_lib, c["x"][:16], c["w"], 4, 32, out=torch.bfloat16)
