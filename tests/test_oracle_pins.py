"""Pins of the CPU oracle against what the pages and mathematics fix (CPU only).

Each test names the passage it follows.  Page short names:
[WDQ]  the Wan-Dancer-14B mixed-precision quantization report (mtrt.cn)
[SVDQ] "SVDQuant：4-bit量化让扩散模型在消费级GPU上高效运行" (kongchang.com)
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from dit_dequant_gemm_amd import synth
from pinlib import exact_group_quantize, f32_bits, frac_of_f32, nearest_level

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BITS = (3, 4, 5, 6, 7)


def _f32_bits_arr(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_rne_matches_library_conversion():
    """bf16 round-to-nearest-even, checked against torch's CPU conversion."""
    import torch
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.normal(0, 1, 20000), rng.normal(0, 1e-3, 5000), rng.normal(0, 1e4, 5000),
        [0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-42],
    ]).astype(np.float32)
    # exact ties: low 16 bits == 0x8000 with odd and even kept parts
    ties = (rng.integers(0x3F000000 >> 16, 0x47000000 >> 16, 4000).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([x, ties.view(np.float32)])
    got = O.bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(_f32_bits_arr(got), _f32_bits_arr(ref))


# ---------------------------------------------------------------- quantizer
@pytest.mark.parametrize("bits", BITS)
def test_quantizer_matches_exact_binary32_model(bits):
    """[WDQ] §3.1: abs-max x1.01, step = 2*abs_max/(2^b-1), round, clamp.

    The oracle's numpy float32 arithmetic must equal exact rational arithmetic
    with explicit binary32 rounding after each operation (reading R2), bit for
    bit, on small groups of varied magnitude (including subnormal ones).
    """
    rng = np.random.default_rng(100 + bits)
    rows = [rng.normal(0, 0.02, 128), rng.normal(0, 1.0, 128), rng.standard_t(3, 128) * 5,
            rng.normal(0, 1e-39, 128), rng.uniform(-1, 1, 128), np.round(rng.normal(0, 4, 128))]
    w = np.stack(rows).astype(np.float32)
    q_u, scales = O.quantize_groups(w, bits)
    nh = O.n_half(bits)
    for i in range(w.shape[0]):
        step, qs = exact_group_quantize(w[i], bits)
        assert f32_bits(step) == int(_f32_bits_arr(scales[i, 0])[0])
        assert list(q_u[i].astype(int) - nh) == qs


@pytest.mark.parametrize("bits", BITS)
def test_code_is_nearest_level_brute_force(bits):
    """Each code is the level nearest to the weight (ties to even) -- brute force
    over all 2*n_half+1 levels with exact arithmetic.  The only allowed
    difference is where w/step lies within 2^-20 of a tie, since the page's
    step first rounds the quotient to float32."""
    rng = np.random.default_rng(200 + bits)
    w = rng.normal(0, 0.02, (3, 128)).astype(np.float32)
    q_u, scales = O.quantize_groups(w, bits)
    nh = O.n_half(bits)
    for i in range(3):
        step = frac_of_f32(scales[i, 0])
        for j in range(128):
            q_best, tie_dist = nearest_level(frac_of_f32(w[i, j]), step, nh)
            if tie_dist > Fraction(1, 2 ** 20):
                assert int(q_u[i, j]) - nh == q_best


@pytest.mark.parametrize("bits", BITS)
def test_quantizer_invariants(bits):
    """Consequences of the §3.1 formula (reading R1/R3):
    codes lie in [0, 2^b-2]; each nonzero group holds +-n_half (its abs-max
    element); |w - w_hat| <= step/2; sign symmetry; all-zero groups."""
    rng = np.random.default_rng(300 + bits)
    w = np.concatenate([rng.normal(0, 0.02, (32, 512)), rng.standard_t(4, (32, 512)) * 0.01]).astype(np.float32)
    w[5, 128:256] = 0.0                                  # one all-zero group
    q_u, s = O.quantize_groups(w, bits)
    nh = O.n_half(bits)
    assert q_u.max() <= 2 ** bits - 2
    qg = q_u.reshape(64, 4, 128).astype(int)
    nz = s > 0
    has_extreme = (qg == 0).any(-1) | (qg == 2 * nh).any(-1)
    assert np.all(has_extreme[nz])
    assert s[5, 1] == 0 and np.all(q_u[5, 128:256] == nh)
    wh = O.dequant_f32(q_u, s, bits)
    err = np.abs(w.astype(np.float64) - wh.astype(np.float64)).reshape(64, 4, 128)
    bound = s.astype(np.float64)[..., None] / 2 * (1 + 2 ** -21)
    assert np.all(err <= bound)
    q_neg, s_neg = O.quantize_groups(-w, bits)
    assert np.array_equal(_f32_bits_arr(s_neg), _f32_bits_arr(s))
    assert np.array_equal(q_neg.astype(int), 2 * nh - q_u.astype(int))


def test_outlier_example_collapses_normal_values():
    """[SVDQ] outlier example: values in [-1, 1] plus one outlier of 100 at
    4 bit -- the step is ~13.47 and every ordinary value lands on code 0."""
    rng = np.random.default_rng(7)
    g = rng.uniform(-1, 1, 128).astype(np.float32)
    g[37] = 100.0
    q_u, s = O.quantize_groups(g[None, :], 4)
    assert s[0, 0] == pytest.approx(2 * 100 * 1.01 / 15, rel=1e-6)
    q = q_u[0].astype(int) - O.n_half(4)
    assert q[37] == 7
    assert np.all(np.delete(q, 37) == 0)


def test_per_group_scale_count_5120():
    """[WDQ] §3.1 table: in=5120 gives 5120 x 40 = 204,800 per-group scales
    (5120 per-channel); storage out*(in/128)*4 bytes."""
    w = np.ones((5120, 5120), dtype=np.float32)
    _, s = O.quantize_groups(w, 4)
    assert s.size == 204_800 and s.dtype == np.float32 and s.nbytes == 5120 * 40 * 4
    _, sc = O.quantize(w, 4, "channel")
    assert sc.size == 5120


# ---------------------------------------------------------------- packing
@pytest.mark.parametrize("bits,ratio", [(3, (8, 3)), (4, (2, 1)), (5, (8, 5)), (6, (4, 3)), (7, (8, 7))])
def test_packed_byte_counts(bits, ratio):
    """[WDQ] §3.3 table: 8 weights -> 3/5/7 bytes, 2 -> 1 byte, 4 -> 3 bytes."""
    nw, nb = ratio
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 2 ** bits - 1, size=nw * 16).astype(np.uint8)
    assert O.pack_codes(codes, bits).size == 16 * nb
    q_u, _ = O.quantize_groups(rng.normal(0, 1, (3, 256)).astype(np.float32), bits)
    assert O.pack_codes(q_u, bits).size == 3 * 256 * bits // 8 == O.packed_nbytes(3, 256, bits)
    assert O.packed_nbytes(1, 128, bits) == 16 * bits      # one group: 16*b bytes


def _read_golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or not line.strip():
            continue
        rows.append([p.strip() for p in line.split("|")])
    return rows


def test_pack_int4_golden():
    """[WDQ] §3.3 4-bit pack/unpack: even-index code in the high nibble."""
    rows = _read_golden("pack_int4.txt")
    assert len(rows) == 4
    for codes, packed in rows:
        c = np.array([int(v) for v in codes.split()], dtype=np.uint8)
        p = np.array([int(v, 16) for v in packed.split()], dtype=np.uint8)
        assert np.array_equal(O.pack_codes(c, 4), p)
        # the page's unpack: high nibble, low nibble, interleaved
        assert np.array_equal(O.unpack_codes(p, 4, c.size), c)
        hi, lo = p >> 4, p & 0xF
        assert np.array_equal(np.stack([hi, lo], 1).reshape(-1), c)


def test_pack_msb_first_golden():
    """Reading R4: MSB-first continuous bitstream (hand-derived fixtures)."""
    rows = _read_golden("pack_msb_first.txt")
    assert len(rows) == 8
    for b, codes, packed in rows:
        b = int(b)
        c = np.array([int(v) for v in codes.split()], dtype=np.uint8)
        p = np.array([int(v, 16) for v in packed.split()], dtype=np.uint8)
        assert np.array_equal(O.pack_codes(c, b), p)
        assert np.array_equal(O.unpack_codes(p, b, c.size), c)


@pytest.mark.parametrize("bits", BITS)
def test_pack_matches_bitstring_brute_force(bits):
    """Independent construction: concatenate binary strings, cut into bytes."""
    rng = np.random.default_rng(50 + bits)
    c = rng.integers(0, 2 ** bits - 1, size=8 * 37).astype(np.uint8)
    s = "".join(format(int(v), "0%db" % bits) for v in c)
    ref = np.array([int(s[i:i + 8], 2) for i in range(0, len(s), 8)], dtype=np.uint8)
    assert np.array_equal(O.pack_codes(c, bits), ref)


@pytest.mark.parametrize("bits", BITS)
def test_pack_unpack_round_trip(bits):
    rng = np.random.default_rng(60 + bits)
    w = rng.normal(0, 0.02, (16, 384)).astype(np.float32)
    q_u, s = O.quantize_groups(w, bits)
    p = O.pack_codes(q_u, bits)
    assert np.array_equal(O.unpack_codes(p, bits, q_u.size).reshape(q_u.shape), q_u)
    assert np.array_equal(O.dequant_from_packed(p, s, bits, 16, 384), O.dequant_bf16(q_u, s, bits))


# ---------------------------------------------------------------- SNR behaviour
def _config_tensors():
    c1 = synth.config1()["w"]
    c2 = synth.config2(m=1)["w"][:256]
    c3u = synth._student_t_weight(np.random.default_rng([3, 0]), 256, 3072)
    c4 = synth.config4(m=1)["w"][:256]
    c5 = synth.config5_weights("down", rows=128)
    return {"c1": c1, "c2": c2, "c3_up": c3u, "c4": c4, "c5_down": c5}


@pytest.mark.slow
def test_snr_rises_tensor_channel_group():
    """[WDQ] §2.1 table: per-tensor < per-channel < per-group SNR, on every
    workload tensor (first rows) at every bit width."""
    for name, w in _config_tensors().items():
        for b in BITS:
            snr = {}
            for gran in ("tensor", "channel", "group"):
                q_u, s = O.quantize(w, b, gran)
                snr[gran] = O.snr_db(w, O.dequant_f32(q_u, s, b))
            assert snr["tensor"] < snr["channel"] < snr["group"], (name, b, snr)


def test_snr_gains_about_6db_per_bit():
    """Uniform quantization noise is step^2/12 and the step halves per extra
    bit (2^b - 1 levels): about 20*log10(2) = 6.02 dB per bit on Gaussian data."""
    w = np.random.default_rng(11).normal(0, 0.02, (256, 1024)).astype(np.float32)
    snrs = []
    for b in BITS:
        q_u, s = O.quantize_groups(w, b)
        snrs.append(O.snr_db(w, O.dequant_f32(q_u, s, b)))
    d = np.diff(snrs)
    assert np.all(d > 5.5) and np.all(d < 6.8), snrs
    # closed form for the 4-bit level: noise ~ mean(step^2)/12
    q_u, s = O.quantize_groups(w, 4)
    pred = 10 * np.log10(np.mean(w.astype(np.float64) ** 2) / (np.mean(s.astype(np.float64) ** 2) / 12))
    assert abs(snrs[1] - pred) < 0.5


# ---------------------------------------------------------------- contractions
def test_gemm_ref_matches_naive_loop():
    """Textbook definition Y[m, n] = sum_k X[m, k] * W[n, k], with exact sums."""
    rng = np.random.default_rng(3)
    x = synth.to_bf16(rng.normal(0, 1, (5, 19)))
    w = synth.to_bf16(rng.normal(0, 1, (7, 19)))
    y = O.gemm_ref(x, w)
    for m in range(5):
        for n in range(7):
            exact = math.fsum(float(x[m, k]) * float(w[n, k]) for k in range(19))
            assert y[m, n] == pytest.approx(exact, rel=1e-14, abs=1e-14)


def test_lowrank_ref_definition():
    """T is X @ L1 rounded to float32 then bf16; Y adds T @ L2 in float64."""
    rng = np.random.default_rng(4)
    x = synth.to_bf16(rng.normal(0, 1, (6, 32)))
    l1 = synth.to_bf16(rng.normal(0, 1, (32, 8)))
    l2 = synth.to_bf16(rng.normal(0, 1, (8, 5)))
    w = synth.to_bf16(rng.normal(0, 1, (5, 32)))
    y, t = O.lowrank_fused_ref(x, w, l1, l2)
    for m in range(6):
        for j in range(8):
            exact = math.fsum(float(x[m, k]) * float(l1[k, j]) for k in range(32))
            assert t[m, j] == O.bf16_rne(np.float32(exact))[()]
        for n in range(5):
            exact = math.fsum([float(x[m, k]) * float(w[n, k]) for k in range(32)]
                              + [float(t[m, j]) * float(l2[j, n]) for j in range(8)])
            assert y[m, n] == pytest.approx(exact, rel=1e-13, abs=1e-12)


def test_eckart_young_rank_r_residual():
    """[SVDQ]: the top-r singular triplets give the best rank-r approximation.
    ||W - W_r||_F^2 equals the sum of the dropped squared singular values
    (from eigvalsh(W^T W), an independent routine) and random rank-r
    candidates never do better.  The oracle's split reproduces W exactly up to
    float32 rounding of the residual."""
    rng = np.random.default_rng(5)
    w = rng.normal(0, 1, (24, 16))
    r = 4
    lam = np.sort(np.linalg.eigvalsh(w.T @ w))[::-1]
    best = float(np.sum(lam[r:]))
    l1, l2, res = O.svd_split(w.astype(np.float32), r)
    lr = (l1.astype(np.float64) @ l2.astype(np.float64)).T
    # with bf16 factors the residual is within bf16 rounding of the optimum
    assert abs(np.sum((w - lr) ** 2) - best) <= 0.05 * best
    u, s, vt = np.linalg.svd(w)
    wr = (u[:, :r] * s[:r]) @ vt[:r]
    assert np.sum((w - wr) ** 2) == pytest.approx(best, rel=1e-9)
    for _ in range(50):
        a = rng.normal(size=(24, r))
        b = np.linalg.lstsq(a, w, rcond=None)[0]
        assert np.sum((w - a @ b) ** 2) >= best * (1 - 1e-9)
    w32 = w.astype(np.float32)
    assert np.allclose(lr + res.astype(np.float64), w32.astype(np.float64), rtol=0, atol=1e-6)


@pytest.mark.slow
def test_lowrank_absorbs_outliers_config4():
    """[SVDQ] 技术原理详解: after the rank-32 branch takes the outlier term, the
    4-bit residual's error is far below quantizing W directly (workload 4)."""
    c = synth.config4(m=1)
    w = c["w"]
    l1, l2, res = O.svd_split(w, 32)
    q_r, s_r = O.quantize_groups(res, 4)
    approx = (l1.astype(np.float64) @ l2.astype(np.float64)).T + O.dequant_f32(q_r, s_r, 4)
    q_w, s_w = O.quantize_groups(w, 4)
    direct = O.dequant_f32(q_w, s_w, 4)
    w64 = w.astype(np.float64)
    e_lr = np.linalg.norm(approx - w64) / np.linalg.norm(w64)
    e_q = np.linalg.norm(direct - w64) / np.linalg.norm(w64)
    assert e_lr < 0.3 * e_q, (e_lr, e_q)
