"""FP4 weights and FP8 activations ([FP4] §3.1.2, §3.2, §4.1): the oracle
against what the formats and the mathematics fix.  All on the CPU."""
import numpy as np
import pytest

from oracle import fp4 as F


def test_e2m1_values_are_the_standard_fp4_set():
    # the OCP FP4 (E2M1) magnitudes
    assert list(F.fp4_values("e2m1")) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e1m2_is_uniform_and_e3m0_is_powers_of_two():
    assert np.allclose(F.fp4_values("e1m2"), np.arange(8) * 0.25)
    e3 = F.fp4_values("e3m0")
    assert e3[0] == 0.0 and np.all(e3[2:] / e3[1:-1] == 2.0) and e3[-1] == 16.0 and e3[1] == 0.25


def test_e4m3_facts():
    v = F.e4m3_values()
    assert len(v) == 127 and v[-1] == 448.0                 # 0x7E is the largest finite value
    assert v[1] == 2.0 ** -9 and v[8] == 2.0 ** -6           # smallest subnormal, smallest normal
    assert F.e4m3_decode([0x38, 0x40, 0xC0, 0x7E])[0] == 1.0
    assert list(F.e4m3_decode([0x38, 0x40, 0xC0, 0x7E])) == [1.0, 2.0, -2.0, 448.0]
    assert np.all(np.diff(v) > 0)


def _brute_nearest(r, levels):
    d = np.abs(np.abs(r)[:, None] - levels[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.where(cand, np.arange(len(levels))[None, :], 10 ** 6)
    even = np.where(cand & (np.arange(len(levels))[None, :] % 2 == 0), np.arange(len(levels))[None, :], 10 ** 6)
    return np.where(cand.sum(axis=1) > 1, even.min(axis=1), idx.min(axis=1))


@pytest.mark.parametrize("fmt", list(F.FP4_FORMATS))
def test_fp4_rounding_is_nearest_ties_to_even(fmt):
    lv = F.fp4_values(fmt)
    rng = np.random.default_rng(1)
    r = np.concatenate([rng.uniform(-lv[-1] * 1.1, lv[-1] * 1.1, 4000),
                        (lv[1:] + lv[:-1]) / 2, -(lv[1:] + lv[:-1]) / 2, lv, -lv])
    got = F._nearest_index(np.abs(r), lv)
    want = np.minimum(_brute_nearest(np.minimum(np.abs(r), lv[-1]), lv), 7)
    assert np.array_equal(got, want)


def test_e4m3_rounding_is_nearest_ties_to_even():
    lv = F.e4m3_values()
    rng = np.random.default_rng(2)
    r = np.concatenate([rng.uniform(-500, 500, 3000), rng.uniform(-0.02, 0.02, 3000),
                        (lv[1:] + lv[:-1]) / 2, lv])
    codes = F.e4m3_round(r)
    want = _brute_nearest(np.minimum(np.abs(r), 448.0), lv)
    assert np.array_equal(codes & 0x7F, want)
    assert np.all(((codes & 0x80) != 0) == ((r < 0) & (want > 0)))


def test_pack_order_worked_example():
    codes = np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8)
    assert list(F.pack_fp4(codes)[0]) == [0x21, 0x43, 0x0F]
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, size=(5, 256)).astype(np.uint8)
    assert np.array_equal(F.unpack_fp4(F.pack_fp4(c)), c)


@pytest.mark.parametrize("fmt", list(F.FP4_FORMATS))
def test_fp4_group_quantizer(fmt):
    rng = np.random.default_rng(4)
    w = (rng.standard_t(4, size=(8, 512)) * 0.02).astype(np.float32)
    w[0, :128] = 0.0                                          # a zero group
    codes, s = F.quantize_fp4_groups(w, fmt)
    assert s[0, 0] == 0.0 and np.all(codes[0, :128] == 0)
    lv = F.fp4_values(fmt)
    for r in range(8):
        for g in range(4):
            sl = slice(128 * g, 128 * g + 128)
            if s[r, g] == 0:
                continue
            # the group's largest magnitude takes the top code
            j = np.argmax(np.abs(w[r, sl]))
            assert codes[r, sl][j] & 7 == 7
            # every code is the nearest level to fl32(w / s)
            q = (w[r, sl] / s[r, g]).astype(np.float32)
            assert np.array_equal(codes[r, sl] & 7, np.minimum(_brute_nearest(np.minimum(np.abs(q), lv[-1]), lv), 7))
    # sign: negative weights carry bit 3 unless they round to zero
    assert np.all(((codes & 8) != 0) <= (w < 0))


def test_rows_e4m3_quantizer():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, size=(6, 384)).astype(np.float32)
    x[2] = 0.0
    codes, s = F.quantize_rows_e4m3(x)
    assert s[2] == 0 and np.all(codes[2] == 0)
    for r in (0, 1, 3):
        j = np.argmax(np.abs(x[r]))
        assert codes[r, j] & 0x7F == 0x7E                     # the row's amax maps to 448
    xhat = F.e4m3_decode(codes) * s[:, None]
    assert np.all(np.abs(xhat - x) <= np.abs(x) * 2.0 ** -4 + s[:, None] * 2.0 ** -9)


def test_w4a8_reference_against_loops():
    rng = np.random.default_rng(6)
    m, n, k = 3, 4, 256
    xc = rng.integers(0, 255, size=(m, k)).astype(np.uint8)
    xc[(xc & 0x7F) == 0x7F] = 0x38                             # no NaN codes
    wc = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    sx = rng.uniform(0.01, 2, m).astype(np.float32)
    sw = rng.uniform(0.01, 2, (n, 2)).astype(np.float32)
    y = F.w4a8_ref(xc, sx, wc, sw, "e2m1")
    qx = F.e4m3_decode(xc)
    vw = F.fp4_decode(wc, "e2m1")
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                acc += float(sw[j, kk // 128]) * qx[i, kk] * vw[j, kk]
            assert abs(y[i, j] - float(sx[i]) * acc) <= 1e-9 * max(1.0, abs(y[i, j]))


@pytest.mark.parametrize("fmt", list(F.FP4_FORMATS))
def test_power_of_two_scales(fmt):
    rng = np.random.default_rng(7)
    w = (rng.normal(0, 0.02, size=(6, 384))).astype(np.float32)
    w[1, :128] = 0.0
    w[2, 128:256] *= np.float32(1e-40)                        # group scale below 2^-126
    codes, s = F.quantize_fp4_groups(w, fmt, pow2=True)
    _, s_plain = F.quantize_fp4_groups(w, fmt)
    nz = s > 0
    m, _ = np.frexp(s[nz].astype(np.float64))
    assert np.all(m == 0.5)                                    # powers of two
    assert np.all(s[nz] >= s_plain[nz]) and np.all(s[nz] < 2 * s_plain[nz] + 2.0 ** -126)
    assert s[1, 0] == 0 and np.all(codes[1, :128] == 0)
    assert s[2, 1] == np.float32(2.0 ** -126)
    lv = F.fp4_values(fmt)
    q = (w.reshape(6, 3, 128) / np.where(s > 0, s, 1)[:, :, None]).astype(np.float32)
    assert np.all(np.abs(q) <= lv[-1])                         # nothing saturates
    want = np.minimum(_brute_nearest(np.minimum(np.abs(q.reshape(-1)), lv[-1]), lv), 7).reshape(6, 384)
    assert np.array_equal(np.where(np.repeat(s, 128, axis=1) > 0, codes & 7, 0), np.where(np.repeat(s, 128, axis=1) > 0, want, 0))
    # exactly a power of two already: kept
    assert np.all(F._pow2_at_least(np.float32([0.25, 1.0, 3.0, 2.0 ** -130])) == np.float32([0.25, 1.0, 4.0, 2.0 ** -126]))


def test_tiled_layout_positions_by_hand():
    """R24 positions worked out by hand for n = 40 (two blocks, the second
    padded), k = 256 (G = 2)."""
    n, k = 40, 256
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.random((n, 2), dtype=np.float32) + 1
    t, ts = F.tile_fp4(packed, scales)
    assert t.shape == (2 * 2 * 2048,) and ts.shape == (2 * 2 * 32,)
    # column 33 (block 1, j = 1), group 1, row byte 64 + 32*1 + 16*0 + 5:
    # (1*2 + 1)*2048 + 1*1024 + 0*512 + 1*16 + 5 = 7189
    assert t[7189] == packed[33, 64 + 32 + 5]
    # column 0, group 0, row byte 16 + 15 (s = 0, h = 1, t = 15): 512 + 15
    assert t[527] == packed[0, 31]
    # column 31, group 1, row byte 64 + 32 + 16 + 0 (s = 1, h = 1): 2048 + 1024 + 512 + 31*16
    assert t[2048 + 1024 + 512 + 496] == packed[31, 112]
    # padded column 45 of block 1 reads zero everywhere
    assert t[2 * 2048 + 13 * 16: 2 * 2048 + 14 * 16].sum() == 0
    assert ts[(1 * 2 + 1) * 32 + 1] == scales[33, 1] and ts[(1 * 2 + 0) * 32 + 13] == 0
    assert ts[0 * 32 + 31] == scales[31, 0]


def test_tiled_layout_is_a_permutation_and_inverts():
    n, k = 70, 384
    # every byte value distinct per position: tag each byte by its position
    packed = (np.arange(n * k // 2, dtype=np.int64).reshape(n, k // 2) % 251 + 1).astype(np.uint8)
    scales = np.arange(n * 3, dtype=np.float32).reshape(n, 3) + 1
    t, ts = F.tile_fp4(packed, scales)
    back, bs = F.untile_fp4(t, ts, n, k)
    assert np.array_equal(back, packed) and np.array_equal(bs, scales)
    # multiset of bytes kept, the rest zeros (padding)
    assert np.array_equal(np.sort(t[t > 0]), np.sort(packed.reshape(-1)))
    assert np.count_nonzero(t) == packed.size and np.count_nonzero(ts) == scales.size


def test_fp6_formats_published_facts():
    e23, e32 = F.fp6_values("e2m3"), F.fp6_values("e3m2")
    assert len(e23) == 32 and len(e32) == 32
    assert e23[-1] == 7.5 and e32[-1] == 28.0                  # largest finite values of the two formats
    assert e23[1] == 0.125 and e32[1] == 0.0625                # smallest subnormals
    assert e23[8] == 1.0 and e32[4] == 0.25                    # smallest normals
    assert np.all(np.diff(e23) > 0) and np.all(np.diff(e32) > 0)
    assert list(F.fp6_decode([8, 40, 31, 63], "e2m3")) == [1.0, -1.0, 7.5, -7.5]


@pytest.mark.parametrize("fmt", list(F.FP6_FORMATS))
def test_fp6_rows_quantizer(fmt):
    lv = F.fp6_values(fmt)
    rng = np.random.default_rng(8)
    x = rng.normal(0, 1, size=(5, 256)).astype(np.float32)
    x[3] = 0.0
    codes, s = F.quantize_rows_fp6(x, fmt)
    assert s[3] == 0 and np.all(codes[3] == 0)
    for r in (0, 1, 2, 4):
        assert codes[r, np.argmax(np.abs(x[r]))] & 31 == 31     # the row's amax takes the top code
        q = (x[r] / s[r]).astype(np.float32)
        want = _brute_nearest(np.minimum(np.abs(q), lv[-1]), lv)
        assert np.array_equal(codes[r] & 31, want)
    assert np.all(((codes & 32) != 0) <= (x < 0))
    # midpoints of every pair of levels (scale 1: a row whose amax is the top level)
    mids = np.concatenate([(lv[1:] + lv[:-1]) / 2, [lv[-1]]]).astype(np.float32)
    c, s1 = F.quantize_rows_fp6(mids[None, :], fmt)
    assert s1[0] == np.float32(lv[-1]) / np.float32(lv[-1])
    assert np.array_equal(c[0] & 31, _brute_nearest(mids, lv))


def test_fp6_tiled_positions_by_hand():
    m, k = 40, 256                                              # two row blocks (second padded), G = 2
    codes = np.zeros((m, k), dtype=np.uint8)
    codes[0, 5] = 1          # row 0, g 0, s 0, h 0, j 5: bit 30 -> piece 0 byte 3 = 0x40
    codes[0, 10] = 63        # j 10: bits 60..65 -> piece 0 byte 7 = 0xF0, piece 1 byte 0 = 0x03
    codes[33, 223] = 1       # row 33 (b 1, r 1), k 223 = g 1, s 1, h 0, j 31: bit 186 -> piece 2 byte 7 bit 2
    t = F.pack_fp6_tiled(codes)
    assert t.shape == (2 * 2 * 3072,)
    assert t[3] == 0x40 and t[7] == 0xF0 and t[256] == 0x03
    # record (1, 1) at (1*2 + 1)*3072; piece ((1*2 + 0)*3 + 2)*256; row 1 at 8
    assert t[9216 + 2048 + 8 + 7] == 0x04
    assert np.count_nonzero(t) == 4
    assert np.array_equal(F.unpack_fp6_tiled(t, m, k), codes)


def test_fp6_tiled_round_trip_and_bijection():
    rng = np.random.default_rng(9)
    m, k = 70, 384
    codes = rng.integers(0, 64, size=(m, k)).astype(np.uint8)
    t = F.pack_fp6_tiled(codes)
    assert t.size == 3 * 3 * 3072                               # ceil(70/32) row blocks x 3 groups
    assert np.array_equal(F.unpack_fp6_tiled(t, m, k), codes)
    # every set bit of the input lands once: bit counts agree
    assert int(np.unpackbits(t).sum()) == int(np.unpackbits(codes).sum())


def test_w4a6_reference_against_loops():
    rng = np.random.default_rng(10)
    m, n, k = 3, 4, 256
    xc = rng.integers(0, 64, size=(m, k)).astype(np.uint8)
    wc = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    sx = rng.uniform(0.01, 2, m).astype(np.float32)
    sw = rng.uniform(0.01, 2, (n, 2)).astype(np.float32)
    for afmt in F.FP6_FORMATS:
        y = F.w4a6_ref(xc, sx, wc, sw, "e2m1", afmt)
        qx, vw = F.fp6_decode(xc, afmt), F.fp4_decode(wc, "e2m1")
        for i in range(m):
            for j in range(n):
                acc = sum(float(sw[j, kk // 128]) * qx[i, kk] * vw[j, kk] for kk in range(k))
                assert abs(y[i, j] - float(sx[i]) * acc) <= 1e-9 * max(1.0, abs(y[i, j]))


# ------------------------------------------------------------------ FP6 weights (R27, R28)
@pytest.mark.parametrize("fmt", list(F.FP6_FORMATS))
def test_fp6_group_quantizer(fmt):
    lv = F.fp6_values(fmt)
    rng = np.random.default_rng(11)
    w = (rng.standard_t(4, size=(8, 512)) * 0.02).astype(np.float32)
    w[0, :128] = 0.0                                          # a zero group
    codes, s = F.quantize_fp6_groups(w, fmt)
    assert s[0, 0] == 0.0 and np.all(codes[0, :128] == 0)
    for r in range(8):
        for g in range(4):
            sl = slice(128 * g, 128 * g + 128)
            if s[r, g] == 0:
                continue
            assert codes[r, sl][np.argmax(np.abs(w[r, sl]))] & 31 == 31   # the group's amax takes the top code
            q = (w[r, sl] / s[r, g]).astype(np.float32)
            assert np.array_equal(codes[r, sl] & 31, _brute_nearest(np.minimum(np.abs(q), lv[-1]), lv))
    assert np.all(((codes & 32) != 0) <= (w < 0))
    assert codes.max() < 64


def test_fp6_group_quantizer_worked_examples():
    """Groups whose scale is a power of two, so every quotient is exact and the
    codes can be read off the level tables by hand (ties to the even code)."""
    # E2M3: amax 0.9375 -> s = 0.125; r = 7.5, -3.75, 0.9375 (tie 0.875 | 1.0),
    # 0.0625 (tie 0 | 0.125), -0.1875 (tie 0.125 | 0.25)
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, :5] = [0.9375, -0.46875, 0.1171875, 0.0078125, -0.0234375]
    c, s = F.quantize_fp6_groups(w, "e2m3")
    assert s[0, 0] == np.float32(0.125)
    assert list(c[0, :5]) == [31, 32 | 23, 8, 0, 32 | 2]
    # E3M2: amax 0.875 -> s = 0.03125; r = 28, 18 (tie 16 | 20), 1.125 (tie 1 | 1.25), -0.09375 (tie .0625 | .125)
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, :4] = [0.875, 0.5625, 0.03515625, -0.0029296875]
    c, s = F.quantize_fp6_groups(w, "e3m2")
    assert s[0, 0] == np.float32(0.03125)
    assert list(c[0, :4]) == [31, 28, 12, 32 | 2]


@pytest.mark.parametrize("fmt", list(F.FP6_FORMATS))
def test_fp6_group_power_of_two_scales(fmt):
    lv = F.fp6_values(fmt)
    rng = np.random.default_rng(12)
    w = rng.normal(0, 0.02, size=(6, 384)).astype(np.float32)
    w[1, :128] = 0.0
    codes, s = F.quantize_fp6_groups(w, fmt, pow2=True)
    _, s_plain = F.quantize_fp6_groups(w, fmt)
    nz = s > 0
    m, _ = np.frexp(s[nz].astype(np.float64))
    assert np.all(m == 0.5) and np.all(s[nz] >= s_plain[nz]) and np.all(s[nz] < 2 * s_plain[nz])
    assert s[1, 0] == 0 and np.all(codes[1, :128] == 0)
    q = (w.reshape(6, 3, 128) / np.where(s > 0, s, 1)[:, :, None]).astype(np.float32).reshape(6, 384)
    assert np.all(np.abs(q) <= lv[-1])                         # nothing saturates
    want = _brute_nearest(np.abs(q.reshape(-1)), lv).reshape(6, 384)
    live = np.repeat(s, 128, axis=1) > 0
    assert np.array_equal(np.where(live, codes & 31, 0), np.where(live, want, 0))


def test_tiled_group_scales_by_hand():
    n, k = 40, 256                                             # two column blocks (second padded), G = 2
    scales = np.arange(1, n * 2 + 1, dtype=np.float32).reshape(n, 2)
    ts = F.tile_group_scales(scales)
    assert ts.shape == (2 * 2 * 32,)
    assert ts[(1 * 2 + 1) * 32 + 1] == scales[33, 1]           # block 1, group 1, column 33
    assert ts[0 * 32 + 31] == scales[31, 0] and ts[(0 * 2 + 1) * 32 + 0] == scales[0, 1]
    assert ts[(1 * 2 + 0) * 32 + 13] == 0                       # column 45: padding
    assert np.array_equal(F.untile_group_scales(ts, n, k), scales)
    assert np.count_nonzero(ts) == scales.size


def test_w6a8_reference_against_loops():
    rng = np.random.default_rng(13)
    m, n, k = 3, 4, 256
    xc = rng.integers(0, 255, size=(m, k)).astype(np.uint8)
    xc[(xc & 0x7F) == 0x7F] = 0x38                             # no NaN codes
    wc = rng.integers(0, 64, size=(n, k)).astype(np.uint8)
    sx = rng.uniform(0.01, 2, m).astype(np.float32)
    sw = rng.uniform(0.01, 2, (n, 2)).astype(np.float32)
    for wfmt in F.FP6_FORMATS:
        y = F.w6a8_ref(xc, sx, wc, sw, wfmt)
        qx, vw = F.e4m3_decode(xc), F.fp6_decode(wc, wfmt)
        for i in range(m):
            for j in range(n):
                acc = sum(float(sw[j, kk // 128]) * qx[i, kk] * vw[j, kk] for kk in range(k))
                assert abs(y[i, j] - float(sx[i]) * acc) <= 1e-9 * max(1.0, abs(y[i, j]))
