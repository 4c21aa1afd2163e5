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
