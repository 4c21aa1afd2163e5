"""The RPBH rotation ([ORQ] §2.1, §2.2): the oracle against what the
mathematics fixes.  All on the CPU."""
import numpy as np
import pytest
import scipy.linalg

import oracle as O
from dit_dequant_gemm_amd import synth


@pytest.mark.parametrize("h", [1, 2, 4, 8, 64, 1024])
def test_hadamard_is_sylvester(h):
    hm = O.hadamard(h)
    assert np.array_equal(hm, scipy.linalg.hadamard(h).astype(np.float64))
    assert np.array_equal(hm @ hm.T, h * np.eye(h))


def test_hadamard_rejects_other_orders():
    for h in (0, 3, 6, 96):
        with pytest.raises(ValueError):
            O.hadamard(h)


def test_worked_examples_order_two():
    r2 = np.sqrt(0.5)
    a, b = 0.75, -2.0
    ident = np.array([0, 1])
    plus = np.array([1, 1])
    got = O.rpbh_rotate([[a, b]], ident, plus, 2)[0]
    assert np.allclose(got, [(a + b) * r2, (a - b) * r2], rtol=0, atol=1e-15)
    # signs act after the permutation: first swap, then flip the new first entry
    got = O.rpbh_rotate([[a, b]], np.array([1, 0]), np.array([-1, 1]), 2)[0]
    assert np.allclose(got, [(-b + a) * r2, (-b - a) * r2], rtol=0, atol=1e-15)
    # two blocks of two: each block on its own
    got = O.rpbh_rotate([[1.0, 2.0, 3.0, 5.0]], np.arange(4), np.ones(4), 2)[0]
    assert np.allclose(got, [3 * r2, -1 * r2, 8 * r2, -2 * r2], rtol=0, atol=1e-15)


@pytest.mark.parametrize("d,h", [(64, 2), (64, 8), (64, 64), (96, 32)])
def test_rotation_is_orthogonal(d, h):
    perm, signs = synth.rpbh_draw(d, 1)
    p = O.rpbh_matrix(perm, signs, h)
    assert np.allclose(p @ p.T, np.eye(d), rtol=0, atol=1e-13)
    x = np.random.default_rng(2).normal(size=(5, d))
    assert np.allclose(np.linalg.norm(O.rpbh_rotate(x, perm, signs, h), axis=1),
                       np.linalg.norm(x, axis=1), rtol=1e-13)


def test_rotations_cancel_in_the_product():
    """[ORQ] §2.2: weights rotated offline, activations online, same product."""
    d, h = 256, 64
    perm, signs = synth.rpbh_draw(d, 3)
    rng = np.random.default_rng(4)
    x = rng.normal(size=(7, d))
    w = rng.normal(size=(11, d))
    y = O.rpbh_rotate(x, perm, signs, h) @ O.rpbh_rotate(w, perm, signs, h).T
    assert np.allclose(y, x @ w.T, rtol=0, atol=1e-12 * np.abs(x @ w.T).max())


def test_a_spike_spreads_over_one_block():
    """Pi_d e_k has h nonzero entries of magnitude 1/sqrt(h), all in the block
    holding position perm^-1(k)."""
    d, h = 128, 16
    perm, signs = synth.rpbh_draw(d, 5)
    for k in (0, 17, 127):
        e = np.zeros((1, d))
        e[0, k] = 1.0
        v = O.rpbh_rotate(e, perm, signs, h)[0]
        nz = np.nonzero(np.abs(v) > 1e-12)[0]
        b = int(np.nonzero(perm == k)[0][0]) // h
        assert np.array_equal(nz, np.arange(b * h, b * h + h))
        assert np.allclose(np.abs(v[nz]), 1.0 / np.sqrt(h), rtol=1e-14)


def test_rotation_helps_group_quantization_of_outlier_columns():
    """Weights with a few large input columns (the outlier structure of the
    low-rank workload) quantize much better in the rotated basis; the error is
    measured in the original basis (the rotation is orthogonal)."""
    rng = np.random.default_rng(6)
    w = rng.normal(0.0, 0.02, size=(128, 1024))
    w[:, rng.choice(1024, 8, replace=False)] *= 50.0
    w = synth.to_bf16(w)
    perm, signs = synth.rpbh_draw(1024, 7)
    wr = O.rpbh_rotate(w, perm, signs, 128).astype(np.float32)
    q_u, s = O.quantize_groups(w, 4)
    q_r, s_r = O.quantize_groups(wr, 4)
    snr_plain = O.snr_db(w, O.dequant_f32(q_u, s, 4))
    snr_rot = O.snr_db(wr, O.dequant_f32(q_r, s_r, 4))
    assert snr_rot > snr_plain + 3.0, (snr_plain, snr_rot)


def test_rotate_checks_shapes():
    perm, signs = synth.rpbh_draw(64, 1)
    with pytest.raises(ValueError):
        O.rpbh_rotate(np.zeros((2, 64)), perm, signs, 48)
    with pytest.raises(ValueError):
        O.rpbh_rotate(np.zeros((2, 64)), perm[:32], signs, 32)
