"""GPU parity of the RPBH rotation ([ORQ] §2.1, §2.2) against the oracle's
float64 rotation, and the rotated product end to end.

float32 outputs: per element |gpu - ref| <= (log2 h + 1) 2^-24 sum_block|x| / sqrt(h)
(each butterfly stage rounds once; partial sums never exceed the block's
absolute sum).  bf16 outputs: within one bf16 ulp of the float64 value, and
equal to its round-to-nearest-even in at least 99% of the elements (the rest
sit within float32 error of a bf16 rounding boundary)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from dit_dequant_gemm_amd import synth
from parity_util import check_product, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _draw(d, seed):
    perm, signs = synth.rpbh_draw(d, seed)
    return perm, signs, torch.from_numpy(perm).cuda(), torch.from_numpy(signs).cuda()


def _f32_bound(x, perm, signs, h):
    t = np.abs(np.asarray(x, dtype=np.float64)[:, perm])
    n, d = t.shape
    blk = t.reshape(n, d // h, h).sum(axis=2, keepdims=True)
    return np.broadcast_to((math.log2(h) + 1) * 2.0 ** -24 * blk / math.sqrt(h),
                           (n, d // h, h)).reshape(n, d) * 1.01 + 1e-37


def _check_f32(got, x, perm, signs, h):
    ref = O.rpbh_rotate(x, perm, signs, h)
    err = np.abs(got.astype(np.float64) - ref)
    bound = _f32_bound(x, perm, signs, h)
    assert np.all(err <= bound), float(np.max(err / bound))


def _check_bf16(got, x, perm, signs, h):
    ref = O.rpbh_rotate(x, perm, signs, h)
    ulp = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7        # one bf16 ulp (<= 2^-7 relative)
    assert np.all(np.abs(got - ref) <= ulp + _f32_bound(x, perm, signs, h))
    exact = np.mean(got == synth.to_bf16(ref))
    assert exact >= 0.99, exact


@pytest.mark.parametrize("n,d,h", [(5, 64, 2), (7, 256, 64), (3, 1024, 128), (9, 3072, 128),
                                   (2, 5120, 1024), (4, 16384, 256), (3, 13824, 512), (6, 384, 8)])
def test_rotate_f32(gpu_lib, n, d, h):
    _case(f"rpbh_rotate f32 n={n} d={d} h={h}")
    x = np.random.default_rng(d + h).normal(0, 1, size=(n, d)).astype(np.float32)
    perm, signs, pd, sd = _draw(d, h)
    got = host(gpu_lib.rpbh_rotate(dev_f32(x), pd, sd, h))
    _check_f32(got, x, perm, signs, h)


@pytest.mark.parametrize("h", [2, 32, 128, 1024])
def test_rotate_bf16_in_and_out(gpu_lib, h):
    _case(f"rpbh_rotate bf16 -> bf16 / f32, h={h}")
    n, d = 33, 2048
    x = synth.to_bf16(np.random.default_rng(h).normal(0, 1, size=(n, d)))
    perm, signs, pd, sd = _draw(d, 100 + h)
    _check_bf16(host(gpu_lib.rpbh_rotate(dev_bf16(x), pd, sd, h)), x, perm, signs, h)
    _check_f32(host(gpu_lib.rpbh_rotate(dev_bf16(x), pd, sd, h, out_dtype=torch.float32)),
               x, perm, signs, h)
    _check_bf16(host(gpu_lib.rpbh_rotate(dev_f32(x), pd, sd, h, out_dtype=torch.bfloat16)),
                x, perm, signs, h)


def test_rotate_in_place(gpu_lib):
    _case("rpbh_rotate in place")
    n, d, h = 17, 1536, 512
    x = np.random.default_rng(1).normal(0, 1, size=(n, d)).astype(np.float32)
    perm, signs, pd, sd = _draw(d, 2)
    t = dev_f32(x)
    out = gpu_lib.rpbh_rotate(t, pd, sd, h, out=t)
    assert out.data_ptr() == t.data_ptr()
    _check_f32(host(t), x, perm, signs, h)


def test_rotate_out_of_range_entries_read_zero(gpu_lib):
    _case("rpbh_rotate perm entries outside [0, d)")
    n, d, h = 3, 256, 16
    x = np.random.default_rng(3).normal(0, 1, size=(n, d)).astype(np.float32)
    perm, signs = synth.rpbh_draw(d, 4)
    bad = perm.copy()
    bad[[0, 5, 77, 255]] = [-1, d, 10 ** 6, -(10 ** 6)]
    valid = (bad >= 0) & (bad < d)
    t = np.where(valid[None, :], x[:, np.clip(bad, 0, d - 1)], 0.0) * np.where(signs < 0, -1.0, 1.0)
    ref = np.einsum("jt,nbt->nbj", O.hadamard(h) / np.sqrt(h), t.reshape(n, d // h, h)).reshape(n, d)
    got = host(gpu_lib.rpbh_rotate(dev_f32(x), torch.from_numpy(bad).cuda(),
                                   torch.from_numpy(signs).cuda(), h))
    assert np.allclose(got, ref, rtol=0, atol=1e-5)


def test_rotate_empty(gpu_lib):
    _case("rpbh_rotate n=0")
    pd = torch.arange(128, dtype=torch.int32, device="cuda")
    sd = torch.ones(128, dtype=torch.int8, device="cuda")
    out = gpu_lib.rpbh_rotate(torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"), pd, sd, 128)
    assert out.shape == (0, 128)


def test_rotate_attention_projection_activations_sampled(gpu_lib):
    """The bench's activation rotation (4096 x 3072 bf16, h = 128) on sampled rows."""
    _case("rpbh_rotate 4096 x 3072 bf16, h=128 (sampled rows)")
    c = synth.config2()
    perm, signs, pd, sd = _draw(3072, 9)
    got = host(gpu_lib.rpbh_rotate(dev_bf16(c["x"]), pd, sd, 128))
    rows = np.r_[0:64, 2000:2064, 4032:4096]
    _check_bf16(got[rows], c["x"][rows], perm, signs, 128)


@pytest.mark.parametrize("bits", [3, 4, 6])
def test_rotated_product_end_to_end(gpu_lib, bits):
    """Weights rotated (float32) then quantized, activations rotated (bf16),
    then the dequant-GEMM: against the oracle's chain on the same inputs."""
    _case(f"rotated W4-style product, bits={bits}")
    m, n, k, h = 96, 384, 1024, 128
    rng = np.random.default_rng(bits)
    w = rng.normal(0, 0.02, size=(n, k))
    w[:, rng.choice(k, 6, replace=False)] *= 40.0             # outlier input columns
    w = synth.to_bf16(w)
    x = synth.to_bf16(rng.normal(0, 1, size=(m, k)))
    perm, signs, pd, sd = _draw(k, 20 + bits)
    wr = gpu_lib.rpbh_rotate(dev_bf16(w), pd, sd, h, out_dtype=torch.float32)
    qw = gpu_lib.quantize_pack(wr, bits)
    xr = gpu_lib.rpbh_rotate(dev_bf16(x), pd, sd, h)
    y = host(gpu_lib.dequant_gemm(xr, qw, torch.float32))
    wr_ref = O.rpbh_rotate(w, perm, signs, h).astype(np.float32)
    xr_ref = synth.to_bf16(O.rpbh_rotate(x, perm, signs, h))
    q_u, s = O.quantize_groups(wr_ref, bits)
    y_ref = O.gemm_ref(xr_ref, O.dequant_bf16(q_u, s, bits))
    check_product(y, y_ref, False, f"rotated product bits={bits}")


@pytest.mark.parametrize("n,d,h,f32", [(600, 16384, 64, False), (520, 16384, 64, True),
                                       (9000, 256, 16, False), (700, 13824, 128, True)])
def test_rotate_several_rows_per_wave(gpu_lib, n, d, h, f32):
    """Row counts above the resident waves: each wave rotates several rows,
    loading the next while it computes (two row buffers), or one after the
    other where two float32 rows do not fit next to the table."""
    _case(f"rpbh_rotate n={n} d={d} h={h} f32={f32} (several rows per wave)")
    rng = np.random.default_rng(n + d)
    x = rng.normal(0, 1, size=(n, d)).astype(np.float32)
    if not f32:
        x = synth.to_bf16(x)
    perm, signs, pd, sd = _draw(d, n)
    xd = dev_f32(x) if f32 else dev_bf16(x)
    got = host(gpu_lib.rpbh_rotate(xd, pd, sd, h, out_dtype=torch.float32))
    rows = np.r_[0:8, n // 2:n // 2 + 8, n - 8:n]
    _check_f32(got[rows], x[rows], perm, signs, h)
    # every row, through a cheaper exact property: the rotation keeps each row's norm
    nx = np.linalg.norm(x.astype(np.float64), axis=1)
    assert np.allclose(np.linalg.norm(got.astype(np.float64), axis=1), nx, rtol=2e-6)
