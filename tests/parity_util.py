"""Shared helpers for the GPU parity tests (test code only)."""
import numpy as np
import torch

import oracle as O

REL_FRO = 1e-3      # relative Frobenius error bound of the product
ROW_MAX = 2e-2      # per-row max-abs error, relative to the row's max |Y_ref|


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda", torch.bfloat16)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_product(y_gpu, y_ref64, out_bf16: bool, what: str = ""):
    """The bar: relative Frobenius <= 1e-3 and per-row max-abs <= 2e-2 * row max.

    For a bf16 output the reference is bf16_RNE(fl32(Y_ref)), same bounds."""
    y = np.asarray(y_gpu, dtype=np.float64)
    ref = np.asarray(y_ref64, dtype=np.float64)
    if out_bf16:
        ref = O.bf16_rne(ref.astype(np.float32)).astype(np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    den = np.linalg.norm(ref)
    rel = np.linalg.norm(y - ref) / den if den > 0 else np.linalg.norm(y)
    rmax = np.max(np.abs(ref), axis=1)
    rerr = np.max(np.abs(y - ref), axis=1)
    worst = float(np.max(rerr / np.where(rmax > 0, rmax, 1.0)))
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3e}"
    assert worst <= ROW_MAX, f"{what}: worst row max-abs ratio {worst:.3e}"
    return rel, worst


def sample_rows(m: int, seed: int, count: int = 128, tail: int = 64):
    """Sorted row indices: the first rows, random interior rows and the last
    `tail` rows (so ragged last tiles are always covered)."""
    rng = np.random.default_rng(seed)
    head = np.arange(min(m, 32))
    last = np.arange(max(0, m - tail), m)
    mid = rng.choice(m, size=min(m, count), replace=False)
    return np.unique(np.concatenate([head, mid, last]))


def sample_weight_rows(n: int, seed: int, count: int = 96):
    rng = np.random.default_rng(seed + 1000)
    return np.unique(np.concatenate([np.arange(min(n, 16)), rng.choice(n, size=min(n, count), replace=False),
                                     np.arange(max(0, n - 16), n)]))
