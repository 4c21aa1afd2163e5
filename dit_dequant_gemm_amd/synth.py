"""Seeded synthetic inputs for the DiT linear-layer workloads.

This module only draws random numbers and rounds them to bf16; it holds none
of the quantization or matmul arithmetic.  Both the HIP path (bench, binding
tests) and the CPU oracle's tests take their inputs from here.

Every array comes from ``numpy.random.default_rng(seed)`` with a seed list
``[config, stream]`` so that any one array can be drawn without drawing the
others (config 1 uses the single seed 0 and the draw order W, outlier columns,
X).  "bf16" means: float64 draw -> float32 (round to nearest) -> bf16 (round to
nearest, ties to even), returned as float32 arrays holding bf16-exact values.

Workloads (shapes are out x in for weights, tokens x in for activations):

1. single linear: W 256x512 ~ N(0, 0.02^2), 4 input columns x20; X 64x512
   ~ N(0, 1); 4-bit.
2. DiT attention projection: W 3072x3072 ~ N(0, 0.02^2); X 4096x3072 ~ N(0,1)
   (the M=16 variant is its first 16 rows); 4-bit.
3. DiT MLP pair: up 12288x3072 and down 3072x12288, 0.02 * t(4) / sqrt(2)
   (unit-variance Student-t with 4 degrees of freedom, std 0.02); X_up
   4096x3072, X_down 4096x12288 ~ N(0, 1); each at 3/5/6/7 bit.
4. outlier absorption: W 3072x3072 = N(0, 0.02^2) + a rank-8 term of entry
   RMS 1.0 on 16 fixed input channels C; X 4096x3072 ~ N(0, 1) with the same
   16 channels x30; rank-32 branch, 4-bit residual.
5. Wan-14B-shaped block: qkv 15360x5120, o 5120x5120, up 13824x5120,
   down 5120x13824 ~ N(0, 0.02^2); per-tensor bits drawn with probabilities
   3:0.002, 4:0.21, 5:0.55, 6:0.23, 7:0.008; X of M in {16, 32760} tokens.
"""
from __future__ import annotations

import numpy as np

__all__ = ["to_bf16", "config1", "config2", "config3", "config4", "config5_weights",
           "config5_bits", "config5_x", "C5_SHAPES", "C5_BIT_CHOICES", "C5_BIT_PROBS",
           "random_case", "rpbh_draw"]


def to_bf16(a) -> np.ndarray:
    """float64/float32 -> float32 (nearest) -> bf16 (nearest even), as float32."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    # add 0x7FFF plus the lowest kept bit, then truncate: round half to even
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def _rng(config: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([config, stream])


def _normal_rows(rng, rows, cols, std=1.0, chunk=4096):
    """N(0, std^2) draws in row chunks (float64 -> bf16 per chunk), bounded memory."""
    out = np.empty((rows, cols), dtype=np.float32)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        out[r0:r1] = to_bf16(rng.normal(0.0, std, size=(r1 - r0, cols)))
    return out


def config1():
    """Single linear (256x512, 4 outlier input columns x20), X 64x512, seed 0."""
    rng = np.random.default_rng(0)
    w = rng.normal(0.0, 0.02, size=(256, 512))
    cols = rng.choice(512, size=4, replace=False)
    w[:, cols] *= 20.0
    x = rng.normal(0.0, 1.0, size=(64, 512))
    return {"w": to_bf16(w), "x": to_bf16(x), "bits": 4, "outlier_cols": np.sort(cols)}


def config2(m: int = 4096):
    """Attention projection 3072x3072; X has ``m`` rows (<= 4096; 16 for the M=16 variant)."""
    if not 1 <= m <= 4096:
        raise ValueError("m must be in [1, 4096]")
    w = _normal_rows(_rng(2, 0), 3072, 3072, 0.02)
    x = _normal_rows(_rng(2, 1), 4096, 3072)[:m]
    return {"w": w, "x": x, "bits": 4}


def _student_t_weight(rng, rows, cols, chunk=2048):
    out = np.empty((rows, cols), dtype=np.float32)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        t = rng.standard_t(4, size=(r1 - r0, cols))
        out[r0:r1] = to_bf16(0.02 * t / np.sqrt(2.0))
    return out


def config3(which: str = "up", m: int = 4096):
    """MLP pair: which in {"up", "down"}; returns W, X (m rows) and the bit sweep."""
    if which == "up":
        w = _student_t_weight(_rng(3, 0), 12288, 3072)
        x = _normal_rows(_rng(3, 2), 4096, 3072)[:m]
    elif which == "down":
        w = _student_t_weight(_rng(3, 1), 3072, 12288)
        x = _normal_rows(_rng(3, 3), 4096, 12288)[:m]
    else:
        raise ValueError(which)
    return {"w": w, "x": x, "bits_sweep": (3, 5, 6, 7)}


def config4(m: int = 4096):
    """Outlier absorption: W = noise + rank-8 outliers on 16 channels; X with x30 channels."""
    rng = _rng(4, 0)
    noise = rng.normal(0.0, 0.02, size=(3072, 3072))
    chans = np.sort(rng.choice(3072, size=16, replace=False))
    a = rng.normal(0.0, 1.0, size=(3072, 8))
    b = rng.normal(0.0, 1.0, size=(8, 16))
    outl = np.zeros((3072, 3072))
    outl[:, chans] = (a @ b) / np.sqrt(8.0)
    w = to_bf16(noise + outl)
    xr = _rng(4, 1)
    x = np.empty((4096, 3072), dtype=np.float32)
    for r0 in range(0, 4096, 1024):
        blk = xr.normal(0.0, 1.0, size=(1024, 3072))
        blk[:, chans] *= 30.0
        x[r0:r0 + 1024] = to_bf16(blk)
    return {"w": w, "x": x[:m], "bits": 4, "rank": 32, "channels": chans}


C5_SHAPES = {            # name: (out, in)
    "qkv": (15360, 5120),
    "o": (5120, 5120),
    "up": (13824, 5120),
    "down": (5120, 13824),
}
C5_BIT_CHOICES = (3, 4, 5, 6, 7)
C5_BIT_PROBS = (0.002, 0.21, 0.55, 0.23, 0.008)
_C5_STREAM = {"qkv": 0, "o": 1, "up": 2, "down": 3}


def config5_weights(name: str, rows=None):
    """One Wan-14B block weight (optionally only its first ``rows`` rows)."""
    n, k = C5_SHAPES[name]
    rows = n if rows is None else rows
    return _normal_rows(_rng(5, _C5_STREAM[name]), rows, k, 0.02)


def config5_bits():
    """Per-tensor bit widths drawn with the block's shares (order qkv, o, up, down)."""
    rng = _rng(5, 100)
    b = rng.choice(C5_BIT_CHOICES, size=4, p=C5_BIT_PROBS)
    return dict(zip(("qkv", "o", "up", "down"), (int(v) for v in b)))


def config5_x(name: str, m: int, rows=None):
    """Activations for block weight ``name`` with ``m`` tokens (first ``rows`` only)."""
    _, k = C5_SHAPES[name]
    rows = m if rows is None else rows
    stream = 10 + 2 * _C5_STREAM[name] + (0 if m == 16 else 1)
    return _normal_rows(_rng(5, stream), rows, k)


def random_case(seed: int, m: int, n: int, k: int, wstd: float = 0.02):
    """Small seeded case for fuzzing: W n x k ~ N(0, wstd^2), X m x k ~ N(0, 1)."""
    rng = np.random.default_rng([99, seed])
    return {"w": to_bf16(rng.normal(0.0, wstd, size=(n, k))),
            "x": to_bf16(rng.normal(0.0, 1.0, size=(m, k)))}


def rpbh_draw(d: int, seed: int):
    """The random draws of a rotation over d coordinates: a permutation of
    0..d-1 (int32) and Rademacher signs +-1 (int8)."""
    rng = np.random.default_rng([77, seed, d])
    perm = rng.permutation(d).astype(np.int32)
    signs = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    return perm, signs
