"""Plain, slow, obviously-correct CPU oracle for the low-bit dequant-GEMM path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never links, imports or executes it, and it shares no code with the
HIP library: it reads no header, table or helper of the product.

Sources (cited by title and section only):

* [WDQ]  The Wan-Dancer-14B mixed-precision quantization report
  (www.mtrt.cn, news 3666).
  - §3.1 "Per-Group(128) symmetric quantization": groups of 128 consecutive
    weights along the input dimension, abs-max times 1.01, step = 2*abs_max /
    (2^bits - 1), codes rounded and clamped to +-n_half.
  - §3.1 comparison table: per-channel vs per-group scale counts.
  - §2.1 table: typical SNR per-tensor < per-channel < per-group.
  - §3.3 "Multi-Bit Packed Storage": table of weights per byte group
    (3b: 8->3 B, 4b: 2->1 B, 5b: 8->5 B, 6b: 4->3 B, 7b: 8->7 B) and the 4-bit
    pack/unpack pseudo-code (even-index code in the high nibble).
  - §3.3 storage format: packed uint8, float32 per-group scales, int8 bit
    width, int32 padded input dimension.
  - §3.4 "GPU-Native Dequantize": unsigned code minus n_half, times the group
    scale, in float32.
  - §5.3 / §5.4: the page's forward dequantizes and then runs a bf16 matmul.
* [SVDQ] "SVDQuant：4-bit量化让扩散模型在消费级GPU上高效运行" (www.kongchang.com).
  - section on why diffusion models are hard to quantize: an outlier of 100
    among values in [-1, 1] makes 4-bit levels useless for the normal values.
  - section "SVDQuant 的核心思路": W = U S V^T, the top-k singular triplets give
    the best rank-k approximation.
  - section "技术原理详解": a 16-bit low-rank branch takes the outliers, the
    residual is quantized to 4 bit.

Readings where the pages are silent or garbled:

R1  n_half = 2^(bits-1) - 1 (the clamp bound, also the unsigned offset).
R2  All arithmetic of the quantizer is IEEE float32: abs-max (exact),
    a1 = fl32(a * fl32(1.01)), step = fl32(2*a1 / (2^bits - 1)) with a correctly
    rounded division, r = fl32(w / step) correctly rounded, q = round-half-even(r).
R3  An all-zero group (step == 0) gets code 0 (q_u = n_half) and scale 0.
R4  Codes of bits b in {3,5,6,7} are packed as one continuous MSB-first
    bitstream over the row-major flattened codes; this is the only
    generalisation that reproduces the 4-bit rule of §3.3.  Beyond 4 bit the
    pages fix only the byte count, so this is a convention ("parity unpinned"
    by the pages beyond size and round trip).
R5  The weights fed to the matmul are bf16_RNE(fl32(q * scale)) (dequantize in
    float32 as §3.4, then a bf16 matmul as §5.4).
R6  The low-rank intermediate is T = bf16_RNE(fl32(X @ L1)); the branch adds
    T @ L2.  L1 = V_r sqrt(S_r) (in x r), L2 = sqrt(S_r) U_r^T (r x out), both
    rounded to bf16; the residual R = fl32(W - (L1 @ L2)^T) absorbs the
    rounding of the factors.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "GROUP", "SUPPORTED_BITS", "MULT_1P01", "n_half",
    "bf16_rne", "quantize", "quantize_groups", "pack_codes", "unpack_codes",
    "packed_nbytes", "dequant_f32", "dequant_bf16", "dequant_from_packed",
    "gemm_ref", "lowrank_t_ref", "lowrank_fused_ref", "svd_split", "snr_db",
    "quantize_pack",
]

GROUP = 128                      # [WDQ] §3.1: 128 consecutive weights share a scale
SUPPORTED_BITS = (3, 4, 5, 6, 7)  # [WDQ] §3.3 table
MULT_1P01 = np.float32(1.01)     # nearest float32 to 1.01 (0x3F8147AE), reading R2


def n_half(bits: int) -> int:
    """Largest code magnitude, 2^(bits-1) - 1 (reading R1)."""
    return (1 << (bits - 1)) - 1


def _check_bits(bits: int) -> None:
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"bits must be one of {SUPPORTED_BITS}, got {bits}")


# --------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even) of float32 values
# --------------------------------------------------------------------------
def bf16_rne(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returned as float32 holding bf16-exact values.  Finite input only.
    Written from the definition: keep the top 16 bits of the float32 pattern,
    look at the dropped 16 bits, round up if they exceed half, or equal half
    and the kept pattern is odd.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_rne: finite input only")
    u = x.view(np.uint32)
    keep = u >> np.uint32(16)
    dropped = u & np.uint32(0xFFFF)
    half = np.uint32(0x8000)
    round_up = (dropped > half) | ((dropped == half) & ((keep & np.uint32(1)) == 1))
    keep = keep + round_up.astype(np.uint32)
    return (keep << np.uint32(16)).astype(np.uint32).view(np.float32)


# --------------------------------------------------------------------------
# Quantizer: [WDQ] §3.1 (per group of 128 along the input dimension)
# --------------------------------------------------------------------------
def quantize(w, bits: int, granularity: str = "group", group: int = GROUP):
    """Symmetric abs-max quantizer of [WDQ] §3.1 at a chosen scale granularity.

    ``granularity``: "group" (128 consecutive inputs, the method), "channel"
    (one scale per output row) or "tensor" (one scale) -- the last two are the
    coarser variants [WDQ] §2.1 compares against.

    Returns ``(q_u, scales)``: unsigned codes (uint8, shape of ``w``) in
    [0, 2^bits - 2] and float32 scales of shape (rows, groups_per_row); for
    "tensor" the scale array has shape (1, 1).
    """
    _check_bits(bits)
    w32 = np.ascontiguousarray(w, dtype=np.float32)
    if w32.ndim != 2:
        raise ValueError("w must be 2-D (out x in)")
    if not np.all(np.isfinite(w32)):
        raise ValueError("finite weights only")
    n, k = w32.shape
    if granularity == "group":
        if k % group:
            raise ValueError("in-dimension must be a multiple of the group size")
        wg = w32.reshape(n, k // group, group)
    elif granularity == "channel":
        wg = w32.reshape(n, 1, k)
    elif granularity == "tensor":
        wg = w32.reshape(1, 1, n * k)
    else:
        raise ValueError(granularity)

    # step 2: abs-max of each group, exact in float32
    a = np.max(np.abs(wg), axis=-1)
    # step 3: times fl32(1.01), one float32 rounding
    a1 = a * MULT_1P01
    # step 4: step = 2*a1 / (2^bits - 1); 2*a1 is exact, the division rounds once
    step = (np.float32(2.0) * a1) / np.float32((1 << bits) - 1)
    assert step.dtype == np.float32
    nh = n_half(bits)
    # step 6: r = fl32(w / step), round half to even, clamp to +-n_half
    with np.errstate(divide="ignore", invalid="ignore"):
        r = wg / step[..., None]
    assert r.dtype == np.float32
    q = np.rint(r)
    q = np.clip(q, -nh, nh)
    # step 5 (reading R3): an all-zero group (or a step that underflows to 0)
    q = np.where(step[..., None] == 0, np.float32(0), q)
    # step 7: unsigned code
    q_u = (q.astype(np.int32) + nh).astype(np.uint8).reshape(n, k)
    return q_u, step.astype(np.float32)


def quantize_groups(w, bits: int, group: int = GROUP):
    """Per-group(128) quantizer of the method: ``(q_u, scales (N, K/128))``."""
    return quantize(w, bits, "group", group)


# --------------------------------------------------------------------------
# Packing: [WDQ] §3.3 (byte counts, 4-bit nibble order) + reading R4
# --------------------------------------------------------------------------
def packed_nbytes(n: int, k: int, bits: int) -> int:
    """Bytes of the packed stream: n*k*bits/8 ([WDQ] §3.3 table)."""
    _check_bits(bits)
    total_bits = n * k * bits
    if total_bits % 8:
        raise ValueError("n*k*bits must be a multiple of 8")
    return total_bits // 8


def pack_codes(q_u, bits: int) -> np.ndarray:
    """MSB-first continuous bitstream of the row-major flattened codes.

    Bit 0 of the stream is the most significant bit of byte 0.  For bits=4 the
    even-index code lands in the high nibble, as the 4-bit pseudo-code of
    [WDQ] §3.3 does.
    """
    _check_bits(bits)
    codes = np.ascontiguousarray(q_u, dtype=np.uint8).reshape(-1)
    if codes.size * bits % 8:
        raise ValueError("code count * bits must be a multiple of 8")
    if codes.size and int(codes.max()) >= (1 << bits):
        raise ValueError("code does not fit in the bit width")
    # one row of 8 bits per code, most significant first; keep the low `bits`
    per_code = np.unpackbits(codes[:, None], axis=1, bitorder="big")[:, 8 - bits:]
    return np.packbits(per_code.reshape(-1), bitorder="big")


def unpack_codes(packed, bits: int, count: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`: the first ``count`` codes as uint8."""
    _check_bits(bits)
    stream = np.unpackbits(np.ascontiguousarray(packed, dtype=np.uint8), bitorder="big")
    if stream.size < count * bits:
        raise ValueError("packed stream too short")
    fields = stream[: count * bits].reshape(count, bits).astype(np.uint16)
    weights = (1 << np.arange(bits - 1, -1, -1)).astype(np.uint16)
    return (fields * weights).sum(axis=1).astype(np.uint8)


def quantize_pack(w, bits: int):
    """The whole offline step: ``(packed uint8, scales float32, q_u)``."""
    q_u, scales = quantize_groups(w, bits)
    return pack_codes(q_u, bits), scales, q_u


# --------------------------------------------------------------------------
# Dequantization: [WDQ] §3.4, and reading R5 for what the matmul consumes
# --------------------------------------------------------------------------
def dequant_f32(q_u, scales, bits: int) -> np.ndarray:
    """w_hat = fl32((q_u - n_half) * scale) for every weight ([WDQ] §3.4).

    ``scales`` has shape (rows, groups_per_row) -- (N, K/128) for the method,
    (N, 1) per-channel, (1, 1) per-tensor; each scale covers K/groups_per_row
    consecutive inputs of its row (every weight for the (1, 1) case).
    """
    _check_bits(bits)
    q_u = np.asarray(q_u, dtype=np.uint8)
    n, k = q_u.shape
    scales = np.asarray(scales, dtype=np.float32)
    q = (q_u.astype(np.int32) - n_half(bits)).astype(np.float32)   # exact
    if scales.shape == (1, 1):
        out = q * scales[0, 0]
    else:
        rows, groups = scales.shape
        if rows != n or k % groups:
            raise ValueError("scales shape does not match the codes")
        out = (q.reshape(n, groups, k // groups) * scales[:, :, None]).reshape(n, k)
    assert out.dtype == np.float32        # one float32 rounding per product
    return out


def dequant_bf16(q_u, scales, bits: int) -> np.ndarray:
    """bf16_RNE(fl32((q_u - n_half) * scale)): the matmul operand (reading R5)."""
    return bf16_rne(dequant_f32(q_u, scales, bits))


def dequant_from_packed(packed, scales, bits: int, n: int, k: int) -> np.ndarray:
    """Unpack then dequantize to the bf16-valued matmul operand (N x K)."""
    q_u = unpack_codes(packed, bits, n * k).reshape(n, k)
    return dequant_bf16(q_u, scales, bits)


# --------------------------------------------------------------------------
# Contractions: float64 reference of Y = X @ w_hat^T (+ T @ L2)
# --------------------------------------------------------------------------
def gemm_ref(x, w_hat) -> np.ndarray:
    """Y = X @ w_hat^T in float64 (X is M x K, w_hat is N x K)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_hat, dtype=np.float64).T


def lowrank_t_ref(x, l1) -> np.ndarray:
    """T = bf16_RNE(fl32(X @ L1)) -- the bf16 low-rank intermediate (reading R6)."""
    t64 = np.asarray(x, dtype=np.float64) @ np.asarray(l1, dtype=np.float64)
    return bf16_rne(t64.astype(np.float32))


def lowrank_fused_ref(x, w_hat, l1, l2):
    """Y = X @ w_hat^T + T @ L2 in float64 with T = bf16(X @ L1); returns (Y, T)."""
    t = lowrank_t_ref(x, l1)
    y = gemm_ref(x, w_hat) + t.astype(np.float64) @ np.asarray(l2, dtype=np.float64)
    return y, t


def svd_split(w, r: int):
    """Rank-r SVD split of [SVDQ] (reading R6).

    Returns ``(L1 (K x r), L2 (r x N), R (N x K))``: L1, L2 as float32 arrays
    holding bf16 values, R = fl32(W - (L1 @ L2)^T) the float32 residual.
    """
    w64 = np.asarray(w, dtype=np.float64)
    u, s, vt = np.linalg.svd(w64, full_matrices=False)
    root = np.sqrt(s[:r])
    l1 = bf16_rne((vt[:r].T * root).astype(np.float32))          # in x r
    l2 = bf16_rne((root[:, None] * u[:, :r].T).astype(np.float32))  # r x out
    resid = (w64 - (l1.astype(np.float64) @ l2.astype(np.float64)).T).astype(np.float32)
    return l1, l2, resid


def snr_db(w, w_hat) -> float:
    """10*log10(sum w^2 / sum (w - w_hat)^2), in float64."""
    w = np.asarray(w, dtype=np.float64)
    e = w - np.asarray(w_hat, dtype=np.float64)
    den = float(np.sum(e * e))
    num = float(np.sum(w * w))
    if den == 0.0:
        return float("inf")
    return 10.0 * np.log10(num / den)
