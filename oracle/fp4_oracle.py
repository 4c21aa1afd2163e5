"""CPU oracle for the FP4-weight / FP8-activation (W4A8) product.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module; the
product (libddg.so) shares no code with it.

Source: [FP4] the FP4DiT article (aijishu.com).
  - §3.1.2: floating-point quantization -- the exponent picks a range, the
    mantissa gives uniform levels inside it.
  - §3.2.1 / §4.1: 4-bit weight formats E2M1, E3M0 (denser near zero, for the
    first linear of the pointwise feed-forward network) and E1M2; weight groups
    of 128.
  - §3.2.3 / §4.1: per-token online min-max activation quantization to 8 bits
    (W4A8) and 6 bits (W4A6); §3.3: FP6 saves memory over FP8.

Readings where the article is silent:

R18  The 4-bit formats are sign + magnitude minifloats, subnormal when the
     exponent field is 0: E2M1 bias 1 (0, .5, 1, 1.5, 2, 3, 4, 6), E1M2 bias 1
     (0, .25, .5, .75, 1, 1.25, 1.5, 1.75), E3M0 bias 3 (0, 2^-2 .. 2^4).  Code =
     sign << 3 | magnitude index; a zero magnitude is always code 0.
R19  Weight groups are 128 consecutive weights along the input dimension (as the
     integer path; the article's "along the output channel" is garbled next to
     its group size and the storage of [WDQ]).  Scale s = fl32(amax / vmax),
     r = fl32(w / s) (correctly rounded division), code = the nearest format value
     to |r|, ties to the even code; an all-zero group gets scale 0 and code 0.
R20  The 8-bit activations are FP8 E4M3 (bias 7, largest 448, no infinities),
     the 8-bit format of the MFMA that takes FP4 operands; per token (row)
     s_x = fl32(amax / 448), r = fl32(x / s_x), q = E4M3 round-to-nearest-even
     of r (|r| clamped to 448 first); an all-zero row gets scale 0 and zeros.
R21  Packing: two codes per byte, the even index in the low nibble (the operand
     order of the gfx950 FP4 matrix instructions), rows of k/2 bytes.
R22  The product: Y[m, n] = s_x[m] * sum_g s_w[n, g] * sum_{k in g} q_x[m, k] v_w[n, k],
     q_x and v_w the exact E4M3 and FP4 values.
R24  Tiled storage (an option of this implementation, not of the article): the
     same codes and scales, reordered for the matrix instructions.  Columns
     are taken in blocks of 32 (the last padded with zero codes and zero
     scales); block b, group g is 2048 contiguous bytes: byte 1024 s + 512 h +
     16 j + t holds byte 32 s + 16 h + t of column 32 b + j's 64-byte slice of
     group g (rows of R21).  Blocks are ordered (b, g).  Scales: 32 floats per
     (b, g), column 32 b + j at position j.
R25  The 6-bit activations (W4A6) are FP6, E2M3 (bias 1, largest 7.5) or E3M2
     (bias 3, largest 28), sign + magnitude, subnormal when the exponent field
     is 0, no infinities; per token as R20 with 7.5 or 28 in place of 448.
R26  FP6 storage (an option of this implementation: the article fixes none):
     rows padded to a multiple of 32 with zero codes; for row block b (32
     rows), group g, 64-wide step s, half h (k = 128 g + 64 s + 32 h + j, j <
     32) the 32 codes form a 192-bit little-endian string, code j at bits 6 j;
     its 8-byte piece u (bits 64 u ..) of row 32 b + r sits at byte
     ((s * 2 + h) * 3 + u) * 256 + 8 r of record (b, g), 3072 bytes, records
     ordered (b, g).
R23  Power-of-two scale mode (the scale format the matrix instructions apply
     themselves, E8M0): s = the smallest power of two >= fl32(amax / vmax), and at
     least 2^-126; then as R19 with that s.  Every code stays within the format's
     range, at the cost of up to one bit of it.
R27  FP6 weights (a width the article names for activations only: §3.3's FP6
     saves memory over FP8, §4.1's W4A6; this implementation also offers it for
     weights): R25's formats E2M3 / E3M2 per group of 128 along the input
     dimension, scale and rounding as R19 with 7.5 or 28 as vmax (R23 with
     pow2); code = sign << 5 | magnitude index.  Storage: the codes in R26's
     layout with the weight's rows (output channels) in place of tokens, the
     scales tiled as R24's (32 per (column block, group)).
R28  W6A8: Y[m, n] = s_x[m] * sum_g s_w[n, g] * sum_{k in g} q_x[m, k] v_w[n, k],
     q_x the E4M3 activations of R20, v_w the FP6 weight values.
"""
from __future__ import annotations

import numpy as np

__all__ = ["FP4_FORMATS", "fp4_values", "minifloat_value", "quantize_fp4_groups", "pack_fp4",
           "unpack_fp4", "fp4_decode", "e4m3_values", "e4m3_round", "e4m3_decode",
           "quantize_rows_e4m3", "w4a8_ref", "tile_fp4", "untile_fp4", "FP6_FORMATS", "fp6_values",
           "quantize_rows_fp6", "fp6_decode", "pack_fp6_tiled", "unpack_fp6_tiled", "w4a6_ref",
           "quantize_fp6_groups", "tile_group_scales", "untile_group_scales", "w6a8_ref"]

FP4_FORMATS = {"e2m1": (2, 1, 1), "e3m0": (3, 0, 3), "e1m2": (1, 2, 1)}   # ebits, mbits, bias
FP6_FORMATS = {"e2m3": (2, 3, 1), "e3m2": (3, 2, 3)}
GROUP = 128
E4M3_MAX = 448.0


def minifloat_value(code: int, ebits: int, mbits: int, bias: int) -> float:
    """Value of a sign + magnitude minifloat code (subnormal when the exponent field is 0)."""
    sign = -1.0 if (code >> (ebits + mbits)) & 1 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        return sign * (m / float(1 << mbits)) * 2.0 ** (1 - bias)
    return sign * (1.0 + m / float(1 << mbits)) * 2.0 ** (e - bias)


def fp4_values(fmt: str) -> np.ndarray:
    """The 8 magnitudes of a 4-bit format, by magnitude index (R18)."""
    eb, mb, bias = FP4_FORMATS[fmt]
    return np.array([minifloat_value(i, eb, mb, bias) for i in range(8)], dtype=np.float64)


def fp4_decode(codes, fmt: str) -> np.ndarray:
    mag = fp4_values(fmt)[np.asarray(codes) & 7]
    return np.where(np.asarray(codes) & 8, -mag, mag)


def _nearest_index(mag_r, levels):
    """Index of the level nearest each |r| (levels ascending), ties to the even index."""
    mag_r = np.asarray(mag_r, dtype=np.float64)
    idx = np.searchsorted(levels, mag_r, side="left")          # levels[idx-1] < r <= levels[idx]
    idx = np.clip(idx, 1, len(levels) - 1)
    lo, hi = levels[idx - 1], levels[idx]
    dlo, dhi = mag_r - lo, hi - mag_r
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (idx % 2 == 0))
    out = np.where(pick_hi, idx, idx - 1)
    out = np.where(mag_r >= levels[-1], len(levels) - 1, out)
    return out


def _pow2_at_least(s):
    """Smallest power of two >= s (float32 s > 0), at least 2^-126 (R23)."""
    s = np.asarray(s, dtype=np.float32)
    m, e = np.frexp(s.astype(np.float64))            # s = m 2^e, m in [0.5, 1)
    p = np.where(m == 0.5, np.ldexp(1.0, e - 1), np.ldexp(1.0, e))
    return np.maximum(p, 2.0 ** -126).astype(np.float32)


def quantize_fp4_groups(w, fmt: str, pow2: bool = False):
    """(codes n x k uint8 in 0..15, scales n x k/128 float32) per R19 (R23 with pow2)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    levels = fp4_values(fmt)
    vmax = np.float32(levels[-1])
    g = w.reshape(n, k // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = (amax / vmax).astype(np.float32)
        if pow2:
            s = np.where(s > 0, _pow2_at_least(np.where(s > 0, s, 1.0)), np.float32(0)).astype(np.float32)
        r = (g / s[:, :, None]).astype(np.float32)
    zero = s[:, :, None] == 0
    r = np.where(zero, np.float32(0), r)
    idx = _nearest_index(np.abs(r), levels)
    codes = np.where((idx > 0) & (r < 0), idx | 8, idx).astype(np.uint8)
    return codes.reshape(n, k), s


def pack_fp4(codes) -> np.ndarray:
    """Rows of k codes -> rows of k/2 bytes, even index in the low nibble (R21)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def tile_fp4(packed, scales):
    """Row storage (n x k/2 bytes, n x k/128 scales) -> tiled storage (R24):
    (flat bytes of ceil(n/32) * G * 2048, flat floats of ceil(n/32) * G * 32)."""
    p = np.asarray(packed, dtype=np.uint8)
    sc = np.asarray(scales, dtype=np.float32)
    n, kb = p.shape
    g = kb // 64
    nb = -(-n // 32)
    pp = np.zeros((nb * 32, kb), dtype=np.uint8)
    pp[:n] = p
    ss = np.zeros((nb * 32, g), dtype=np.float32)
    ss[:n] = sc
    # axes of a row slice: block b, column j, group g, step s, half h, byte t
    t = pp.reshape(nb, 32, g, 2, 2, 16).transpose(0, 2, 3, 4, 1, 5)
    return t.reshape(-1).copy(), ss.reshape(nb, 32, g).transpose(0, 2, 1).reshape(-1).copy()


def untile_fp4(tiled, tscales, n: int, k: int):
    """Inverse of tile_fp4 (padding dropped)."""
    g = k // GROUP
    nb = -(-n // 32)
    t = np.asarray(tiled, dtype=np.uint8).reshape(nb, g, 2, 2, 32, 16).transpose(0, 4, 1, 2, 3, 5)
    s = np.asarray(tscales, dtype=np.float32).reshape(nb, g, 32).transpose(0, 2, 1)
    return t.reshape(nb * 32, k // 2)[:n].copy(), s.reshape(nb * 32, g)[:n].copy()


def e4m3_values() -> np.ndarray:
    """All finite E4M3 magnitudes (codes 0..126), ascending (bias 7; 127 is NaN)."""
    return np.array([minifloat_value(c, 4, 3, 7) for c in range(127)], dtype=np.float64)


def e4m3_round(r) -> np.ndarray:
    """E4M3 codes (uint8) of float32 values: clamp to +-448, round to nearest even (R20)."""
    r = np.asarray(r, dtype=np.float64)
    mag = np.minimum(np.abs(r), E4M3_MAX)
    idx = _nearest_index(mag, e4m3_values())
    return np.where((idx > 0) & (r < 0), idx | 0x80, idx).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    mag = e4m3_values()[c & 0x7F]
    return np.where(c & 0x80, -mag, mag)


def quantize_rows_e4m3(x):
    """(codes m x k uint8, scales m float32) per token (R20)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (x / s[:, None]).astype(np.float32)
    r = np.where(s[:, None] == 0, np.float32(0), r)
    return e4m3_round(r), s


def w4a8_ref(xcodes, xscales, wcodes, wscales, fmt: str) -> np.ndarray:
    """R22 in float64: s_x[m] * sum_g s_w[n, g] (Q_x,g @ V_w,g^T)."""
    qx = e4m3_decode(xcodes)
    vw = fp4_decode(wcodes, fmt)
    m, k = qx.shape
    n = vw.shape[0]
    y = np.zeros((m, n), dtype=np.float64)
    sw = np.asarray(wscales, dtype=np.float64)
    for g in range(k // GROUP):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        y += (qx[:, sl] @ vw[:, sl].T) * sw[None, :, g]
    return y * np.asarray(xscales, dtype=np.float64)[:, None]


def fp6_values(fmt: str) -> np.ndarray:
    """The 32 magnitudes of a 6-bit format, by magnitude index (R25)."""
    eb, mb, bias = FP6_FORMATS[fmt]
    return np.array([minifloat_value(i, eb, mb, bias) for i in range(32)], dtype=np.float64)


def fp6_decode(codes, fmt: str) -> np.ndarray:
    c = np.asarray(codes)
    mag = fp6_values(fmt)[c & 31]
    return np.where(c & 32, -mag, mag)


def quantize_rows_fp6(x, fmt: str):
    """(codes m x k uint8 in 0..63, scales m float32) per token (R25)."""
    x = np.asarray(x, dtype=np.float32)
    levels = fp6_values(fmt)
    vmax = np.float32(levels[-1])
    amax = np.max(np.abs(x), axis=1)
    s = (amax / vmax).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (x / s[:, None]).astype(np.float32)
    r = np.where(s[:, None] == 0, np.float32(0), r)
    idx = _nearest_index(np.minimum(np.abs(r), vmax), levels)
    return np.where((idx > 0) & (r < 0), idx | 32, idx).astype(np.uint8), s


def pack_fp6_tiled(codes) -> np.ndarray:
    """m x k codes -> the R26 storage (flat bytes, ceil(m/32) * (k/128) * 3072)."""
    c = np.asarray(codes, dtype=np.uint8)
    m, k = c.shape
    g = k // GROUP
    nb = -(-m // 32)
    cc = np.zeros((nb * 32, k), dtype=np.uint64)
    cc[:m] = c
    # the 192-bit string of each (row, group, step, half): 32 codes, code j at bits 6 j
    units = cc.reshape(nb, 32, g, 2, 2, 32)                       # b, r, g, s, h, j
    bits = np.zeros(units.shape[:-1] + (192,), dtype=np.uint8)
    for j in range(32):
        for t in range(6):
            bits[..., 6 * j + t] = (units[..., j] >> np.uint64(t)) & np.uint64(1)
    byts = np.packbits(bits.reshape(units.shape[:-1] + (24, 8)), axis=-1, bitorder="little")[..., 0]
    pieces = byts.reshape(nb, 32, g, 2, 2, 3, 8)                  # b, r, g, s, h, u, byte
    return pieces.transpose(0, 2, 3, 4, 5, 1, 6).reshape(-1).copy()


def unpack_fp6_tiled(data, m: int, k: int) -> np.ndarray:
    """Inverse of pack_fp6_tiled (padding rows dropped)."""
    g = k // GROUP
    nb = -(-m // 32)
    pieces = np.asarray(data, dtype=np.uint8).reshape(nb, g, 2, 2, 3, 32, 8)
    byts = pieces.transpose(0, 5, 1, 2, 3, 4, 6).reshape(nb, 32, g, 2, 2, 24)
    bits = np.unpackbits(byts[..., None], axis=-1, bitorder="little").reshape(nb, 32, g, 2, 2, 192)
    codes = np.zeros((nb, 32, g, 2, 2, 32), dtype=np.uint8)
    for t in range(6):
        codes |= (bits[..., t::6][..., :32] << t).astype(np.uint8)
    return codes.reshape(nb * 32, k)[:m].copy()


def w4a6_ref(xcodes, xscales, wcodes, wscales, wfmt: str, afmt: str) -> np.ndarray:
    """R22 with FP6 activations, in float64."""
    qx = fp6_decode(xcodes, afmt)
    vw = fp4_decode(wcodes, wfmt)
    m, k = qx.shape
    y = np.zeros((m, vw.shape[0]), dtype=np.float64)
    sw = np.asarray(wscales, dtype=np.float64)
    for g in range(k // GROUP):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        y += (qx[:, sl] @ vw[:, sl].T) * sw[None, :, g]
    return y * np.asarray(xscales, dtype=np.float64)[:, None]


def quantize_fp6_groups(w, fmt: str, pow2: bool = False):
    """(codes n x k uint8 in 0..63, scales n x k/128 float32) per R27: R19's
    group quantizer with the FP6 levels (R23's scales with pow2)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    levels = fp6_values(fmt)
    vmax = np.float32(levels[-1])
    g = w.reshape(n, k // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = (amax / vmax).astype(np.float32)
        if pow2:
            s = np.where(s > 0, _pow2_at_least(np.where(s > 0, s, 1.0)), np.float32(0)).astype(np.float32)
        r = (g / s[:, :, None]).astype(np.float32)
    r = np.where(s[:, :, None] == 0, np.float32(0), r)
    idx = _nearest_index(np.abs(r), levels)
    codes = np.where((idx > 0) & (r < 0), idx | 32, idx).astype(np.uint8)
    return codes.reshape(n, k), s


def tile_group_scales(scales) -> np.ndarray:
    """n x G group scales -> R24's tiled order: 32 per (column block, group),
    column 32 b + j at position j, blocks padded with zeros (flat floats)."""
    sc = np.asarray(scales, dtype=np.float32)
    n, g = sc.shape
    nb = -(-n // 32)
    ss = np.zeros((nb * 32, g), dtype=np.float32)
    ss[:n] = sc
    return ss.reshape(nb, 32, g).transpose(0, 2, 1).reshape(-1).copy()


def untile_group_scales(tscales, n: int, k: int) -> np.ndarray:
    """Inverse of tile_group_scales (padding dropped)."""
    g = k // GROUP
    nb = -(-n // 32)
    s = np.asarray(tscales, dtype=np.float32).reshape(nb, g, 32).transpose(0, 2, 1)
    return s.reshape(nb * 32, g)[:n].copy()


def w6a8_ref(xcodes, xscales, wcodes, wscales, wfmt: str) -> np.ndarray:
    """R28 in float64: s_x[m] * sum_g s_w[n, g] (Q_x,g @ V_w,g^T)."""
    qx = e4m3_decode(xcodes)
    vw = fp6_decode(wcodes, wfmt)
    m, k = qx.shape
    y = np.zeros((m, vw.shape[0]), dtype=np.float64)
    sw = np.asarray(wscales, dtype=np.float64)
    for g in range(k // GROUP):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        y += (qx[:, sl] @ vw[:, sl].T) * sw[None, :, g]
    return y * np.asarray(xscales, dtype=np.float64)[:, None]
