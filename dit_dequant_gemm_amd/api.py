"""Python binding of libddg.so (ctypes).  Argument marshalling only.

PyTorch supplies device memory and the current HIP stream; every step of
the computation runs in the library's gfx950 kernels.  When the shared
library is missing or cannot be loaded every call raises ``RuntimeError``:
there is no CPU or PyTorch fallback.

The record mirrors the stored format of the Wan-Dancer-14B quantization
report (§3.3): ``{name}_packed`` (uint8), ``{name}_scales`` (float32 per
128-group), ``{name}_bw`` (int8 bit width) and ``{name}_nin`` (int32 padded
input dimension).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

GROUP = 128
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libddg.so")
_LIB: Optional[ctypes.CDLL] = None

DDG_BF16, DDG_F32 = 0, 1

# entry point -> (restype, argtypes)
_c_i64, _c_int, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t


class GemmDesc(ctypes.Structure):
    """ddg_gemm_desc: one product of a grouped call."""
    _fields_ = [("x", _vp), ("packed", _vp), ("scales", _vp), ("y", _vp),
                ("m", _c_i64), ("k", _c_i64), ("n", _c_i64), ("bits", _c_int), ("y_dtype", _c_int)]


MAX_GROUPED = 256
SIGNATURES = {
    "ddg_version": (_c_int, []),
    "ddg_status_string": (ctypes.c_char_p, [_c_int]),
    "ddg_packed_bytes": (_c_int, [_c_i64, _c_i64, _c_int, ctypes.POINTER(_c_i64), ctypes.POINTER(_c_i64)]),
    "ddg_quantize_pack": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_int, _vp, _vp, _vp]),
    "ddg_dequantize": (_c_int, [_vp, _vp, _c_int, _c_i64, _c_i64, _vp, _vp]),
    "ddg_dequant_gemm": (_c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _c_int, _c_i64, _vp, _c_int, _vp, _sz, _vp]),
    "ddg_dequant_gemm_grouped": (_c_int, [ctypes.POINTER(GemmDesc), _c_int, _vp]),
    "ddg_workspace_bytes": (_c_int, [_c_i64, _c_i64, _c_i64, _c_int, ctypes.POINTER(_sz)]),
    "ddg_quant_sse": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _vp, _vp, _vp]),
    "ddg_pd_allocate": (_c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_c_i64), _c_int,
                                 ctypes.POINTER(_c_int), _c_int, ctypes.c_double,
                                 ctypes.POINTER(ctypes.c_double), _c_int, _c_int,
                                 ctypes.POINTER(_c_int), ctypes.POINTER(ctypes.c_double)]),
    "ddg_lowrank_down": (_c_int, [_vp, _c_i64, _c_i64, _vp, _c_int, _vp, _vp]),
    "ddg_lowrank_fused_gemm": (_c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _c_int, _c_i64, _vp, _vp,
                                        _c_int, _vp, _c_int, _vp, _sz, _vp]),
    "ddg_lowrank_fused_gemm_noalloc": (_c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _c_int, _c_i64, _vp, _vp,
                                                _c_int, _vp, _c_int, _vp]),
    "ddg_rpbh_rotate": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _vp, _vp, _c_int, _vp, _c_int, _vp]),
    "ddg_fp4_quantize_pack": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_int, _vp, _vp, _vp]),
    "ddg_fp8_quantize_rows": (_c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp]),
    "ddg_w4a8_gemm": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _vp, _c_int, _c_i64, _vp, _c_int, _vp]),
    "ddg_fp6_quantize_rows": (_c_int, [_vp, _c_i64, _c_i64, _c_int, _vp, _vp, _vp]),
    "ddg_w4a6_gemm": (_c_int, [_vp, _vp, _c_i64, _c_i64, _c_int, _vp, _vp, _c_int, _c_i64, _vp, _c_int, _vp]),
    "ddg_fp6_quantize_pack": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_int, _vp, _vp, _vp]),
    "ddg_w6a8_gemm": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _vp, _c_int, _c_i64, _vp, _c_int, _vp]),
}

FP4_FORMATS = {"e2m1": 0, "e3m0": 1, "e1m2": 2}
FP4_POW2 = 0x100
FP4_TILED = 0x200
FP6_FORMATS = {"e2m3": 0, "e3m2": 1}

ROTATE_MAX_D, ROTATE_MAX_H = 16384, 1024


class DDGError(RuntimeError):
    """A libddg entry point returned a negative status."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libddg.so (once).  Raises RuntimeError when it is missing."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libddg.so not found at {p}; build it with "
                           "`python -m dit_dequant_gemm_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ddg_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DDGError(status, where)


# The raw handle of torch's current stream, without building a Stream object
# (that costs several microseconds per call, more than a 16-token product
# takes on the GPU).
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(device: torch.device) -> int:
    if _RAW_STREAM is not None:
        idx = device.index
        return _RAW_STREAM(torch.cuda.current_device() if idx is None else idx)
    return torch.cuda.current_stream(device).cuda_stream


def _require_cuda(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def packed_sizes(n: int, k: int, bits: int):
    """(packed bytes, number of scales) of an n x k weight at `bits`."""
    pb, ns = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().ddg_packed_bytes(n, k, bits, ctypes.byref(pb), ctypes.byref(ns)),
           "ddg_packed_bytes")
    return pb.value, ns.value


@dataclass
class QWeight:
    """Quantized weight record: packed codes, per-group scales, bit width,
    padded input dimension (``k``) and the original input dimension."""
    packed: torch.Tensor      # uint8, n*k*bits/8
    scales: torch.Tensor      # float32, (n, k/128)
    bits: int
    n: int
    k: int                    # padded input dimension (multiple of 128)
    orig_in: int

    def state_dict(self, prefix: str) -> dict:
        return {
            f"{prefix}_packed": self.packed,
            f"{prefix}_scales": self.scales,
            f"{prefix}_bw": torch.tensor(self.bits, dtype=torch.int8),
            f"{prefix}_nin": torch.tensor(self.k, dtype=torch.int32),
        }

    @classmethod
    def from_state_dict(cls, sd: dict, prefix: str, orig_in: Optional[int] = None,
                        device="cuda") -> "QWeight":
        """The record's four fields, checked against one another on the host
        (the kernels size their reads from n, k and bits): ValueError for a
        width outside 3..7, a padded input dimension that is not a positive
        multiple of 128, scales that are not whole rows of k/128, packed bytes
        other than n*k*bits/8, or orig_in outside (k - 128, k]."""
        bits = int(sd[f"{prefix}_bw"])
        k = int(sd[f"{prefix}_nin"])
        if bits < 3 or bits > 7:
            raise ValueError(f"{prefix}_bw = {bits}: widths are 3..7")
        if k <= 0 or k % GROUP:
            raise ValueError(f"{prefix}_nin = {k}: not a positive multiple of {GROUP}")
        scales = sd[f"{prefix}_scales"]
        packed = sd[f"{prefix}_packed"]
        if scales.dtype != torch.float32 or packed.dtype != torch.uint8:
            raise ValueError(f"{prefix}: scales must be float32 and packed uint8")
        if scales.numel() == 0 or scales.numel() % (k // GROUP):
            raise ValueError(f"{prefix}_scales: {scales.numel()} values are not whole rows of {k // GROUP}")
        n = scales.numel() // (k // GROUP)
        pb, ns = packed_sizes(n, k, bits)
        if packed.numel() != pb or scales.numel() != ns:
            raise ValueError(f"{prefix}_packed: {packed.numel()} bytes, {pb} expected for {n} x {k} at {bits} bits")
        orig = orig_in or k
        if not k - GROUP < orig <= k:
            raise ValueError(f"orig_in = {orig} does not pad to {k}")
        scales = scales.to(device=device).contiguous().view(n, k // GROUP)
        packed = packed.to(device=device).contiguous().view(-1)
        return cls(packed, scales, bits, n, k, orig)


def quantize_pack(w: torch.Tensor, bits: int) -> QWeight:
    """Quantize an (out x in) bf16/float32 GPU weight per 128-group and pack it."""
    _require_cuda(w, "w")
    if w.dim() != 2 or w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("w must be a 2-D bf16 or float32 tensor")
    n, orig_in = w.shape
    k = -(-orig_in // GROUP) * GROUP
    if k != orig_in:                      # zero-pad the input dimension (record's _nin)
        w = torch.nn.functional.pad(w, (0, k - orig_in)).contiguous()
    pb, ns = packed_sizes(n, k, bits)
    packed = torch.empty(pb, dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, k // GROUP), dtype=torch.float32, device=w.device)
    lib = load_library()
    _check(lib.ddg_quantize_pack(w.data_ptr(), DDG_F32 if w.dtype == torch.float32 else DDG_BF16,
                                 n, k, bits, packed.data_ptr(), scales.data_ptr(),
                                 _stream_ptr(w.device)), "ddg_quantize_pack")
    return QWeight(packed, scales, bits, n, k, orig_in)


def rpbh_rotate(x: torch.Tensor, perm: torch.Tensor, signs: torch.Tensor, h: int,
                out_dtype: Optional[torch.dtype] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows of x (n x d, bf16 or float32) rotated by the random-permuted block
    Hadamard map: permute by perm (int32), flip by signs (int8, negative = -1),
    then a normalised Walsh-Hadamard transform on each block of h.  Rotate the
    weight rows once (then quantize them) and every activation row with the
    same perm, signs and h: the product is unchanged."""
    for t, name in ((x, "x"), (perm, "perm"), (signs, "signs")):
        _require_cuda(t, name)
    if x.dim() != 2 or x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be a 2-D bf16 or float32 tensor")
    n, d = x.shape
    if perm.dtype != torch.int32 or signs.dtype != torch.int8 or perm.shape != (d,) or signs.shape != (d,):
        raise ValueError("perm must be int32 and signs int8, each of length d")
    x = x.contiguous()
    perm = perm.contiguous()
    signs = signs.contiguous()
    odt = out_dtype or (out.dtype if out is not None else x.dtype)
    if out is None:
        out = torch.empty((n, d), dtype=odt, device=x.device)
    elif out.shape != (n, d) or out.dtype != odt or not out.is_contiguous():
        raise ValueError("out must be a contiguous n x d tensor of the output dtype")
    code = {torch.bfloat16: DDG_BF16, torch.float32: DDG_F32}
    if odt not in code:
        raise ValueError("out dtype must be bf16 or float32")
    _check(load_library().ddg_rpbh_rotate(x.data_ptr(), code[x.dtype], n, d, perm.data_ptr(),
                                          signs.data_ptr(), h, out.data_ptr(), code[odt],
                                          _stream_ptr(x.device)), "ddg_rpbh_rotate")
    return out


class QWeightFP4:
    """A weight in a 4-bit floating-point format: packed (n x k/2 bytes, code
    2i in the low nibble of byte i), scales (n x k/128 float32), fmt; pow2:
    the scales are powers of two, applied by the matrix instructions; tiled:
    codes and scales in 32-column blocks ordered for the matrix operands
    (flat, ceil(n/32) * k/128 * 2048 bytes and * 32 floats)."""

    def __init__(self, packed: torch.Tensor, scales: torch.Tensor, fmt: str, n: int, k: int,
                 pow2: bool = False, tiled: bool = False):
        self.packed, self.scales, self.fmt, self.n, self.k = packed, scales, fmt, n, k
        self.pow2, self.tiled = pow2, tiled

    @property
    def fmt_code(self) -> int:
        return FP4_FORMATS[self.fmt] | (FP4_POW2 if self.pow2 else 0) | (FP4_TILED if self.tiled else 0)


def fp4_quantize_pack(w: torch.Tensor, fmt: str = "e2m1", pow2: bool = False, tiled: bool = False) -> QWeightFP4:
    """Per-group(128) 4-bit float quantization of an (out x in) GPU weight;
    pow2 rounds each group scale up to a power of two; tiled writes the
    storage ordered for the matrix operands."""
    _require_cuda(w, "w")
    if fmt not in FP4_FORMATS:
        raise ValueError(f"fmt must be one of {sorted(FP4_FORMATS)}")
    if w.dim() != 2 or w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("w must be a 2-D bf16 or float32 tensor")
    w = w.contiguous()
    n, k = w.shape
    g = max(k // GROUP, 0)
    if tiled:
        nb = -(-n // 32)
        packed = torch.empty((nb * g * 2048,), dtype=torch.uint8, device=w.device)
        scales = torch.empty((nb * g * 32,), dtype=torch.float32, device=w.device)
    else:
        packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
        scales = torch.empty((n, g), dtype=torch.float32, device=w.device)
    q = QWeightFP4(packed, scales, fmt, n, k, pow2, tiled)
    _check(load_library().ddg_fp4_quantize_pack(w.data_ptr(), DDG_F32 if w.dtype == torch.float32 else DDG_BF16,
                                                n, k, q.fmt_code, packed.data_ptr(), scales.data_ptr(),
                                                _stream_ptr(w.device)), "ddg_fp4_quantize_pack")
    return q


def fp8_quantize_rows(x: torch.Tensor):
    """Per-token E4M3 codes (m x k uint8) and scales (m float32) of a bf16 X."""
    _require_cuda(x, "x")
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 2-D bf16 tensor")
    x = x.contiguous()
    m, k = x.shape
    xq = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    xs = torch.empty((m,), dtype=torch.float32, device=x.device)
    _check(load_library().ddg_fp8_quantize_rows(x.data_ptr(), m, k, xq.data_ptr(), xs.data_ptr(),
                                                _stream_ptr(x.device)), "ddg_fp8_quantize_rows")
    return xq, xs


def w4a8_gemm(xq: torch.Tensor, xs: torch.Tensor, qw: QWeightFP4, out_dtype=torch.bfloat16,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = s_x[m] * sum_g s_w[n, g] (X_q W_q^T)_g on the FP8 x FP4 matrix cores."""
    for t, name in ((xq, "xq"), (xs, "xs")):
        _require_cuda(t, name)
    if xq.dtype != torch.uint8 or xq.dim() != 2 or xq.shape[1] != qw.k or xs.shape != (xq.shape[0],):
        raise ValueError("xq must be m x k uint8 codes with m float32 scales")
    m = xq.shape[0]
    y = out if out is not None else torch.empty((m, qw.n), dtype=out_dtype, device=xq.device)
    if y.shape != (m, qw.n) or y.dtype not in (torch.bfloat16, torch.float32) or not y.is_contiguous():
        raise ValueError("out must be a contiguous m x n bf16 or float32 tensor")
    _check(load_library().ddg_w4a8_gemm(xq.contiguous().data_ptr(), xs.contiguous().data_ptr(), m, qw.k,
                                        qw.packed.data_ptr(), qw.scales.data_ptr(), qw.fmt_code,
                                        qw.n, y.data_ptr(), DDG_F32 if y.dtype == torch.float32 else DDG_BF16,
                                        _stream_ptr(xq.device)), "ddg_w4a8_gemm")
    return y


def dequantize(qw: QWeight) -> torch.Tensor:
    """Dense bf16 w_hat (n x padded in)."""
    out = torch.empty((qw.n, qw.k), dtype=torch.bfloat16, device=qw.packed.device)
    _check(load_library().ddg_dequantize(qw.packed.data_ptr(), qw.scales.data_ptr(), qw.bits,
                                         qw.n, qw.k, out.data_ptr(),
                                         _stream_ptr(qw.packed.device)), "ddg_dequantize")
    return out


def _prep_x(x: torch.Tensor, qw: QWeight) -> torch.Tensor:
    _require_cuda(x, "x")
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 2-D bf16 tensor")
    if x.shape[1] == qw.k:
        return x
    if x.shape[1] != qw.orig_in:
        raise ValueError(f"x has {x.shape[1]} inputs, weight expects {qw.orig_in}")
    return torch.nn.functional.pad(x, (0, qw.k - qw.orig_in)).contiguous()


def _out(x: torch.Tensor, n: int, out_dtype, out):
    if out is None:
        return torch.empty((x.shape[0], n), dtype=out_dtype, device=x.device)
    _require_cuda(out, "out")
    if out.shape != (x.shape[0], n) or out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out has the wrong shape or dtype")
    return out


# Workspaces kept per (device, stream): calls on one stream are ordered, so
# they may share one; calls on different streams get their own.
_WORKSPACES: dict = {}


def _cached_workspace(device: torch.device, stream: int, nbytes: int) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def _capturing() -> bool:
    """True while the current stream is being captured into a graph."""
    return torch.cuda.is_current_stream_capturing()


def dequant_gemm(x: torch.Tensor, qw: QWeight, out_dtype=torch.bfloat16,
                 out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X @ w_hat^T with on-the-fly dequantization.  workspace: optional
    scratch (uint8, at least workspace_bytes(m, n, k, 0) bytes) for the
    split-K and stream-K forms; by default one kept per device and stream is
    used.  Under graph capture no workspace is used (whole tiles): a call that
    splits K tags its partial sums with a launch epoch that every replay of a
    graph would repeat, so replays could read an earlier replay's sums; a
    workspace passed under capture raises ValueError."""
    x = _prep_x(x, qw)
    y = _out(x, qw.n, out_dtype, out)
    sp = _stream_ptr(x.device)
    if _capturing():
        if workspace is not None:
            raise ValueError("dequant_gemm: no workspace under graph capture (split K is launch-specific)")
    elif workspace is None:
        workspace = _cached_workspace(x.device, sp, workspace_bytes(x.shape[0], qw.n, qw.k, 0))
    wp, wb = (0, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    _check(load_library().ddg_dequant_gemm(
        x.data_ptr(), x.shape[0], qw.k, qw.packed.data_ptr(), qw.scales.data_ptr(), qw.bits,
        qw.n, y.data_ptr(), DDG_F32 if y.dtype == torch.float32 else DDG_BF16, wp or None, wb,
        sp), "ddg_dequant_gemm")
    return y


def dequant_gemm_grouped(items, out_dtype=torch.bfloat16):
    """Several independent products Y_i = X_i @ w_hat_i^T in as few launches
    as possible.  items: sequence of (x, qw) or (x, qw, out); returns the
    list of outputs.  All tensors on the same device; the current stream."""
    items = list(items)
    if not items:
        return []
    descs = (GemmDesc * len(items))()
    outs, keep = [], []
    for i, it in enumerate(items):
        x, qw = it[0], it[1]
        out = it[2] if len(it) > 2 else None
        x = _prep_x(x, qw)
        y = _out(x, qw.n, out_dtype, out)
        keep.append(x)
        outs.append(y)
        descs[i] = GemmDesc(x.data_ptr(), qw.packed.data_ptr(), qw.scales.data_ptr(), y.data_ptr(),
                            x.shape[0], qw.k, qw.n, qw.bits,
                            DDG_F32 if y.dtype == torch.float32 else DDG_BF16)
    _check(load_library().ddg_dequant_gemm_grouped(descs, len(items), _stream_ptr(outs[0].device)),
           "ddg_dequant_gemm_grouped")
    return outs


def workspace_bytes(m: int, n: int, k: int, r: int) -> int:
    """Workspace bytes of lowrank_fused_gemm for an m x k input, an n x k
    weight and rank r."""
    b = ctypes.c_size_t()
    _check(load_library().ddg_workspace_bytes(m, n, k, r, ctypes.byref(b)), "ddg_workspace_bytes")
    return b.value


def lowrank_down(x: torch.Tensor, lora_down: torch.Tensor,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """T = bf16(X @ L1) alone (lora_down = L1^T, r x in, bf16): the pre-pass of
    lowrank_fused_gemm.  x: (m x in) bf16 with in a multiple of 128."""
    for t, name in ((x, "x"), (lora_down, "lora_down")):
        _require_cuda(t, name)
        if t.dtype != torch.bfloat16 or t.dim() != 2:
            raise ValueError(f"{name} must be a 2-D bf16 tensor")
    m, k = x.shape
    r = lora_down.shape[0]
    if lora_down.shape[1] != k:
        raise ValueError("lora_down has the wrong input dimension")
    if out is None:
        out = torch.empty(m, r, dtype=torch.bfloat16, device=x.device)
    elif out.shape != (m, r) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous (m x r) bf16 tensor")
    _check(load_library().ddg_lowrank_down(x.data_ptr(), m, k, lora_down.data_ptr(), r,
                                           out.data_ptr(), _stream_ptr(x.device)),
           "ddg_lowrank_down")
    return out


def lowrank_fused_gemm(x: torch.Tensor, qw: QWeight, lora_down: torch.Tensor,
                       lora_up: torch.Tensor, out_dtype=torch.bfloat16,
                       out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X @ w_hat^T + bf16(X @ L1) @ L2 with lora_down = L1^T (r x in) and
    lora_up = L2^T (out x r), both bf16.  Under graph capture only T's bytes
    of the workspace are handed over (whole tiles, unsplit pre-pass: see
    dequant_gemm)."""
    x = _prep_x(x, qw)
    for t, name in ((lora_down, "lora_down"), (lora_up, "lora_up")):
        _require_cuda(t, name)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16")
    r = lora_down.shape[0]
    if lora_down.shape[1] != qw.k:
        if lora_down.shape[1] != qw.orig_in:
            raise ValueError("lora_down has the wrong input dimension")
        lora_down = torch.nn.functional.pad(lora_down, (0, qw.k - qw.orig_in)).contiguous()
    if lora_up.shape != (qw.n, r):
        raise ValueError("lora_up must be (out x r)")
    y = _out(x, qw.n, out_dtype, out)
    need = workspace_bytes(x.shape[0], qw.n, qw.k, r)
    if workspace is None:
        workspace = _cached_workspace(x.device, _stream_ptr(x.device), max(need, 256))
    wbytes = workspace.numel() * workspace.element_size()
    if _capturing():
        # T's bytes alone: whole tiles and the unsplit pre-pass, nothing that
        # depends on the launch (see dequant_gemm)
        wbytes = min(wbytes, -(-x.shape[0] * r * 2 // 256) * 256)
    _check(load_library().ddg_lowrank_fused_gemm(
        x.data_ptr(), x.shape[0], qw.k, qw.packed.data_ptr(), qw.scales.data_ptr(), qw.bits,
        qw.n, lora_down.data_ptr(), lora_up.data_ptr(), r, y.data_ptr(),
        DDG_F32 if y.dtype == torch.float32 else DDG_BF16, workspace.data_ptr(),
        wbytes, _stream_ptr(x.device)),
        "ddg_lowrank_fused_gemm")
    return y


NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024


def lowrank_fused_gemm_noalloc(x: torch.Tensor, qw: QWeight, lora_down: torch.Tensor,
                               lora_up: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """lowrank_fused_gemm without a workspace (for callers that cannot
    allocate): T goes to the library's own device array, shared by every call
    on the GPU.  Allocates nothing: x (m x k), lora_down (r x k), lora_up
    (n x r) and out (m x n) must already have the shapes of the record."""
    for t, name in ((x, "x"), (lora_down, "lora_down"), (lora_up, "lora_up"), (out, "out")):
        _require_cuda(t, name)
    r = lora_down.shape[0]
    if (x.dtype != torch.bfloat16 or lora_down.dtype != torch.bfloat16 or lora_up.dtype != torch.bfloat16
            or x.dim() != 2 or x.shape[1] != qw.k or lora_down.shape != (r, qw.k)
            or lora_up.shape != (qw.n, r) or out.shape != (x.shape[0], qw.n)
            or out.dtype not in (torch.bfloat16, torch.float32)):
        raise ValueError("x, lora_down, lora_up (bf16) and out must have the record's shapes")
    _check(load_library().ddg_lowrank_fused_gemm_noalloc(
        x.data_ptr(), x.shape[0], qw.k, qw.packed.data_ptr(), qw.scales.data_ptr(), qw.bits,
        qw.n, lora_down.data_ptr(), lora_up.data_ptr(), r, out.data_ptr(),
        DDG_F32 if out.dtype == torch.float32 else DDG_BF16, _stream_ptr(x.device)),
        "ddg_lowrank_fused_gemm_noalloc")
    return out


# ------------------------------------------------------------------ bit allocation
PD_CANDIDATES = (3, 4, 5, 6, 7)


def quant_sse(w: torch.Tensor):
    """(row_sse n x 5 float64, total 5 float64) GPU tensors: sum of
    (w - w_hat32)^2 per row and over the tensor at widths 3..7."""
    _require_cuda(w, "w")
    if w.dim() != 2 or w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("w must be a 2-D bf16 or float32 tensor")
    n, k = w.shape
    if k % GROUP:
        w = torch.nn.functional.pad(w, (0, GROUP - k % GROUP)).contiguous()
        k = w.shape[1]
    rows = torch.empty((max(n, 1), 5), dtype=torch.float64, device=w.device)
    total = torch.empty(5, dtype=torch.float64, device=w.device)
    _check(load_library().ddg_quant_sse(w.data_ptr(), DDG_F32 if w.dtype == torch.float32 else DDG_BF16,
                                        n, k, rows.data_ptr(), total.data_ptr(),
                                        _stream_ptr(w.device)), "ddg_quant_sse")
    return rows[:n], total


def sse_table(weights):
    """(sse N x 5, nparams N) numpy arrays: the squared-error sums of every
    tensor at widths 3..7 (the totals of ddg_quant_sse, the tables the
    allocation searches over) and each tensor's element count (weights padded
    along the input dimension count their real elements)."""
    import numpy as np
    totals = [quant_sse(w)[1] for w in weights]
    sse = np.stack([t.cpu().numpy() for t in totals]) if totals else np.empty((0, 5))
    nparams = np.array([w.numel() for w in weights], dtype=np.int64)
    return sse, nparams


def pd_allocate(sse, nparams, target_bpw: float, t_init, iters: int = 500,
                candidates=PD_CANDIDATES):
    """PD-guided widths for every tensor (host-side search in the library).
    sse: N x len(candidates) squared-error sums (sse_table); t_init: restarts
    x N starting parameters.  Returns (bits, info dict)."""
    import numpy as np
    sse = np.ascontiguousarray(sse, dtype=np.float64)
    nparams = np.ascontiguousarray(nparams, dtype=np.int64)
    t_init = np.ascontiguousarray(t_init, dtype=np.float64)
    cand = np.ascontiguousarray(candidates, dtype=np.int32)
    n = nparams.shape[0]
    if sse.shape != (n, cand.shape[0]) or t_init.ndim != 2 or t_init.shape[1] != n:
        raise ValueError("sse must be N x len(candidates) and t_init restarts x N")
    bits = np.empty(n, dtype=np.int32)
    info = np.empty(3, dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    _check(load_library().ddg_pd_allocate(
        sse.ctypes.data_as(dp), nparams.ctypes.data_as(ctypes.POINTER(_c_i64)), n,
        cand.ctypes.data_as(ctypes.POINTER(_c_int)), cand.shape[0], float(target_bpw),
        t_init.ctypes.data_as(dp), t_init.shape[0], iters, bits.ctypes.data_as(ctypes.POINTER(_c_int)),
        info.ctypes.data_as(dp)), "ddg_pd_allocate")
    return bits.astype(np.int64), {"mse": float(info[0]), "bpw": float(info[1]), "restart": int(info[2])}


def fp6_quantize_rows(x: torch.Tensor, fmt: str = "e2m3"):
    """Per-token FP6 codes of a bf16 X in the tiled 6-bit storage (flat uint8,
    ceil(m/32) * k/128 * 3072 bytes) and the m float32 scales."""
    _require_cuda(x, "x")
    if fmt not in FP6_FORMATS:
        raise ValueError(f"fmt must be one of {sorted(FP6_FORMATS)}")
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 2-D bf16 tensor")
    x = x.contiguous()
    m, k = x.shape
    xq = torch.empty((-(-m // 32) * max(k // GROUP, 0) * 3072,), dtype=torch.uint8, device=x.device)
    xs = torch.empty((m,), dtype=torch.float32, device=x.device)
    _check(load_library().ddg_fp6_quantize_rows(x.data_ptr(), m, k, FP6_FORMATS[fmt], xq.data_ptr(), xs.data_ptr(),
                                                _stream_ptr(x.device)), "ddg_fp6_quantize_rows")
    return xq, xs


def w4a6_gemm(xq: torch.Tensor, xs: torch.Tensor, fmt: str, qw: QWeightFP4, out_dtype=torch.bfloat16,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = s_x[m] * sum_g s_w[n, g] (X_q W_q^T)_g on the FP6 x FP4 matrix cores
    (X from fp6_quantize_rows in format fmt; tiled FP4 weights of any format)."""
    for t, name in ((xq, "xq"), (xs, "xs")):
        _require_cuda(t, name)
    if fmt not in FP6_FORMATS:
        raise ValueError(f"fmt must be one of {sorted(FP6_FORMATS)}")
    m = xs.shape[0]
    if xq.dtype != torch.uint8 or xq.numel() != -(-m // 32) * (qw.k // GROUP) * 3072 or xs.dim() != 1:
        raise ValueError("xq must be the tiled 6-bit storage of m x k codes, with m float32 scales")
    y = out if out is not None else torch.empty((m, qw.n), dtype=out_dtype, device=xq.device)
    if y.shape != (m, qw.n) or y.dtype not in (torch.bfloat16, torch.float32) or not y.is_contiguous():
        raise ValueError("out must be a contiguous m x n bf16 or float32 tensor")
    _check(load_library().ddg_w4a6_gemm(xq.contiguous().data_ptr(), xs.contiguous().data_ptr(), m, qw.k,
                                        FP6_FORMATS[fmt], qw.packed.data_ptr(), qw.scales.data_ptr(), qw.fmt_code,
                                        qw.n, y.data_ptr(), DDG_F32 if y.dtype == torch.float32 else DDG_BF16,
                                        _stream_ptr(xq.device)), "ddg_w4a6_gemm")
    return y


class QWeightFP6:
    """A weight in a 6-bit floating-point format (fmt "e2m3" or "e3m2") per
    group of 128: packed, the tiled 6-bit storage with the weight's rows in
    place of tokens (flat, ceil(n/32) * k/128 * 3072 bytes); scales, tiled 32
    per (column block, group) (flat, ceil(n/32) * k/128 * 32 floats); pow2:
    the scales are powers of two, applied by the matrix instructions."""

    def __init__(self, packed: torch.Tensor, scales: torch.Tensor, fmt: str, n: int, k: int,
                 pow2: bool = False):
        self.packed, self.scales, self.fmt, self.n, self.k, self.pow2 = packed, scales, fmt, n, k, pow2

    @property
    def fmt_code(self) -> int:
        return FP6_FORMATS[self.fmt] | (FP4_POW2 if self.pow2 else 0)


def fp6_quantize_pack(w: torch.Tensor, fmt: str = "e2m3", pow2: bool = False) -> QWeightFP6:
    """Per-group(128) 6-bit float quantization of an (out x in) GPU weight
    into the tiled 6-bit storage; pow2 rounds each group scale up to a power
    of two."""
    _require_cuda(w, "w")
    if fmt not in FP6_FORMATS:
        raise ValueError(f"fmt must be one of {sorted(FP6_FORMATS)}")
    if w.dim() != 2 or w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("w must be a 2-D bf16 or float32 tensor")
    w = w.contiguous()
    n, k = w.shape
    g, nb = max(k // GROUP, 0), -(-n // 32)
    packed = torch.empty((nb * g * 3072,), dtype=torch.uint8, device=w.device)
    scales = torch.empty((nb * g * 32,), dtype=torch.float32, device=w.device)
    q = QWeightFP6(packed, scales, fmt, n, k, pow2)
    _check(load_library().ddg_fp6_quantize_pack(w.data_ptr(), DDG_F32 if w.dtype == torch.float32 else DDG_BF16,
                                                n, k, q.fmt_code, packed.data_ptr(), scales.data_ptr(),
                                                _stream_ptr(w.device)), "ddg_fp6_quantize_pack")
    return q


def w6a8_gemm(xq: torch.Tensor, xs: torch.Tensor, qw: QWeightFP6, out_dtype=torch.bfloat16,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = s_x[m] * sum_g s_w[n, g] (X_q W_q^T)_g on the FP8 x FP6 matrix cores
    (X from fp8_quantize_rows, W from fp6_quantize_pack)."""
    for t, name in ((xq, "xq"), (xs, "xs")):
        _require_cuda(t, name)
    if xq.dtype != torch.uint8 or xq.dim() != 2 or xq.shape[1] != qw.k or xs.shape != (xq.shape[0],):
        raise ValueError("xq must be m x k uint8 codes with m float32 scales")
    m = xq.shape[0]
    y = out if out is not None else torch.empty((m, qw.n), dtype=out_dtype, device=xq.device)
    if y.shape != (m, qw.n) or y.dtype not in (torch.bfloat16, torch.float32) or not y.is_contiguous():
        raise ValueError("out must be a contiguous m x n bf16 or float32 tensor")
    _check(load_library().ddg_w6a8_gemm(xq.contiguous().data_ptr(), xs.contiguous().data_ptr(), m, qw.k,
                                        qw.packed.data_ptr(), qw.scales.data_ptr(), qw.fmt_code,
                                        qw.n, y.data_ptr(), DDG_F32 if y.dtype == torch.float32 else DDG_BF16,
                                        _stream_ptr(xq.device)), "ddg_w6a8_gemm")
    return y
