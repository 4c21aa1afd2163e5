"""The C ABI on the host (CPU only): the library loads, exports every entry
point declared in include/ddg.h, and rejects bad arguments before any HIP
call.  No compute call is made here: every call either expects an error that
the host checks return before any launch, or is an empty (M == 0) no-op, so
the file is safe to run where a GPU is present (the fake addresses below are
never handed to a kernel)."""
import ctypes
import os
import re

import pytest
import torch

from dit_dequant_gemm_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddg.h")

OK, E_ARG, E_SHAPE, E_ALIGN, E_WS = 0, -1, -2, -3, -4
FAKE = 0x10000          # aligned non-null address; never dereferenced by these calls
MISALIGNED = 0x10004


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return api.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("ddg_quantize_pack", "ddg_dequant_gemm", "ddg_lowrank_fused_gemm",
              "ddg_dequantize", "ddg_packed_bytes", "ddg_workspace_bytes",
              "ddg_status_string", "ddg_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(api.SIGNATURES)


def test_version_and_status_strings(lib):
    assert lib.ddg_version() == 1
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert lib.ddg_status_string(st)
    assert lib.ddg_status_string(12345) == b"unknown status"


@pytest.mark.parametrize("bits,ratio", [(3, 3 / 8), (4, 1 / 2), (5, 5 / 8), (6, 6 / 8), (7, 7 / 8)])
def test_packed_bytes(lib, bits, ratio):
    pb, ns = ctypes.c_int64(), ctypes.c_int64()
    assert lib.ddg_packed_bytes(5120, 5120, bits, ctypes.byref(pb), ctypes.byref(ns)) == OK
    assert pb.value == int(5120 * 5120 * ratio) and ns.value == 204_800
    assert lib.ddg_packed_bytes(16, 100, bits, ctypes.byref(pb), ctypes.byref(ns)) == E_SHAPE
    assert lib.ddg_packed_bytes(16, 0, bits, ctypes.byref(pb), ctypes.byref(ns)) == E_SHAPE
    assert lib.ddg_packed_bytes(-1, 128, bits, ctypes.byref(pb), ctypes.byref(ns)) == E_SHAPE
    assert lib.ddg_packed_bytes(16, 128, bits, None, ctypes.byref(ns)) == E_ARG
    assert lib.ddg_packed_bytes(0, 128, bits, ctypes.byref(pb), ctypes.byref(ns)) == OK
    assert pb.value == 0


def test_packed_bytes_bad_bits(lib):
    pb, ns = ctypes.c_int64(), ctypes.c_int64()
    for b in (0, 1, 2, 8, 16, -4):
        assert lib.ddg_packed_bytes(16, 128, b, ctypes.byref(pb), ctypes.byref(ns)) == E_ARG


def test_workspace_bytes(lib):
    b = ctypes.c_size_t()
    sk = 256 * 256 * 256 * 4 + 256 * 8          # stream-K slots and flags (fewer than 1024 tiles)
    assert lib.ddg_workspace_bytes(4096, 3072, 3072, 32, ctypes.byref(b)) == OK and b.value == 4096 * 64 + sk
    assert lib.ddg_workspace_bytes(3, 16, 128, 8, ctypes.byref(b)) == OK and b.value == 256
    assert lib.ddg_workspace_bytes(0, 16, 128, 32, ctypes.byref(b)) == OK and b.value == 0
    # r = 0: the stream-K area of the plain product, where its tiles are few
    assert lib.ddg_workspace_bytes(4096, 3072, 3072, 0, ctypes.byref(b)) == OK and b.value == sk
    assert lib.ddg_workspace_bytes(64, 3072, 3072, 0, ctypes.byref(b)) == OK and b.value == 0
    assert lib.ddg_workspace_bytes(32760, 5120, 5120, 0, ctypes.byref(b)) == OK and b.value == 0
    assert lib.ddg_workspace_bytes(1024, 5120, 5120, 32, ctypes.byref(b)) == OK and b.value == 1024 * 64 + sk
    # 16 tokens, K >= 8192, fewer than 12800 columns: 8 parts x (1 KiB + 8 bytes)
    # per block of 16 columns, blocks padded to a multiple of 4
    split16 = lambda n: 8 * 1024 * ((n // 16 + 3) // 4 * 4) + -(-8 * 8 * ((n // 16 + 3) // 4 * 4) // 256) * 256
    assert lib.ddg_workspace_bytes(16, 5120, 13824, 0, ctypes.byref(b)) == OK and b.value == split16(5120) == 2641920
    assert lib.ddg_workspace_bytes(1, 1040, 8192, 0, ctypes.byref(b)) == OK and b.value == split16(1040)
    # with a rank, at most 64 rows and at least 8 groups: the pre-pass's float32
    # partials after the split-K area (chunks of ceil(G / 32) groups)
    def part(m, k, r):
        g = k // 128
        gpc = -(-g // 32)
        return -(-(-(-g // gpc) * m * r * 4) // 256) * 256 if m <= 64 and g >= 8 else 0
    assert part(16, 13824, 32) == 27 * 16 * 32 * 4 and part(16, 5120, 32) == 20 * 16 * 32 * 4
    assert lib.ddg_workspace_bytes(16, 5120, 13824, 32, ctypes.byref(b)) == OK and \
        b.value == 1024 + split16(5120) + part(16, 13824, 32)
    assert lib.ddg_workspace_bytes(16, 5120, 5120, 32, ctypes.byref(b)) == OK and b.value == 1024 + part(16, 5120, 32)
    assert lib.ddg_workspace_bytes(64, 3072, 1024, 8, ctypes.byref(b)) == OK and b.value == 1024 + 8 * 64 * 8 * 4
    assert lib.ddg_workspace_bytes(16, 5120, 896, 32, ctypes.byref(b)) == OK and b.value == 1024     # 7 groups
    assert lib.ddg_workspace_bytes(65, 3072, 3072, 32, ctypes.byref(b)) == OK and b.value == 4352 + sk
    assert lib.ddg_workspace_bytes(16, 5120, 5120, 0, ctypes.byref(b)) == OK and b.value == 0       # K < 8192
    assert lib.ddg_workspace_bytes(16, 12800, 8192, 0, ctypes.byref(b)) == OK and b.value == 0      # skinny kernel
    assert lib.ddg_workspace_bytes(17, 5120, 13824, 0, ctypes.byref(b)) == OK and b.value == 0      # M > 16
    assert lib.ddg_workspace_bytes(64, -1, 128, 32, ctypes.byref(b)) == E_SHAPE
    assert lib.ddg_workspace_bytes(64, 16, -128, 32, ctypes.byref(b)) == E_SHAPE
    for r in (4, 12, 136, -8):
        assert lib.ddg_workspace_bytes(64, 16, 128, r, ctypes.byref(b)) == E_SHAPE
    assert lib.ddg_workspace_bytes(64, 16, 128, 32, None) == E_ARG


def test_quantize_pack_rejects_bad_arguments(lib):
    q = lib.ddg_quantize_pack
    assert q(FAKE, 0, 16, 128, 9, FAKE, FAKE, None) == E_ARG         # bits
    assert q(FAKE, 7, 16, 128, 4, FAKE, FAKE, None) == E_ARG         # dtype
    assert q(FAKE, 0, 16, 100, 4, FAKE, FAKE, None) == E_SHAPE       # k % 128
    assert q(FAKE, 0, -2, 128, 4, FAKE, FAKE, None) == E_SHAPE
    assert q(None, 0, 16, 128, 4, FAKE, FAKE, None) == E_ARG         # null
    assert q(FAKE, 0, 16, 128, 4, None, FAKE, None) == E_ARG
    assert q(FAKE, 0, 16, 128, 4, FAKE, None, None) == E_ARG
    assert q(MISALIGNED, 0, 16, 128, 4, FAKE, FAKE, None) == E_ALIGN
    assert q(FAKE, 0, 16, 128, 4, FAKE + 8, FAKE, None) == E_ALIGN
    assert q(FAKE, 0, 16, 128, 4, FAKE, FAKE + 2, None) == E_ALIGN
    assert q(None, 0, 0, 128, 4, None, None, None) == OK              # empty: no-op


def test_dequantize_rejects_bad_arguments(lib):
    d = lib.ddg_dequantize
    assert d(FAKE, FAKE, 2, 16, 128, FAKE, None) == E_ARG
    assert d(FAKE, FAKE, 4, 16, 64, FAKE, None) == E_SHAPE
    assert d(None, FAKE, 4, 16, 128, FAKE, None) == E_ARG
    assert d(FAKE, FAKE, 4, 16, 128, MISALIGNED, None) == E_ALIGN
    assert d(None, None, 4, 0, 128, None, None) == OK


def test_dequant_gemm_rejects_bad_arguments(lib):
    gl = lib.ddg_dequant_gemm

    def g(*a, ws=None, wsb=0):
        return gl(*a[:-1], ws, wsb, a[-1])

    assert g(FAKE, 4, 128, FAKE, FAKE, 8, 32, FAKE, 0, None) == E_ARG      # bits
    assert g(FAKE, 4, 128, FAKE, FAKE, 4, 32, FAKE, 5, None) == E_ARG      # y dtype
    assert g(FAKE, 4, 130, FAKE, FAKE, 4, 32, FAKE, 0, None) == E_SHAPE    # k
    assert g(FAKE, 4, 2 ** 20 + 128, FAKE, FAKE, 4, 32, FAKE, 0, None) == E_SHAPE
    assert g(FAKE, 4, 128, FAKE, FAKE, 4, 24, FAKE, 0, None) == E_SHAPE    # n % 16
    assert g(FAKE, 4, 128, FAKE, FAKE, 4, 0, FAKE, 0, None) == E_SHAPE     # n == 0
    assert g(FAKE, -1, 128, FAKE, FAKE, 4, 32, FAKE, 0, None) == E_SHAPE   # m < 0
    assert g(FAKE, 2 ** 31, 128, FAKE, FAKE, 4, 32, FAKE, 0, None) == E_SHAPE
    assert g(None, 4, 128, FAKE, FAKE, 4, 32, FAKE, 0, None) == E_ARG
    assert g(FAKE, 4, 128, None, FAKE, 4, 32, FAKE, 0, None) == E_ARG
    assert g(FAKE, 4, 128, FAKE, None, 4, 32, FAKE, 0, None) == E_ARG
    assert g(FAKE, 4, 128, FAKE, FAKE, 4, 32, None, 0, None) == E_ARG
    assert g(MISALIGNED, 4, 128, FAKE, FAKE, 4, 32, FAKE, 0, None) == E_ALIGN
    assert g(FAKE, 4, 128, FAKE + 4, FAKE, 4, 32, FAKE, 0, None) == E_ALIGN
    assert g(FAKE, 4, 128, FAKE, FAKE + 1, 4, 32, FAKE, 0, None) == E_ALIGN
    assert g(FAKE, 4, 128, FAKE, FAKE, 4, 32, FAKE + 8, 1, None) == E_ALIGN
    assert g(None, 0, 128, None, None, 4, 32, None, 0, None) == OK          # M == 0
    assert g(FAKE, 4, 128, FAKE, FAKE, 4, 32, FAKE, 0, None, ws=FAKE + 8, wsb=1 << 20) == E_ALIGN


def test_grouped_gemm_rejects_bad_arguments(lib):
    g = lib.ddg_dequant_gemm_grouped
    D = api.GemmDesc

    def descs(*items):
        arr = (D * len(items))()
        for i, kw in enumerate(items):
            base = dict(x=FAKE, packed=FAKE, scales=FAKE, y=FAKE, m=4, k=128, n=32, bits=4, y_dtype=0)
            base.update(kw)
            arr[i] = D(**base)
        return arr

    assert g(None, 0, None) == OK                                   # empty group
    assert g(None, 2, None) == E_ARG
    assert g(descs({}), -1, None) == E_SHAPE
    assert g(descs({}), api.MAX_GROUPED + 1, None) == E_SHAPE
    # every descriptor is checked before anything runs; the first bad one decides
    assert g(descs({}, {"bits": 8}), 2, None) == E_ARG
    assert g(descs({}, {"k": 100}), 2, None) == E_SHAPE
    assert g(descs({"n": 24}, {"bits": 8}), 2, None) == E_SHAPE
    assert g(descs({}, {"y": None}), 2, None) == E_ARG
    assert g(descs({}, {"x": MISALIGNED}), 2, None) == E_ALIGN
    assert g(descs({}, {"y_dtype": 3}), 2, None) == E_ARG
    assert g(descs({"m": 0, "x": None, "y": None, "packed": None, "scales": None}), 1, None) == OK


def test_lowrank_fused_gemm_rejects_bad_arguments(lib):
    f = lib.ddg_lowrank_fused_gemm
    base = [FAKE, 64, 256, FAKE, FAKE, 4, 64, FAKE, FAKE, 32, FAKE, 0, FAKE, 64 * 64, None]

    def call(**kw):
        a = list(base)
        idx = {"x": 0, "m": 1, "k": 2, "bits": 5, "n": 6, "down": 7, "up": 8, "r": 9, "y": 10,
               "ydt": 11, "ws": 12, "wsb": 13}
        for k, v in kw.items():
            a[idx[k]] = v
        return f(*a)

    assert call(r=12) == E_SHAPE
    assert call(r=0) == E_SHAPE
    assert call(r=256) == E_SHAPE
    assert call(down=None) == E_ARG
    assert call(up=None) == E_ARG
    assert call(ws=None) == E_ARG
    assert call(down=MISALIGNED) == E_ALIGN
    assert call(ws=MISALIGNED) == E_ALIGN
    assert call(wsb=64 * 64 - 1) == E_WS
    assert call(bits=1) == E_ARG
    assert call(k=100) == E_SHAPE
    # the T pre-pass launches 16 work-items per row: at most 2^28 - 16 rows
    assert call(m=(1 << 28) - 15, wsb=1 << 40) == E_SHAPE
    assert call(m=0, x=None, down=None, up=None, ws=None, y=None) == OK


def test_lowrank_down_rejects_bad_arguments(lib):
    """T = bf16(X L1) alone: shapes, null and misaligned pointers are refused
    on the host before any launch; M == 0 is a no-op."""
    f = lib.ddg_lowrank_down

    def call(x=FAKE, m=64, k=256, down=FAKE, r=32, t=FAKE):
        return f(x, m, k, down, r, t, None)

    assert call(r=12) == E_SHAPE and call(r=0) == E_SHAPE and call(r=136) == E_SHAPE
    assert call(k=100) == E_SHAPE and call(k=0) == E_SHAPE and call(k=2 ** 20 + 128) == E_SHAPE
    assert call(m=-1) == E_SHAPE and call(m=(1 << 28) - 15) == E_SHAPE
    assert call(x=None) == E_ARG and call(down=None) == E_ARG and call(t=None) == E_ARG
    assert call(x=MISALIGNED) == E_ALIGN and call(down=MISALIGNED) == E_ALIGN and call(t=FAKE + 8) == E_ALIGN
    assert call(m=0, x=None, down=None, t=None) == OK


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not found"):
        api.load_library(str(tmp_path / "missing.so"))


def test_rpbh_rotate_rejects_bad_arguments(lib):
    f = lib.ddg_rpbh_rotate
    base = dict(x=FAKE, xdt=0, n=4, d=256, perm=FAKE, signs=FAKE, h=64, out=FAKE + (1 << 20), odt=0)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return f(a["x"], a["xdt"], a["n"], a["d"], a["perm"], a["signs"], a["h"], a["out"], a["odt"], None)

    assert call(xdt=2) == E_ARG and call(odt=-1) == E_ARG
    assert call(d=100) == E_SHAPE                  # d % 64
    assert call(d=api.ROTATE_MAX_D + 64) == E_SHAPE
    assert call(h=48) == E_SHAPE and call(h=1) == E_SHAPE and call(h=2048) == E_SHAPE
    assert call(d=192, h=128) == E_SHAPE           # h does not divide d
    assert call(n=-1) == E_SHAPE
    assert call(x=None) == E_ARG and call(perm=None) == E_ARG and call(signs=None) == E_ARG
    assert call(out=None) == E_ARG
    assert call(x=MISALIGNED) == E_ALIGN and call(out=FAKE + (1 << 20) + 8) == E_ALIGN
    assert call(perm=FAKE + 2) == E_ALIGN
    assert call(out=FAKE + 512, xdt=0, odt=0) == E_ARG            # partial overlap
    assert call(out=FAKE, xdt=0, odt=1) == E_ARG                  # same start, other dtype
    assert call(n=0, x=None, perm=None, signs=None, out=None) == OK


def test_weight_quantizers_bound_the_launch(lib):
    """One lane per 32 weights: the quantizers and the dequantizer take at
    most DDG_CHUNK_WEIGHTS_MAX weights (rows padded to 32 for FP4/FP6), so the
    launch stays below 2^32 work-items.  At the bound the shape passes and the
    null pointer is what is rejected; one row more is a shape error."""
    assert re.search(r"#define DDG_CHUNK_WEIGHTS_MAX \(\(INT64_C\(1\) << 37\) - 8192\)", open(HEADER).read())
    cap = (1 << 37) - 8192
    assert (cap // 32 + 255) // 256 * 256 < 1 << 32
    k = 128
    n_max = cap // k                                  # a multiple of 32
    assert n_max % 32 == 0
    q, d = lib.ddg_quantize_pack, lib.ddg_dequantize
    q4, q6 = lib.ddg_fp4_quantize_pack, lib.ddg_fp6_quantize_pack
    assert q(None, 0, n_max, k, 4, FAKE, FAKE, None) == E_ARG
    assert q(FAKE, 0, n_max + 1, k, 4, FAKE, FAKE, None) == E_SHAPE
    assert d(None, FAKE, 4, n_max, k, FAKE, None) == E_ARG
    assert d(FAKE, FAKE, 4, n_max + 1, k, FAKE, None) == E_SHAPE
    for f in (0, 0x200):                              # row and tiled storage
        assert q4(None, 0, n_max, k, f, FAKE, FAKE, None) == E_ARG
        assert q4(FAKE, 0, n_max + 1, k, f, FAKE, FAKE, None) == E_SHAPE
    assert q6(None, 0, n_max, k, 0, FAKE, FAKE, None) == E_ARG
    assert q6(FAKE, 0, n_max + 1, k, 0, FAKE, FAKE, None) == E_SHAPE
    assert q(FAKE, 0, n_max // 2, 2 * k + 128, 4, FAKE, FAKE, None) == E_SHAPE   # the product counts


def test_fp4_and_w4a8_calls_reject_bad_arguments(lib):
    q = lib.ddg_fp4_quantize_pack
    assert q(FAKE, 0, 4, 128, 3, FAKE, FAKE, None) == E_ARG           # fmt
    assert q(FAKE, 0, 4, 128, 0x103, FAKE, FAKE, None) == E_ARG       # power-of-two flag, bad format
    assert q(FAKE, 0, 4, 128, 0x400, FAKE, FAKE, None) == E_ARG       # unknown flag
    assert q(FAKE, 0, 4, 128, 0x303, FAKE, FAKE, None) == E_ARG       # both flags, bad format
    assert q(None, 0, 0, 128, 0x302, None, None, None) == OK          # both flags accepted
    assert q(FAKE, 2, 4, 128, 0, FAKE, FAKE, None) == E_ARG           # dtype
    assert q(FAKE, 0, 4, 100, 0, FAKE, FAKE, None) == E_SHAPE
    assert q(FAKE, 0, -1, 128, 0, FAKE, FAKE, None) == E_SHAPE
    assert q(None, 0, 4, 128, 0, FAKE, FAKE, None) == E_ARG
    assert q(MISALIGNED, 0, 4, 128, 0, FAKE, FAKE, None) == E_ALIGN
    assert q(FAKE, 0, 4, 128, 0, FAKE + 8, FAKE, None) == E_ALIGN
    assert q(None, 0, 0, 128, 0, None, None, None) == OK
    r = lib.ddg_fp8_quantize_rows
    assert r(FAKE, 4, 100, FAKE, FAKE, None) == E_SHAPE
    assert r(FAKE, -1, 128, FAKE, FAKE, None) == E_SHAPE
    assert r(None, 4, 128, FAKE, FAKE, None) == E_ARG
    assert r(MISALIGNED, 4, 128, FAKE, FAKE, None) == E_ALIGN
    assert r(FAKE, 4, 128, FAKE + 4, FAKE, None) == E_ALIGN
    assert r(None, 0, 128, None, None, None) == OK
    g = lib.ddg_w4a8_gemm
    base = [FAKE, FAKE, 4, 128, FAKE, FAKE, 0, 32, FAKE, 0, None]

    def call(**kw):
        a = list(base)
        idx = {"xq": 0, "xs": 1, "m": 2, "k": 3, "packed": 4, "ws": 5, "fmt": 6, "n": 7, "y": 8, "ydt": 9}
        for key, v in kw.items():
            a[idx[key]] = v
        return g(*a)

    assert call(fmt=5) == E_ARG and call(ydt=3) == E_ARG
    assert call(fmt=0x103) == E_ARG and call(fmt=0x400) == E_ARG and call(fmt=0x203) == E_ARG
    assert call(fmt=0x101, m=0, xq=None) == OK and call(fmt=0x302, m=0, xq=None) == OK

    r6 = lib.ddg_fp6_quantize_rows
    assert r6(FAKE, 4, 128, 2, FAKE, FAKE, None) == E_ARG               # fp6 format
    assert r6(FAKE, 4, 100, 0, FAKE, FAKE, None) == E_SHAPE
    assert r6(FAKE, -1, 128, 0, FAKE, FAKE, None) == E_SHAPE
    assert r6(None, 4, 128, 1, FAKE, FAKE, None) == E_ARG
    assert r6(MISALIGNED, 4, 128, 0, FAKE, FAKE, None) == E_ALIGN
    assert r6(FAKE, 4, 128, 0, FAKE + 8, FAKE, None) == E_ALIGN
    assert r6(None, 0, 128, 0, None, None, None) == OK
    g6 = lib.ddg_w4a6_gemm
    base6 = [FAKE, FAKE, 4, 128, 0, FAKE, FAKE, 0x200, 32, FAKE, 0, None]

    def call6(**kw):
        a = list(base6)
        idx = {"xq": 0, "xs": 1, "m": 2, "k": 3, "f6": 4, "packed": 5, "ws": 6, "fmt": 7, "n": 8, "y": 9, "ydt": 10}
        for key, v in kw.items():
            a[idx[key]] = v
        return g6(*a)

    assert call6(f6=2) == E_ARG and call6(fmt=5) == E_ARG and call6(ydt=3) == E_ARG
    assert call6(fmt=0) == E_ARG and call6(fmt=0x101) == E_ARG and call6(fmt=0x203) == E_ARG   # tiled storage only
    assert call6(fmt=0x201, m=0, xq=None) == OK and call6(fmt=0x302, m=0, xq=None) == OK
    assert call6(k=130) == E_SHAPE and call6(n=0) == E_SHAPE and call6(m=-1) == E_SHAPE
    assert call6(xq=None) == E_ARG and call6(y=None) == E_ARG
    assert call6(xq=MISALIGNED) == E_ALIGN
    assert call6(m=0, xq=None) == OK and call6(m=0, fmt=0x300, xq=None) == OK
    assert call(k=130) == E_SHAPE and call(k=2 ** 20 + 128) == E_SHAPE
    assert call(n=0) == E_SHAPE and call(m=-1) == E_SHAPE
    assert call(xq=None) == E_ARG and call(packed=None) == E_ARG and call(y=None) == E_ARG
    assert call(xq=MISALIGNED) == E_ALIGN and call(packed=FAKE + 8) == E_ALIGN
    assert call(ws=FAKE + 2) == E_ALIGN and call(y=FAKE + 1) == E_ALIGN
    assert call(m=0, xq=None, xs=None, packed=None, ws=None, y=None) == OK

    # FP6 weights: quantizer and W6A8 product
    q6 = lib.ddg_fp6_quantize_pack
    assert q6(FAKE, 0, 4, 128, 2, FAKE, FAKE, None) == E_ARG                # fp6 format
    assert q6(FAKE, 0, 4, 128, 0x200, FAKE, FAKE, None) == E_ARG            # no tiled flag: always tiled
    assert q6(FAKE, 2, 4, 128, 0, FAKE, FAKE, None) == E_ARG                # dtype
    assert q6(FAKE, 0, 4, 100, 0, FAKE, FAKE, None) == E_SHAPE
    assert q6(FAKE, 0, -1, 128, 1, FAKE, FAKE, None) == E_SHAPE
    assert q6(FAKE, 0, 4, 128, 0x101, None, FAKE, None) == E_ARG
    assert q6(MISALIGNED, 0, 4, 128, 0, FAKE, FAKE, None) == E_ALIGN
    assert q6(FAKE, 1, 4, 128, 0, FAKE + 8, FAKE, None) == E_ALIGN
    assert q6(None, 0, 0, 128, 0x100, None, None, None) == OK
    g8 = lib.ddg_w6a8_gemm
    base8 = [FAKE, FAKE, 4, 128, FAKE, FAKE, 0, 32, FAKE, 0, None]

    def call8(**kw):
        a = list(base8)
        idx = {"xq": 0, "xs": 1, "m": 2, "k": 3, "packed": 4, "ws": 5, "f6": 6, "n": 7, "y": 8, "ydt": 9}
        for key, v in kw.items():
            a[idx[key]] = v
        return g8(*a)

    assert call8(f6=2) == E_ARG and call8(f6=0x200) == E_ARG and call8(ydt=3) == E_ARG
    assert call8(k=130) == E_SHAPE and call8(k=2 ** 20 + 128) == E_SHAPE and call8(n=0) == E_SHAPE
    assert call8(m=-1) == E_SHAPE
    assert call8(xq=None) == E_ARG and call8(packed=None) == E_ARG and call8(y=None) == E_ARG
    assert call8(xq=MISALIGNED) == E_ALIGN and call8(packed=FAKE + 8) == E_ALIGN and call8(y=FAKE + 1) == E_ALIGN
    assert call8(m=0, xq=None, xs=None, packed=None, ws=None, y=None) == OK
    assert call8(m=0, f6=0x101, xq=None) == OK


def test_noalloc_lowrank_host_checks(lib):
    """The workspace-free low-rank product refuses, on the host and before
    any launch, a T larger than the library's device array (8 MiB: M * r up
    to 4,194,304) and the shapes the workspace call refuses."""
    FAKE = 1 << 20
    def call(m=16, k=128, bits=4, n=16, r=32, ld=FAKE, y=FAKE):
        return lib.ddg_lowrank_fused_gemm_noalloc(FAKE, m, k, FAKE, FAKE, bits, n, ld, FAKE, r, y, 0, None)
    assert call(m=32769, r=128) == E_WS
    assert call(m=4194305, r=8) == E_WS
    assert call(r=4) == E_SHAPE and call(r=136) == E_SHAPE and call(r=12) == E_SHAPE
    assert call(k=100) == E_SHAPE and call(n=20) == E_SHAPE and call(bits=8) == E_ARG
    assert call(ld=0) == E_ARG and call(ld=FAKE + 8) == E_ALIGN
    assert call(m=0) == OK


def test_row_quantizers_and_error_tables_bound_their_rows(lib):
    """One workgroup per row (or per 16 rows): row counts whose launch would
    pass 2^32 work-items are refused on the host before anything is launched."""
    FAKE = 1 << 20
    # at the largest accepted count the shape check passes and the null output
    # is refused next (E_ARG): nothing is launched, with or without a GPU
    assert lib.ddg_fp8_quantize_rows(FAKE, (1 << 24) - 1, 128, None, FAKE, None) == E_ARG
    assert lib.ddg_fp8_quantize_rows(FAKE, 1 << 24, 128, FAKE, FAKE, None) == E_SHAPE
    assert lib.ddg_fp6_quantize_rows(FAKE, (1 << 26) - 32, 128, 0, None, FAKE, None) == E_ARG
    assert lib.ddg_fp6_quantize_rows(FAKE, (1 << 26) - 31, 128, 0, FAKE, FAKE, None) == E_SHAPE
    assert lib.ddg_quant_sse(FAKE, 0, (1 << 24) - 1, 128, FAKE, None, None) == E_ARG
    assert lib.ddg_quant_sse(FAKE, 0, 1 << 24, 128, FAKE, FAKE, None) == E_SHAPE


def test_record_round_trip_and_rejections():
    """The stored record's four fields ([WDQ] §3.3): state_dict -> from_state_dict
    keeps them, and records whose fields disagree are refused on the host."""
    n, k, bits = 48, 384, 5
    pb = n * k * bits // 8
    qw = api.QWeight(torch.arange(pb, dtype=torch.int64).to(torch.uint8), torch.ones((n, k // 128)),
                     bits, n, k, 300)
    sd = qw.state_dict("blocks.0.attn.q")
    assert set(sd) == {f"blocks.0.attn.q_{f}" for f in ("packed", "scales", "bw", "nin")}
    assert sd["blocks.0.attn.q_bw"].dtype == torch.int8 and sd["blocks.0.attn.q_nin"].dtype == torch.int32
    back = api.QWeight.from_state_dict(sd, "blocks.0.attn.q", orig_in=300, device="cpu")
    assert (back.n, back.k, back.bits, back.orig_in) == (n, k, bits, 300)
    assert torch.equal(back.packed, qw.packed) and torch.equal(back.scales, qw.scales)

    def bad(**change):
        d = dict(sd)
        for key, v in change.items():
            d[f"blocks.0.attn.q_{key}"] = v
        with pytest.raises(ValueError):
            api.QWeight.from_state_dict(d, "blocks.0.attn.q", device="cpu")
    bad(bw=torch.tensor(8, dtype=torch.int8))
    bad(bw=torch.tensor(2, dtype=torch.int8))
    bad(bw=torch.tensor(4, dtype=torch.int8))                 # bytes of a 5-bit record
    bad(nin=torch.tensor(400, dtype=torch.int32))
    bad(nin=torch.tensor(1280, dtype=torch.int32))            # scales no longer whole rows
    bad(packed=sd["blocks.0.attn.q_packed"][:-1])             # truncated
    bad(scales=sd["blocks.0.attn.q_scales"].reshape(-1)[:-3])
    bad(scales=sd["blocks.0.attn.q_scales"].double())
    with pytest.raises(ValueError):
        api.QWeight.from_state_dict(sd, "blocks.0.attn.q", orig_in=200, device="cpu")
