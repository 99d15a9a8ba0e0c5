"""Host-side tests of libgrinqh.so that need no GPU.

They check that the library loads, that it exports every function
include/grinqh.h declares, the pure-host layout arithmetic, and that argument
checks reject bad calls with the documented status before touching a device
(every call here fails a host check, so no kernel is ever launched).
"""

import ctypes
import os
import re
import subprocess

import pytest

import input_adaptive_bit_amd as G
from input_adaptive_bit_amd import grinqh as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grinqh.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(grinqh_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_function():
    lib = G.load()
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert set(declared) == set(B.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (grinqh_[a-z_]+)\b", out))
    assert set(declared) <= exported


def test_library_has_gfx950_code_object():
    """The library built here carries a gfx950 device code object."""
    with open(B.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_version_and_status_strings():
    assert G.load().grinqh_version() >= 100
    for st in range(6):
        assert isinstance(G.status_string(st), str) and G.status_string(st)


@pytest.mark.parametrize("d_in,d_out,b_max,words", [(1024, 1024, 8, 64), (4096, 14336, 8, 896),
                                                   (7, 1, 4, 4), (3, 65, 2, 8), (5, 128, 6, 8)])
def test_layout_init_and_packed_bytes(d_in, d_out, b_max, words):
    L = G.grinqh_layout_init(d_in, d_out, b_max)
    assert (L.d_in, L.d_out, L.b_max, L.n_planes, L.row_words) == (d_in, d_out, b_max, b_max // 2, words)
    assert G.grinqh_packed_bytes(L) == d_in * (b_max // 2) * words * 4


@pytest.mark.parametrize("d_in,d_out,b_max", [(0, 10, 8), (10, 0, 8), (10, 10, 3), (10, 10, 10),
                                              (10, 10, 0), ((1 << 20) + 1, 10, 8), (-4, 5, 4)])
def test_layout_init_rejects(d_in, d_out, b_max):
    L = B.Layout()
    st = G.load().grinqh_layout_init(d_in, d_out, b_max, ctypes.byref(L))
    assert st == B.GRINQH_EINVAL
    assert G.load().grinqh_layout_init(8, 8, 8, None) == B.GRINQH_EINVAL


def test_inconsistent_layout_is_rejected_everywhere():
    lib = G.load()
    L = G.grinqh_layout_init(64, 64, 8)
    L.row_words = 5
    assert lib.grinqh_packed_bytes(ctypes.byref(L)) == 0
    assert lib.grinqh_gemv_workspace_bytes(ctypes.byref(L)) == 0
    p = 4096
    assert lib.grinqh_pack(ctypes.byref(L), p, p, None) == B.GRINQH_EINVAL
    assert lib.grinqh_gemv(ctypes.byref(L), p, 0, p, p, p, p, p + 100000, 1, p * 4, 1 << 20, None) \
        == B.GRINQH_EINVAL


def test_argument_checks_before_any_device_call():
    """Fake (never dereferenced) addresses: every call below fails a host check."""
    lib = G.load()
    L = G.grinqh_layout_init(256, 128, 8)
    Lp = ctypes.byref(L)
    A = 1 << 16          # 64 KiB-aligned fake addresses
    X, TH, PL, S, Z, Y, WS = (A * k for k in range(1, 8))
    ok = lambda **kw: dict(dict(x=X, xd=0, th=TH, pl=PL, s=S, z=Z, y=Y, yd=1, ws=WS, wsb=1 << 30), **kw)

    def gemv(a):
        return lib.grinqh_gemv(Lp, a["x"], a["xd"], a["th"], a["pl"], a["s"], a["z"], a["y"], a["yd"],
                               a["ws"], a["wsb"], None)

    for key in ("x", "th", "pl", "s", "z", "y", "ws"):
        assert gemv(ok(**{key: None})) == B.GRINQH_EINVAL, key
    assert gemv(ok(xd=7)) == B.GRINQH_EINVAL
    assert gemv(ok(yd=-1)) == B.GRINQH_EINVAL
    assert gemv(ok(pl=PL + 4)) == B.GRINQH_EALIGN
    assert gemv(ok(x=X + 1)) == B.GRINQH_EALIGN
    assert gemv(ok(xd=1, x=X + 2)) == B.GRINQH_EALIGN
    assert gemv(ok(y=Y + 2)) == B.GRINQH_EALIGN
    assert gemv(ok(s=S + 1)) == B.GRINQH_EALIGN
    assert gemv(ok(ws=WS + 16)) == B.GRINQH_EALIGN
    assert gemv(ok(th=TH + 2)) == B.GRINQH_EALIGN
    assert gemv(ok(y=X + 128)) == B.GRINQH_EINVAL          # y overlaps x
    assert lib.grinqh_gemv(None, X, 0, TH, PL, S, Z, Y, 1, WS, 1 << 30, None) == B.GRINQH_EINVAL
    # the planes of one GEMV must stay below 2 GiB: 2^19 channels x 4 planes x 1 KiB rows is 2 GiB
    big = G.grinqh_layout_init(1 << 19, 4096, 8)
    assert G.grinqh_packed_bytes(big) == 1 << 31
    assert lib.grinqh_gemv(ctypes.byref(big), X, 0, TH, PL, S, Z, Y, 1, WS, 1 << 40, None) == B.GRINQH_EINVAL

    # the no-allocation variant runs the same operand checks
    def noalloc(a):
        return lib.grinqh_gemv_noalloc(Lp, a["x"], a["xd"], a["th"], a["pl"], a["s"], a["z"], a["y"], a["yd"],
                                       None)

    for key in ("x", "th", "pl", "s", "z", "y"):
        assert noalloc(ok(**{key: None})) == B.GRINQH_EINVAL, key
    assert noalloc(ok(xd=7)) == B.GRINQH_EINVAL
    assert noalloc(ok(pl=PL + 4)) == B.GRINQH_EALIGN
    assert noalloc(ok(y=Y + 2)) == B.GRINQH_EALIGN
    assert noalloc(ok(y=X + 128)) == B.GRINQH_EINVAL
    assert lib.grinqh_gemv_noalloc(None, X, 0, TH, PL, S, Z, Y, 1, None) == B.GRINQH_EINVAL
    assert lib.grinqh_gemv_noalloc(ctypes.byref(big), X, 0, TH, PL, S, Z, Y, 1, None) == B.GRINQH_EINVAL

    assert lib.grinqh_pack(Lp, None, PL, None) == B.GRINQH_EINVAL
    assert lib.grinqh_pack(Lp, X, None, None) == B.GRINQH_EINVAL
    assert lib.grinqh_pack(Lp, X, PL + 8, None) == B.GRINQH_EALIGN

    assert lib.grinqh_assign_bits(Lp, None, 0, TH, Y, None, None, None) == B.GRINQH_EINVAL
    assert lib.grinqh_assign_bits(Lp, X, 0, None, Y, None, None, None) == B.GRINQH_EINVAL
    assert lib.grinqh_assign_bits(Lp, X, 0, TH, None, None, None, None) == B.GRINQH_EINVAL
    assert lib.grinqh_assign_bits(Lp, X, 5, TH, Y, None, None, None) == B.GRINQH_EINVAL
    assert lib.grinqh_assign_bits(Lp, X + 1, 0, TH, Y, None, None, None) == B.GRINQH_EALIGN
    assert lib.grinqh_assign_bits(Lp, X, 0, TH, Y, S + 2, None, None) == B.GRINQH_EALIGN

    assert lib.grinqh_debug_codes(Lp, None, PL, Y, None) == B.GRINQH_EINVAL
    assert lib.grinqh_debug_codes(Lp, X, PL + 4, Y, None) == B.GRINQH_EALIGN


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        B.load(str(tmp_path / "missing.so"))


def test_group_argument_checks_before_any_device_call():
    lib = G.load()
    A = 1 << 16
    Ls = [G.grinqh_layout_init(256, 128, 8), G.grinqh_layout_init(128, 64, 8)]
    arr = (B.Layout * 2)(*Ls)
    ops = (B.Operands * 2)(B.Operands(A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A),
                           B.Operands(7 * A, 8 * A, 9 * A, 10 * A, 11 * A, 12 * A))
    WS = 13 * A
    call = lambda n=2, a=arr, o=ops, xd=0, yd=0, ws=WS: lib.grinqh_gemv_group(a, o, n, xd, yd, ws, 1 << 30, None)
    assert call(n=0) == B.GRINQH_EINVAL
    assert call(n=9) == B.GRINQH_EINVAL
    assert call(a=None) == B.GRINQH_EINVAL
    assert call(o=None) == B.GRINQH_EINVAL
    assert call(xd=3) == B.GRINQH_EINVAL
    assert call(ws=None) == B.GRINQH_EINVAL
    assert call(ws=WS + 8) == B.GRINQH_EALIGN
    bad = (B.Layout * 2)(Ls[0], G.grinqh_layout_init(128, 64, 4))           # mixed b_max
    assert call(a=bad) == B.GRINQH_EINVAL
    o2 = (B.Operands * 2)(ops[0], B.Operands(7 * A, 8 * A, 9 * A + 4, 10 * A, 11 * A, 12 * A))
    assert call(o=o2) == B.GRINQH_EALIGN                                     # planes misaligned
    o3 = (B.Operands * 2)(ops[0], B.Operands(7 * A, 8 * A, 9 * A, 10 * A, 11 * A, 6 * A + 64))
    assert call(o=o3) == B.GRINQH_EINVAL                                     # outputs overlap
    o4 = (B.Operands * 2)(ops[0], B.Operands(7 * A, 8 * A, 9 * A, 10 * A, 11 * A, A + 16))
    assert call(o=o4) == B.GRINQH_EINVAL                                     # output overlaps an input
    o5 = (B.Operands * 2)(ops[0], B.Operands(None, 8 * A, 9 * A, 10 * A, 11 * A, 12 * A))
    assert call(o=o5) == B.GRINQH_EINVAL
    assert lib.grinqh_gemv_group_workspace_bytes(bad, 2) == 0
    assert lib.grinqh_gemv_group_workspace_bytes(arr, 0) == 0


def test_calibration_argument_checks_before_any_device_call():
    lib = G.load()
    A = 1 << 16
    X, TH, WS = A, 2 * A, 3 * A
    wsb = lib.grinqh_calibrate_workspace_bytes()
    assert wsb >= 8 * 2048 * 4 and wsb % 256 == 0

    def call(x=X, xd=0, n=1000, levels=(0.2, 0.5), nl=None, th=TH, ws=WS, b=wsb):
        lv = (ctypes.c_double * max(1, len(levels)))(*levels)
        return lib.grinqh_calibrate_thresholds(x, xd, n, lv, len(levels) if nl is None else nl, th, ws, b, None)

    assert call(x=None) == B.GRINQH_EINVAL
    assert call(th=None) == B.GRINQH_EINVAL
    assert call(ws=None) == B.GRINQH_EINVAL
    assert lib.grinqh_calibrate_thresholds(X, 0, 10, None, 1, TH, WS, wsb, None) == B.GRINQH_EINVAL
    assert call(xd=2) == B.GRINQH_EINVAL
    assert call(n=0) == B.GRINQH_EINVAL
    assert call(n=-5) == B.GRINQH_EINVAL
    assert call(n=1 << 32) == B.GRINQH_EINVAL
    assert call(levels=(), nl=0) == B.GRINQH_EINVAL
    assert call(levels=(0.1, 0.2, 0.3, 0.4, 0.5)) == B.GRINQH_EINVAL
    assert call(levels=(0.2, 1.5)) == B.GRINQH_EINVAL
    assert call(levels=(-0.01,)) == B.GRINQH_EINVAL
    assert call(levels=(float("nan"),)) == B.GRINQH_EINVAL
    assert call(x=X + 1) == B.GRINQH_EALIGN
    assert call(xd=1, x=X + 2) == B.GRINQH_EALIGN
    assert call(th=TH + 2) == B.GRINQH_EALIGN
    assert call(ws=WS + 64) == B.GRINQH_EALIGN
    assert call(b=wsb - 1) == B.GRINQH_ENOSPACE


def test_rtn_argument_checks_before_any_device_call():
    lib = G.load()
    A = 1 << 16
    W, Q, S_, Z = A, 2 * A, 3 * A, 4 * A
    call = lambda d_in=64, d_out=8, b=8, w=W, q=Q, s=S_, z=Z: lib.grinqh_quantize_rtn(d_in, d_out, b, w, q, s, z, None)
    for key in ("w", "q", "s", "z"):
        assert call(**{key: None}) == B.GRINQH_EINVAL, key
    assert call(d_in=0) == B.GRINQH_EINVAL
    assert call(d_out=0) == B.GRINQH_EINVAL
    assert call(d_out=(1 << 30) + 1) == B.GRINQH_EINVAL
    assert call(d_in=(1 << 30) + 1) == B.GRINQH_EINVAL          # keeps the kernel's 32-bit row index in range
    for b in (0, 1, 3, 5, 7, 9, 10):
        assert call(b=b) == B.GRINQH_EINVAL, b
    assert call(w=W + 1) == B.GRINQH_EALIGN
    assert call(s=S_ + 1) == B.GRINQH_EALIGN
    assert call(z=Z + 1) == B.GRINQH_EALIGN


def test_prefill_argument_checks_before_any_device_call():
    lib = G.load()
    A = 1 << 20          # 1 MiB-aligned fake addresses, far enough apart for M x d_in
    L = G.grinqh_layout_init(64, 130, 8)
    Lp = ctypes.byref(L)
    X, PL, S, Z, Y, WS = A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A
    assert lib.grinqh_prefill_workspace_bytes(1) == 256
    assert lib.grinqh_prefill_workspace_bytes(65) == 512
    assert lib.grinqh_prefill_workspace_bytes(0) == 0

    def call(L=Lp, x=X, xd=0, M=16, pl=PL, s=S, z=Z, y=Y, yd=1, ws=WS, b=1 << 20):
        return lib.grinqh_prefill_gemm(L, x, xd, M, pl, s, z, y, yd, ws, b, None)

    for key in ("x", "pl", "s", "z", "y", "ws", "L"):
        assert call(**{key: None}) == B.GRINQH_EINVAL, key
    assert call(xd=1) == B.GRINQH_EINVAL                  # the matrix cores take bf16 x
    assert call(yd=7) == B.GRINQH_EINVAL
    assert call(M=0) == B.GRINQH_EINVAL
    assert call(M=(1 << 20) + 1) == B.GRINQH_EINVAL
    odd = G.grinqh_layout_init(60, 130, 8)                 # d_in not a multiple of 8
    assert call(L=ctypes.byref(odd)) == B.GRINQH_EINVAL
    bad = B.Layout(64, 130, 8, 4, 8)                        # row_words inconsistent (12)
    assert call(L=ctypes.byref(bad)) == B.GRINQH_EINVAL
    assert call(x=X + 8) == B.GRINQH_EALIGN
    assert call(pl=PL + 4) == B.GRINQH_EALIGN
    assert call(y=Y + 2) == B.GRINQH_EALIGN                 # fp32 y
    assert call(ws=WS + 16) == B.GRINQH_EALIGN
    assert call(b=255) == B.GRINQH_ENOSPACE
    assert call(y=X + 64) == B.GRINQH_EINVAL                # y overlaps x
    big = G.grinqh_layout_init(1 << 20, 4096, 8)           # 4 GiB of planes
    assert call(L=ctypes.byref(big), M=1, b=1 << 30) == B.GRINQH_EINVAL


def test_force_launch_argument_checks():
    """The test override of the launch shape rejects values outside its
    documented sets, and accepts (then clears) valid ones; host only."""
    import input_adaptive_bit_amd as B
    lib = B.load()
    for bad in [(3, 0, 0), (16, 0, 0), (-1, 0, 0), (0, -1, 0), (0, 257, 0), (0, 0, 4), (0, 0, -1)]:
        assert lib.grinqh_debug_force_launch(*bad) == 1, bad   # GRINQH_EINVAL
    for good in [(1, 7, 1), (8, 256, 3), (2, 64, 2), (0, 0, 0)]:
        assert lib.grinqh_debug_force_launch(*good) == 0, good   # GRINQH_OK


def test_multiply_high_tile_split_is_exact_where_the_host_uses_it():
    """The GEMV takes a workgroup's tile as the high word of item * m with
    m = ceil(2^32 / n_splits), and the host uses that only while
    n_tiles * n_splits * n_splits < 2^32 (otherwise the kernel divides).
    Within that bound the quotient is exact: checked at the bound's edges
    and on random items for many slice counts."""
    import numpy as np
    rng = np.random.default_rng(5)
    for n in list(range(2, 300)) + [1023, 4096, 4097, 16383, 65535]:
        m = ((1 << 32) + n - 1) // n
        n_items_max = ((1 << 32) - 1) // n          # items * n < 2^32
        a = np.concatenate([np.arange(min(n_items_max, 3 * n)), rng.integers(0, n_items_max, 2000),
                            [n_items_max - 1]]).astype(np.uint64)
        q = (a * np.uint64(m)) >> np.uint64(32)
        assert np.array_equal(q, a // np.uint64(n)), n
