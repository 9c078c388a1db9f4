"""The C ABI library loads, exports every declared symbol and rejects bad
arguments before touching the GPU (CPU only: no call here reaches a launch)."""
import ctypes
import os
import re

import pytest

from combine_moe_route_topk_amd import _lib
from oracle.dispatch import resolve_sorted as oracle_resolve_sorted

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_dc.h")
lib = _lib.lib
ARG, UNSUP, WS = _lib.MOE_ERR_ARG, _lib.MOE_ERR_UNSUPPORTED, _lib.MOE_ERR_WORKSPACE
FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for name in names:
        assert hasattr(raw, name), name
    assert set(names) == set(_lib.SIGNATURES), "binding signatures must mirror the header"


def test_version_and_error_string():
    assert lib.moe_abi_version() == 1
    assert lib.moe_route_topk(None, 4, 8, 0, 1, None, None, None) == ARG
    assert b"k" in lib.moe_last_error()
    out = ctypes.c_int32()
    assert lib.moe_resolve_sorted(1, 5, 1, ctypes.byref(out)) == 0
    assert lib.moe_last_error() == b""


@pytest.mark.parametrize("sort", [-1, 0, 1])
@pytest.mark.parametrize("n", [0, 1, 2, 127, 128, 129, 256, 257, 4096])
@pytest.mark.parametrize("cutoff", [-3, 0, 1, 128, 256])
def test_resolve_sorted_matches_oracle(sort, n, cutoff):
    out = ctypes.c_int32(-1)
    assert lib.moe_resolve_sorted(sort, n, cutoff, ctypes.byref(out)) == 0
    assert bool(out.value) == oracle_resolve_sorted(sort, n, cutoff)


def test_resolve_sorted_errors():
    out = ctypes.c_int32()
    assert lib.moe_resolve_sorted(2, 5, 1, ctypes.byref(out)) == ARG
    assert lib.moe_resolve_sorted(1, -1, 1, ctypes.byref(out)) == ARG
    assert lib.moe_resolve_sorted(1, 5, 1, None) == ARG


def test_route_errors():
    f = lib.moe_route_topk
    assert f(FAKE, -1, 8, 2, 1, FAKE, FAKE, None) == ARG
    assert f(FAKE, 4, 0, 1, 1, FAKE, FAKE, None) == ARG
    assert f(FAKE, 4, 8, 9, 1, FAKE, FAKE, None) == ARG
    assert f(FAKE, 4, 2048, 8, 1, FAKE, FAKE, None) == UNSUP
    assert f(FAKE, 4, 128, 65, 1, FAKE, FAKE, None) == UNSUP
    assert f(None, 4, 8, 2, 1, FAKE, FAKE, None) == ARG
    assert f(FAKE, 4, 8, 2, 1, None, FAKE, None) == ARG
    assert f(None, 0, 8, 2, 1, None, None, None) == 0          # N == 0: no-op, no launch


def test_workspace_sizing():
    f = lib.moe_dispatch_workspace_bytes
    assert f(4096, 256, 8, 1) > 0
    assert f(4096, 256, 8, 8) == f(4096, 256, 8, 1) or f(4096, 256, 8, 8) > 0
    assert f(0, 8, 2, 1) > 0
    for bad in ((-1, 8, 2, 1), (4, 0, 1, 1), (4, 8, 9, 1), (4, 8, 2, 3), (4, 8, 2, 0),
                (4, 2048, 2, 1), (2**31, 8, 2, 1)):
        assert f(*bad) == 0, bad
    # grows with the number of chunks
    assert f(1 << 20, 256, 8, 1) > f(4096, 256, 8, 1)
    assert lib.moe_grouped_swiglu_workspace_bytes(16384, 8, 4096, 14336) >= 16384 * 14336 * 2


def _dispatch(**kw):
    a = dict(x=FAKE, x_scales=None, dtype=1, n=4, d=64, idx=FAKE, e=8, k=2, g=1, sort=1,
             cutoff=256, used=None, rows=FAKE, row_scales=None, counts=FAKE, offs=FAKE,
             segs=FAKE, src=FAKE, dst=FAKE, rexp=FAKE, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return lib.moe_dispatch(a["x"], a["x_scales"], a["dtype"], a["n"], a["d"], a["idx"], a["e"],
                            a["k"], a["g"], a["sort"], a["cutoff"], a["used"], a["rows"],
                            a["row_scales"], a["counts"], a["offs"], a["segs"], a["src"],
                            a["dst"], a["rexp"], a["ws"], a["wsb"], None)


def test_dispatch_errors():
    assert _dispatch(n=-1) == ARG
    assert _dispatch(k=9) == ARG
    assert _dispatch(e=2048) == UNSUP
    assert _dispatch(k=65, e=128) == UNSUP
    assert _dispatch(g=3) == ARG
    assert _dispatch(g=0) == ARG
    assert _dispatch(d=0) == ARG
    assert _dispatch(dtype=7) == ARG
    assert _dispatch(sort=5) == ARG
    assert _dispatch(rows=None) == ARG                     # x without rows
    assert _dispatch(x=None) == ARG                        # rows without x
    assert _dispatch(dtype=2, d=100) == ARG                # F8 needs D % 128 == 0
    assert _dispatch(dtype=2, d=128) == ARG                # F8 needs scales
    assert _dispatch(x_scales=FAKE, row_scales=FAKE) == ARG   # scales only for F8
    assert _dispatch(counts=None) == ARG
    assert _dispatch(src=None) == ARG
    assert _dispatch(idx=None) == ARG
    assert _dispatch(ws=None) == WS
    assert _dispatch(wsb=16) == WS
    assert _dispatch(ws=ctypes.c_void_p(0x1004)) == WS     # misaligned
    assert _dispatch(n=2**30, k=4, e=8) == UNSUP           # NK beyond int32


def test_combine_errors():
    f = lib.moe_combine
    assert f(FAKE, 1, -1, 64, 2, FAKE, FAKE, FAKE, 1, None) == ARG
    assert f(FAKE, 1, 4, 0, 2, FAKE, FAKE, FAKE, 1, None) == ARG
    assert f(FAKE, 1, 4, 64, 0, FAKE, FAKE, FAKE, 1, None) == ARG
    assert f(FAKE, 1, 4, 64, 65, FAKE, FAKE, FAKE, 1, None) == UNSUP
    assert f(FAKE, 2, 4, 64, 2, FAKE, FAKE, FAKE, 1, None) == ARG   # F8 y not accepted
    assert f(FAKE, 1, 4, 64, 2, FAKE, FAKE, FAKE, 5, None) == ARG
    assert f(None, 1, 4, 64, 2, FAKE, FAKE, FAKE, 1, None) == ARG
    assert f(None, 1, 0, 64, 2, None, None, None, 1, None) == 0      # N == 0


def test_dequant_and_swiglu_errors():
    assert lib.moe_dequant_rows(FAKE, FAKE, 4, 100, FAKE, None) == ARG
    assert lib.moe_dequant_rows(None, FAKE, 4, 128, FAKE, None) == ARG
    assert lib.moe_dequant_rows(ctypes.c_void_p(0x1001), FAKE, 4, 128, FAKE, None) == ARG
    g = lib.moe_grouped_swiglu
    assert g(FAKE, 16, 100, FAKE, 8, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 30, None) == UNSUP
    assert g(FAKE, -1, 64, FAKE, 8, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 30, None) == ARG
    assert g(None, 16, 64, FAKE, 8, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 30, None) == ARG
    assert g(FAKE, 16, 64, FAKE, 8, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 16, None) == WS
    odd = ctypes.c_void_p(0x1008)    # 8-byte aligned only: the operands are read in 16-byte runs
    assert g(odd, 16, 64, FAKE, 8, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 30, None) == UNSUP
    assert g(FAKE, 16, 64, FAKE, 8, FAKE, FAKE, odd, 128, FAKE, FAKE, 1 << 30, None) == UNSUP
    assert g(FAKE, 16, 64, FAKE, 8, FAKE, FAKE, FAKE, 128, odd, FAKE, 1 << 30, None) == UNSUP
    assert b"16-byte" in lib.moe_last_error()
    # K above 2^22 (32-bit per-lane load offsets within a 256-row tile)
    assert g(FAKE, 16, (1 << 22) + 64, FAKE, 8, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 62, None) == UNSUP
    assert g(FAKE, 16, 64, FAKE, 8, FAKE, FAKE, FAKE, (1 << 22) + 64, FAKE, FAKE, 1 << 62, None) == UNSUP
    assert b"at most" in lib.moe_last_error()
    # more tiles than a launch can index
    assert g(FAKE, (1 << 31) - 1, 64, FAKE, 8, FAKE, FAKE, FAKE, 1 << 22, FAKE, FAKE, 1 << 62, None) == UNSUP
    assert b"too many tiles" in lib.moe_last_error()


def test_row_copy_errors():
    s, g = lib.moe_scatter_rows, lib.moe_gather_rows
    assert s(FAKE, -1, 16, 2, FAKE, FAKE, None) == ARG
    assert s(FAKE, 4, 0, 2, FAKE, FAKE, None) == ARG
    assert s(FAKE, 4, 16, 0, FAKE, FAKE, None) == ARG
    assert s(None, 4, 16, 2, FAKE, FAKE, None) == ARG
    assert s(FAKE, 2**30, 16, 4, FAKE, FAKE, None) == UNSUP
    assert s(FAKE, 4, 16, 65, FAKE, FAKE, None) == UNSUP     # k above MOE_MAX_TOPK
    assert b"k > 64" in lib.moe_last_error()
    assert s(FAKE, 0, 16, 65, None, None, None) == UNSUP     # checked before the N == 0 no-op
    assert s(None, 0, 16, 2, None, None, None) == 0
    assert g(FAKE, 4, 16, 2, FAKE, -1, FAKE, None) == ARG
    assert g(FAKE, 4, 16, 2, None, 8, FAKE, None) == ARG
    assert g(None, 4, 16, 2, None, 0, None, None) == 0


def test_route_dispatch_errors():
    f = lib.moe_route_dispatch

    def call(**kw):
        a = dict(logits=FAKE, renorm=1, idx=FAKE, w=FAKE, x=FAKE, xs=None, dtype=1, n=4, d=64, e=8,
                 k=2, g=1, sort=1, cutoff=256, used=None, rows=FAKE, rs=None, counts=FAKE, offs=FAKE,
                 segs=FAKE, src=FAKE, dst=FAKE, rexp=FAKE, ws=FAKE, wsb=1 << 20)
        a.update(kw)
        return f(a["logits"], a["renorm"], a["idx"], a["w"], a["x"], a["xs"], a["dtype"], a["n"],
                 a["d"], a["e"], a["k"], a["g"], a["sort"], a["cutoff"], a["used"], a["rows"], a["rs"],
                 a["counts"], a["offs"], a["segs"], a["src"], a["dst"], a["rexp"], a["ws"], a["wsb"], None)

    assert call(logits=None) == ARG
    assert call(w=None) == ARG
    assert call(k=9) == ARG
    assert call(g=3) == ARG
    assert call(rows=None) == ARG
    assert call(ws=None) == WS
    assert call(wsb=8) == WS
    assert call(e=2048) == UNSUP
    g = lib.moe_route_dispatch_workspace_bytes
    assert g(4096, 256, 8, 1) >= lib.moe_dispatch_workspace_bytes(4096, 256, 8, 1)
    assert g(4, 8, 9, 1) == 0


def test_grouped_gemm_fp8_errors():
    g = lib.moe_grouped_gemm_fp8     # rows, row_scales, R, K, offsets, E, w, w_scales, N, y, stream
    assert g(FAKE, FAKE, -1, 128, FAKE, 4, FAKE, FAKE, 128, FAKE, None) == ARG
    assert g(FAKE, FAKE, 8, 0, FAKE, 4, FAKE, FAKE, 128, FAKE, None) == ARG
    assert g(FAKE, FAKE, 8, 128, FAKE, 0, FAKE, FAKE, 128, FAKE, None) == ARG
    assert g(FAKE, FAKE, 8, 100, FAKE, 4, FAKE, FAKE, 128, FAKE, None) == UNSUP      # K % 128
    assert g(FAKE, FAKE, 8, 128, FAKE, 4, FAKE, FAKE, 200, FAKE, None) == UNSUP      # N % 128
    assert g(FAKE, FAKE, 8, 128, FAKE, 2000, FAKE, FAKE, 128, FAKE, None) == UNSUP   # E
    assert g(None, FAKE, 8, 128, FAKE, 4, FAKE, FAKE, 128, FAKE, None) == ARG
    assert g(FAKE, FAKE, 8, 128, FAKE, 4, FAKE, None, 128, FAKE, None) == ARG
    assert g(None, None, 0, 128, None, 4, None, None, 128, None, None) == 0           # no rows
    odd = ctypes.c_void_p(0x1008)
    assert g(odd, FAKE, 8, 128, FAKE, 4, FAKE, FAKE, 128, FAKE, None) == UNSUP
    assert g(FAKE, FAKE, 8, 128, FAKE, 4, odd, FAKE, 128, FAKE, None) == UNSUP
    assert g(FAKE, FAKE, 8, 128, FAKE, 4, FAKE, FAKE, 128, odd, None) == UNSUP
    assert g(FAKE, ctypes.c_void_p(0x1002), 8, 128, FAKE, 4, FAKE, FAKE, 128, FAKE, None) == ARG
    assert b"aligned" in lib.moe_last_error()


def test_gather_swiglu_errors():
    g = lib.moe_gather_swiglu
    ws = lib.moe_gather_swiglu_workspace_bytes(1024, 256, 7168, 2048)
    assert ws >= 1024 * 2048 * 2                                      # h
    assert lib.moe_gather_swiglu_workspace_bytes(-1, 8, 128, 128) == 0
    assert lib.moe_gather_swiglu_workspace_bytes(8, 2000, 128, 128) == 0
    assert g(FAKE, -1, 128, FAKE, 4, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 20, None) == ARG
    assert g(FAKE, 8, 0, FAKE, 4, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 20, None) == ARG
    assert g(FAKE, 8, 128, FAKE, 0, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 20, None) == ARG
    assert g(FAKE, 8, 128, FAKE, 2000, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 20, None) == UNSUP
    assert g(FAKE, 8, 192, FAKE, 4, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 20, None) == UNSUP
    assert g(FAKE, 8, 128, FAKE, 4, FAKE, FAKE, FAKE, 64, FAKE, FAKE, 1 << 20, None) == UNSUP
    assert g(FAKE, 1 << 31, 128, FAKE, 4, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 20, None) == UNSUP
    assert g(None, 8, 128, FAKE, 4, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 20, None) == ARG
    assert g(FAKE, 8, 128, None, 4, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 20, None) == ARG
    odd = ctypes.c_void_p(0x1008)
    assert g(odd, 8, 128, FAKE, 4, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 1 << 20, None) == UNSUP
    assert g(FAKE, 8, 128, FAKE, 4, FAKE, odd, FAKE, 128, FAKE, FAKE, 1 << 20, None) == UNSUP
    assert g(FAKE, 8, 128, FAKE, 4, FAKE, FAKE, FAKE, 128, ctypes.c_void_p(0x1001), FAKE,
             1 << 20, None) == UNSUP
    need = lib.moe_gather_swiglu_workspace_bytes(8, 4, 128, 128)
    assert g(FAKE, 8, 128, FAKE, 4, FAKE, FAKE, FAKE, 128, FAKE, FAKE, need - 1, None) == WS
    assert g(FAKE, 8, 128, FAKE, 4, FAKE, FAKE, FAKE, 128, FAKE, None, need, None) == WS
    assert g(FAKE, 8, 128, FAKE, 4, FAKE, FAKE, FAKE, 128, FAKE, ctypes.c_void_p(0x1080), need,
             None) == WS
    assert g(None, 0, 128, None, 4, None, None, None, 128, None, None, 0, None) == 0   # empty


def test_gather_swiglu_combine_errors():
    g = lib.moe_gather_swiglu_combine
    need = lib.moe_gather_swiglu_workspace_bytes(16, 4, 128, 128)
    args = lambda **kw: [kw.get("rows", FAKE), kw.get("n_rows", 16), kw.get("d", 128), FAKE,
                         kw.get("row_pair", None), kw.get("tw", FAKE), kw.get("n", 8), kw.get("k", 2),
                         kw.get("e", 4), FAKE, FAKE, FAKE, kw.get("f", 128), kw.get("out", FAKE),
                         kw.get("ws", FAKE), kw.get("wsb", need), None]
    assert g(*args(n_rows=-1)) == ARG
    assert g(*args(n=-1)) == ARG
    assert g(*args(k=0)) == ARG and g(*args(k=65)) == ARG
    assert g(*args(e=2000)) == UNSUP
    assert g(*args(d=192)) == UNSUP and g(*args(f=64)) == UNSUP
    assert g(*args(n=1 << 30, k=4)) == UNSUP
    assert g(*args(tw=None)) == ARG and g(*args(out=None)) == ARG and g(*args(rows=None)) == ARG
    assert g(*args(out=ctypes.c_void_p(0x1002))) == UNSUP
    assert g(*args(rows=ctypes.c_void_p(0x1008))) == UNSUP
    assert g(*args(wsb=need - 1)) == WS and g(*args(ws=ctypes.c_void_p(0x1040))) == WS
    assert g(*args(n_rows=0, rows=None, tw=None, out=None, ws=None, wsb=0)) == 0


def test_route_dispatch_noalloc_errors_before_any_device_call():
    """The allocation-free variant checks every argument, and that its sizes
    fit the static scratch, before it looks the scratch up (no GPU here: a
    call that got that far would report MOE_ERR_HIP instead)."""
    f = lib.moe_route_dispatch_noalloc

    def call(**kw):
        a = dict(logits=FAKE, renorm=1, idx=FAKE, w=FAKE, x=FAKE, xs=None, dtype=1, n=4, d=64, e=8,
                 k=2, g=1, sort=1, cutoff=256, used=None, rows=FAKE, rs=None, counts=FAKE, offs=FAKE,
                 segs=FAKE, src=FAKE, dst=FAKE, rexp=FAKE)
        a.update(kw)
        return f(a["logits"], a["renorm"], a["idx"], a["w"], a["x"], a["xs"], a["dtype"], a["n"],
                 a["d"], a["e"], a["k"], a["g"], a["sort"], a["cutoff"], a["used"], a["rows"], a["rs"],
                 a["counts"], a["offs"], a["segs"], a["src"], a["dst"], a["rexp"], None)

    assert call(logits=None) == ARG
    assert call(k=9) == ARG
    assert call(g=3) == ARG
    assert call(rows=None) == ARG
    assert call(e=2048) == UNSUP
    # E = 1024 with 2^19 pairs needs 512 chunk histograms of 4 KB: more than the array
    need = lib.moe_route_dispatch_workspace_bytes(1 << 16, 1024, 8, 1)
    assert need > _lib.MOE_NOALLOC_SCRATCH_BYTES
    assert call(n=1 << 16, e=1024, k=8) == UNSUP
    assert b"static array" in lib.moe_last_error()
    # the binding's constant is the header's
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) \+ (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) + int(m.group(2)) == _lib.MOE_NOALLOC_SCRATCH_BYTES
    # the largest sizes at E <= 256 fit
    for n, e, k in ((1 << 18, 256, 8), (4096, 256, 8), (32768, 1024, 8), (1 << 20, 64, 2)):
        assert lib.moe_route_dispatch_workspace_bytes(n, e, k, 1) <= _lib.MOE_NOALLOC_SCRATCH_BYTES
