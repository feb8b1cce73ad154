"""C ABI checks that need no GPU: libprism.so loads, exports every function include/prism.h
declares, sizes workspaces, and rejects invalid arguments before any device work."""
import ctypes
import os
import re

import pytest

from token_level_sparse_prism_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prism.h")


def _ensure_built():
    if not os.path.exists(B.LIB_PATH):
        from token_level_sparse_prism_amd import build
        build.build()


@pytest.fixture(scope="module")
def lib():
    _ensure_built()
    return B.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(prism_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("prism_propose", "prism_refine_attend", "prism_dense_ref", "prism_quantize_keys",
                 "prism_quantize_keys_int2", "prism_propose_int2", "prism_propose_paged", "prism_refine_attend_paged",
                 "prism_workspace_bytes", "prism_workspace_init"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert set(B.EXPORTS) == set(header_functions())


def shape(B_=1, Hq=32, Hkv=8, D=128, T=131072):
    return B.Shape(B_, Hq, Hkv, D, T, None)


def test_workspace_bytes(lib):
    s = shape()
    p = B.workspace_bytes(B.OP_PROPOSE, s, 8192, 0)
    r = B.workspace_bytes(B.OP_REFINE, s, 8192, 2048)
    d = B.workspace_bytes(B.OP_DENSE, s)
    # propose holds per token a 4-byte key and an 8-byte candidate slot
    assert p >= 8 * 131072 * 12
    # refine holds per pool slot a key and G padded logits
    assert r >= 8 * 8192 * (4 + 16)
    assert d > 0
    assert B.workspace_bytes(B.OP_REFINE, s, 1024, 2048) == 0       # kappa > kp
    assert B.workspace_bytes(B.OP_PROPOSE, shape(D=96), 64, 0) == 0  # unsupported D
    assert B.workspace_bytes(B.OP_PROPOSE, shape(Hq=30), 64, 0) == 0  # Hq % Hkv != 0
    assert B.workspace_bytes(7, s, 64, 16) == 0


def _call_propose(lib, s, kp=64, agg=0, q=256, kq=256, sc=256, pool=256, ws=256, wsb=1 << 40):
    return lib.prism_propose(ctypes.c_void_p(q), 1, ctypes.c_void_p(kq), ctypes.c_void_p(sc), ctypes.byref(s),
                             kp, agg, ctypes.c_void_p(pool), None, ctypes.c_void_p(ws), wsb, None)


def test_invalid_arguments_return_before_device_work(lib):
    s = shape(T=4096)
    # fake (never dereferenced) addresses: validation must fail before any launch
    assert _call_propose(lib, s, kp=0) == 1
    assert _call_propose(lib, s, agg=5) == 1
    assert _call_propose(lib, s, q=0) == 1
    assert _call_propose(lib, s, q=258) == 1                      # misaligned q
    assert _call_propose(lib, s, ws=512 + 16) == 1                # misaligned workspace
    assert _call_propose(lib, s, wsb=16) == 3                     # workspace too small
    assert _call_propose(lib, shape(D=100, T=4096)) == 2
    assert _call_propose(lib, shape(Hq=17 * 8, Hkv=8, T=4096)) == 2   # G > 16
    assert _call_propose(lib, shape(T=(1 << 23) + 1)) == 2
    assert _call_propose(lib, shape(Hq=12, Hkv=8, T=4096)) == 1
    f = ctypes.c_void_p
    r = lib.prism_refine_attend(f(256), f(256), f(256), 1, ctypes.byref(s), f(256), 64, 65, 0, 0.0, f(256),
                                f(256), None, f(256), 1 << 40, None)
    assert r == 1                                                 # kappa > kp
    r = lib.prism_refine_attend(f(256), f(256), f(256), 1, ctypes.byref(s), f(256), 64, 16, 0, -1.0, f(256),
                                f(256), None, f(256), 1 << 40, None)
    assert r == 1                                                 # negative scale
    r = lib.prism_refine_attend(f(256), f(256), f(256), 3, ctypes.byref(s), f(256), 64, 16, 0, 0.0, f(256),
                                f(256), None, f(256), 1 << 40, None)
    assert r == 1                                                 # bad dtype
    r = lib.prism_dense_ref(f(256), f(256), f(256), 1, ctypes.byref(s), 0.0, f(256), None, f(256), 16, None)
    assert r == 3
    assert lib.prism_quantize_keys(None, 1, ctypes.byref(s), f(256), f(256), None) == 1
    # INT2 proposal: same validation as the int8 one
    def p2(kp=64, kq=256, s_=s):
        return lib.prism_propose_int2(f(256), 1, f(kq), f(256), ctypes.byref(s_), kp, 0, f(256), None, f(256),
                                      1 << 40, None)
    assert p2(kp=0) == 1
    assert p2(kq=0) == 1
    assert p2(kq=256 + 4) == 1                                    # misaligned codes
    assert p2(s_=shape(D=96, T=4096)) == 2
    assert lib.prism_quantize_keys_int2(None, 1, ctypes.byref(s), f(256), f(256), None) == 1
    assert lib.prism_quantize_keys_int2(f(256), 1, ctypes.byref(s), f(256 + 8), f(256), None) == 1
    assert lib.prism_quantize_keys_int2(f(256), 1, ctypes.byref(shape(D=32, T=64)), f(256), f(256), None) == 2
    # paged calls: the page descriptor is checked before any launch
    def pp(pg, kb=8):
        return lib.prism_propose_paged(f(256), 1, f(256), kb, f(256), ctypes.byref(s), ctypes.byref(pg) if pg else None,
                                       64, 0, f(256), None, f(256), 1 << 40, None)
    good = B.Paging(256, 64, 64, 64 * 64)      # 64 pages of 64 tokens cover T_max = 4096
    assert pp(None) == 1
    assert pp(B.Paging(0, 64, 64, 4096)) == 1          # no table
    assert pp(B.Paging(256, 64, 48, 4096)) == 1        # page size not a power of two
    assert pp(B.Paging(256, 32, 64, 4096)) == 1        # table covers 2048 < T_max tokens
    assert pp(B.Paging(256, 64, 64, 4000)) == 1        # pool not a whole number of pages
    assert pp(B.Paging(258, 64, 64, 4096)) == 1        # misaligned table
    assert pp(good, kb=4) == 1                         # key bits
    r = lib.prism_refine_attend_paged(f(256), f(256), f(256), 1, ctypes.byref(s), ctypes.byref(B.Paging(256, 64, 0, 4096)),
                                      f(256), 64, 16, 0, 0.0, f(256), f(256), None, f(256), 1 << 40, None)
    assert r == 1                                      # page size 0
    assert lib.prism_workspace_init(f(128), 1024, None) == 1
    assert lib.prism_status_str(3) == b"PRISM_ERR_WORKSPACE"
