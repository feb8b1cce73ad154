"""ctypes binding of the plain C oracle (oracle/prism_oracle.c).

TEST INFRASTRUCTURE ONLY.  Arrays are numpy, on the host.  Floating inputs
are passed as float32 (bf16 values widen to float32 exactly); the oracle's
floating outputs are float64.  Builds the library with gcc if it is absent.
"""
import ctypes
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libprism_oracle.so")

AGG_SUM = 0
AGG_MAX = 1

_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i8p = ctypes.POINTER(ctypes.c_int8)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.orc_quantize_rows.argtypes = [_f32p, _i64, _int, _i8p, _f32p]
    lib.orc_quantize_rows_int2.argtypes = [_f32p, _i64, _int, _i8p, _f32p]
    lib.orc_quantize_query.argtypes = [_f32p, _int, _int, _i8p, _f32p]
    lib.orc_propose_unit.argtypes = [_f32p, _int, _int, _i8p, _f32p, _i64, _i64, _int, _i32p, _f32p]
    lib.orc_refine_unit.argtypes = [_f32p, _int, _int, _f32p, _f32p, _i64, _i32p, _i64, _i64,
                                    _int, ctypes.c_double, _i32p, _f64p, _f64p, _f64p, _f64p]
    lib.orc_attend_unit.argtypes = [_f32p, _int, _int, _f32p, _f32p, _i64, _i32p, _i64,
                                    ctypes.c_double, _f64p, _f64p]
    lib.orc_dense_unit.argtypes = [_f32p, _int, _int, _f32p, _f32p, _i64, ctypes.c_double,
                                   _f64p, _f64p]
    lib.orc_propose.argtypes = [_f32p, _int, _int, _int, _int, _i8p, _f32p, _i64, _i32p, _i64,
                                _int, _i32p, _f32p, _int]
    lib.orc_refine.argtypes = [_f32p, _int, _int, _int, _int, _f32p, _f32p, _i64, _i32p, _i32p,
                               _i64, _i64, _int, ctypes.c_double, _i32p, _f64p, _f64p, _int]
    lib.orc_dense.argtypes = [_f32p, _int, _int, _int, _int, _f32p, _f32p, _i64, _i32p,
                              ctypes.c_double, _f64p, _f64p, _int]
    for name in ("orc_quantize_rows", "orc_quantize_rows_int2", "orc_quantize_query", "orc_propose_unit", "orc_refine_unit",
                 "orc_attend_unit", "orc_dense_unit", "orc_propose", "orc_refine", "orc_dense",
                 "orc_max_threads"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def max_threads():
    return load().orc_max_threads()


def quantize_rows(K):
    """O1: per-row int8 absmax quantization. K [..., D] -> (Kq int8 [..., D], scales f32 [...])."""
    K = _f32(K)
    D = K.shape[-1]
    n = K.size // D if D else 0
    Kq = np.empty(K.shape, dtype=np.int8)
    s = np.empty(K.shape[:-1], dtype=np.float32)
    _check(load().orc_quantize_rows(_p(K, ctypes.c_float), n, D, _p(Kq, ctypes.c_int8),
                                    _p(s, ctypes.c_float)), "quantize_rows")
    return Kq, s


def quantize_rows_int2(K):
    """O1' (INT2 keys): per-row 2-bit codes. K [..., D] -> (levels int8 [..., D] in {-3,-1,1,3},
    scales f32 [...]); K is reconstructed as scales[..., None] * levels.  Scoring these levels
    with propose() is the INT2 proposal."""
    K = _f32(K)
    D = K.shape[-1]
    n = K.size // D if D else 0
    lv = np.empty(K.shape, dtype=np.int8)
    s = np.empty(K.shape[:-1], dtype=np.float32)
    _check(load().orc_quantize_rows_int2(_p(K, ctypes.c_float), n, D, _p(lv, ctypes.c_int8),
                                         _p(s, ctypes.c_float)), "quantize_rows_int2")
    return lv, s


def quantize_query(q_group):
    """O2: q_group [G, D] -> (qi int8 [G, D], scale f32)."""
    q = _f32(q_group)
    G, D = q.shape
    qi = np.empty((G, D), dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    _check(load().orc_quantize_query(_p(q, ctypes.c_float), G, D, _p(qi, ctypes.c_int8),
                                     _p(s, ctypes.c_float)), "quantize_query")
    return qi, float(s[0])


def propose_unit(q_group, Kq_rows, scales_rows, T_b, kp, agg=AGG_SUM):
    """O3-O4 for one unit. Returns (pool int32 [kp], scores f32 [T_b])."""
    q = _f32(q_group)
    G, D = q.shape
    Kq = np.ascontiguousarray(Kq_rows, dtype=np.int8)
    sc = _f32(scales_rows)
    assert Kq.shape[0] >= T_b and sc.shape[0] >= T_b
    pool = np.empty(kp, dtype=np.int32)
    scores = np.empty(max(T_b, 1), dtype=np.float32)
    _check(load().orc_propose_unit(_p(q, ctypes.c_float), G, D, _p(Kq, ctypes.c_int8),
                                   _p(sc, ctypes.c_float), T_b, kp, agg,
                                   _p(pool, ctypes.c_int32), _p(scores, ctypes.c_float)),
           "propose_unit")
    return pool, scores[:T_b]


def refine_unit(q_group, K_rows, V_rows, T_b, pool, kappa, agg=AGG_SUM, sm_scale=None):
    """O5-O7 for one unit. Returns dict(idx, out [G,D] f64, lse [G] f64, S [kp] f64, logits [kp,G])."""
    q = _f32(q_group)
    G, D = q.shape
    K = _f32(K_rows)
    V = _f32(V_rows)
    pool = np.ascontiguousarray(pool, dtype=np.int32)
    kp = pool.shape[0]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    idx = np.empty(kappa, dtype=np.int32)
    out = np.empty((G, D), dtype=np.float64)
    lse = np.empty(G, dtype=np.float64)
    S = np.empty(kp, dtype=np.float64)
    lg = np.empty((kp, G), dtype=np.float64)
    _check(load().orc_refine_unit(_p(q, ctypes.c_float), G, D, _p(K, ctypes.c_float),
                                  _p(V, ctypes.c_float), T_b, _p(pool, ctypes.c_int32), kp, kappa,
                                  agg, sm_scale, _p(idx, ctypes.c_int32), _p(out, ctypes.c_double),
                                  _p(lse, ctypes.c_double), _p(S, ctypes.c_double),
                                  _p(lg, ctypes.c_double)), "refine_unit")
    return {"idx": idx, "out": out, "lse": lse, "S": S, "logits": lg}


def attend_unit(q_group, K_rows, V_rows, T_b, token_list, sm_scale=None):
    """O7 over a given token list. Returns (out [G,D] f64, lse [G] f64)."""
    q = _f32(q_group)
    G, D = q.shape
    K = _f32(K_rows)
    V = _f32(V_rows)
    lst = np.ascontiguousarray(token_list, dtype=np.int32)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out = np.empty((G, D), dtype=np.float64)
    lse = np.empty(G, dtype=np.float64)
    _check(load().orc_attend_unit(_p(q, ctypes.c_float), G, D, _p(K, ctypes.c_float),
                                  _p(V, ctypes.c_float), T_b, _p(lst, ctypes.c_int32), lst.shape[0],
                                  sm_scale, _p(out, ctypes.c_double), _p(lse, ctypes.c_double)),
           "attend_unit")
    return out, lse


def dense_unit(q_group, K_rows, V_rows, T_b, sm_scale=None):
    """O8 for one unit. Returns (out [G,D] f64, lse [G] f64)."""
    q = _f32(q_group)
    G, D = q.shape
    K = _f32(K_rows)
    V = _f32(V_rows)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out = np.empty((G, D), dtype=np.float64)
    lse = np.empty(G, dtype=np.float64)
    _check(load().orc_dense_unit(_p(q, ctypes.c_float), G, D, _p(K, ctypes.c_float),
                                 _p(V, ctypes.c_float), T_b, sm_scale, _p(out, ctypes.c_double),
                                 _p(lse, ctypes.c_double)), "dense_unit")
    return out, lse


def _lens(seq_lens, B):
    if seq_lens is None:
        return None
    a = np.ascontiguousarray(seq_lens, dtype=np.int32)
    assert a.shape == (B,)
    return a


def propose(q, Kq, scales, kp, seq_lens=None, agg=AGG_SUM, nthreads=0, want_scores=False):
    """Batched O3-O4. q [B,Hq,D]; Kq [B,Hkv,T_max,D]; scales [B,Hkv,T_max].
    Returns pool [B,Hkv,kp] (and scores [B,Hkv,T_max] if asked; entries t >= T_b unspecified)."""
    q = _f32(q)
    B, Hq, D = q.shape
    Kq = np.ascontiguousarray(Kq, dtype=np.int8)
    _, Hkv, T_max, _ = Kq.shape
    sc = _f32(scales)
    lens = _lens(seq_lens, B)
    pool = np.empty((B, Hkv, kp), dtype=np.int32)
    scores = np.zeros((B, Hkv, T_max), dtype=np.float32) if want_scores else None
    _check(load().orc_propose(_p(q, ctypes.c_float), B, Hq, Hkv, D, _p(Kq, ctypes.c_int8),
                              _p(sc, ctypes.c_float), T_max, _p(lens, ctypes.c_int32), kp, agg,
                              _p(pool, ctypes.c_int32), _p(scores, ctypes.c_float), nthreads),
           "propose")
    return (pool, scores) if want_scores else pool


def refine(q, K, V, pool, kappa, seq_lens=None, agg=AGG_SUM, sm_scale=None, nthreads=0):
    """Batched O5-O7. Returns (idx [B,Hkv,kappa], out [B,Hq,D] f64, lse [B,Hq] f64)."""
    q = _f32(q)
    B, Hq, D = q.shape
    K = _f32(K)
    V = _f32(V)
    _, Hkv, T_max, _ = K.shape
    pool = np.ascontiguousarray(pool, dtype=np.int32)
    kp = pool.shape[-1]
    lens = _lens(seq_lens, B)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    idx = np.empty((B, Hkv, kappa), dtype=np.int32)
    out = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    _check(load().orc_refine(_p(q, ctypes.c_float), B, Hq, Hkv, D, _p(K, ctypes.c_float),
                             _p(V, ctypes.c_float), T_max, _p(lens, ctypes.c_int32),
                             _p(pool, ctypes.c_int32), kp, kappa, agg, sm_scale,
                             _p(idx, ctypes.c_int32), _p(out, ctypes.c_double),
                             _p(lse, ctypes.c_double), nthreads), "refine")
    return idx, out, lse


def dense(q, K, V, seq_lens=None, sm_scale=None, nthreads=0):
    """Batched O8. Returns (out [B,Hq,D] f64, lse [B,Hq] f64)."""
    q = _f32(q)
    B, Hq, D = q.shape
    K = _f32(K)
    V = _f32(V)
    _, Hkv, T_max, _ = K.shape
    lens = _lens(seq_lens, B)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    _check(load().orc_dense(_p(q, ctypes.c_float), B, Hq, Hkv, D, _p(K, ctypes.c_float),
                            _p(V, ctypes.c_float), T_max, _p(lens, ctypes.c_int32), sm_scale,
                            _p(out, ctypes.c_double), _p(lse, ctypes.c_double), nthreads), "dense")
    return out, lse
