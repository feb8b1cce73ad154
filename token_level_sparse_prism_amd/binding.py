"""ctypes binding of libprism.so (C ABI in include/prism.h).

Argument marshalling only: torch tensors supply device memory and the current HIP stream; every
step of the computation runs in the library's kernels.  There is no fallback: if the library is
missing or a call fails, this raises.
"""
import ctypes
import os
from typing import Optional, Tuple

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libprism.so")

PRISM_F32, PRISM_BF16 = 0, 1
AGG_SUM, AGG_MAX = 0, 1
OP_PROPOSE, OP_REFINE, OP_DENSE = 0, 1, 2
STATUS = {0: "PRISM_OK", 1: "PRISM_ERR_INVALID_ARG", 2: "PRISM_ERR_UNSUPPORTED",
          3: "PRISM_ERR_WORKSPACE", 4: "PRISM_ERR_HIP"}
EXPORTS = ("prism_workspace_bytes", "prism_workspace_init", "prism_quantize_keys", "prism_propose",
           "prism_quantize_keys_int2", "prism_propose_int2", "prism_propose_paged", "prism_refine_attend_paged",
           "prism_refine_attend", "prism_dense_ref", "prism_profile_enable", "prism_profile_query",
           "prism_profile_reset", "prism_last_hip_error", "prism_status_str", "prism_read_probe",
           "prism_refine_attend_static", "prism_timeline_read", "prism_timeline_clear")
KERNELS = ("k_quantize_keys", "k_quantize_keys_int2", "k_scan", "k_cand", "k_compact", "k_rscore", "k_attend", "k_dense",
           "k_read_probe")


class PrismError(RuntimeError):
    def __init__(self, fn: str, code: int, hip: int = 0):
        super().__init__(f"{fn} -> {STATUS.get(code, code)}" + (f" (hipError {hip})" if hip else ""))
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("D", ctypes.c_int32), ("T_max", ctypes.c_int64), ("seq_lens", ctypes.c_void_p)]


class Paging(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_slots", ctypes.c_int64)]


_lib = None
_vp = ctypes.c_void_p


def load(path: Optional[str] = None):
    """Load libprism.so (built by token_level_sparse_prism_amd/build.py), or the library at `path`
    (the timeline build lib/libprism_tl.so for bench.py --timeline); raise if it is absent.  The
    first load fixes the library for the process."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run token_level_sparse_prism_amd/build.py")
    lib = ctypes.CDLL(path)
    sp = ctypes.POINTER(Shape)
    lib.prism_workspace_bytes.argtypes = [ctypes.c_int, sp, ctypes.c_int32, ctypes.c_int32]
    lib.prism_workspace_bytes.restype = ctypes.c_size_t
    lib.prism_workspace_init.argtypes = [_vp, ctypes.c_size_t, _vp]
    lib.prism_quantize_keys.argtypes = [_vp, ctypes.c_int, sp, _vp, _vp, _vp]
    lib.prism_propose.argtypes = [_vp, ctypes.c_int, _vp, _vp, sp, ctypes.c_int32, ctypes.c_int, _vp, _vp,
                                  _vp, ctypes.c_size_t, _vp]
    lib.prism_quantize_keys_int2.argtypes = [_vp, ctypes.c_int, sp, _vp, _vp, _vp]
    lib.prism_propose_int2.argtypes = [_vp, ctypes.c_int, _vp, _vp, sp, ctypes.c_int32, ctypes.c_int, _vp, _vp,
                                       _vp, ctypes.c_size_t, _vp]
    pgp = ctypes.POINTER(Paging)
    lib.prism_propose_paged.argtypes = [_vp, ctypes.c_int, _vp, ctypes.c_int32, _vp, sp, pgp, ctypes.c_int32,
                                        ctypes.c_int, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.prism_refine_attend_paged.argtypes = [_vp, _vp, _vp, ctypes.c_int, sp, pgp, _vp, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int, ctypes.c_float, _vp, _vp, _vp, _vp,
                                              ctypes.c_size_t, _vp]
    lib.prism_refine_attend.argtypes = [_vp, _vp, _vp, ctypes.c_int, sp, _vp, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int, ctypes.c_float, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.prism_refine_attend_static.argtypes = [_vp, _vp, _vp, ctypes.c_int, sp, _vp, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int, ctypes.c_float, _vp, _vp, _vp, _vp]
    lib.prism_timeline_read.argtypes = [ctypes.c_int, _vp, ctypes.c_int64]
    lib.prism_timeline_read.restype = ctypes.c_int
    lib.prism_timeline_clear.argtypes = []
    lib.prism_timeline_clear.restype = ctypes.c_int
    lib.prism_dense_ref.argtypes = [_vp, _vp, _vp, ctypes.c_int, sp, ctypes.c_float, _vp, _vp, _vp,
                                    ctypes.c_size_t, _vp]
    for fn in ("prism_workspace_init", "prism_quantize_keys", "prism_propose", "prism_quantize_keys_int2",
               "prism_propose_int2", "prism_propose_paged", "prism_refine_attend_paged", "prism_refine_attend",
               "prism_dense_ref", "prism_last_hip_error", "prism_refine_attend_static"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.prism_profile_enable.argtypes = [ctypes.c_int]
    lib.prism_profile_enable.restype = ctypes.c_int
    lib.prism_profile_query.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)]
    lib.prism_profile_query.restype = ctypes.c_int
    lib.prism_profile_reset.argtypes = []
    lib.prism_profile_reset.restype = None
    lib.prism_read_probe.argtypes = [_vp, ctypes.c_size_t, _vp, _vp]
    lib.prism_read_probe.restype = ctypes.c_int
    lib.prism_status_str.argtypes = [ctypes.c_int]
    lib.prism_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise PrismError(fn, rc, load().prism_last_hip_error() if rc == 4 else 0)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PRISM_F32
    if t.dtype == torch.bfloat16:
        return PRISM_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t: torch.Tensor, name: str):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")


def make_shape(q: torch.Tensor, K: torch.Tensor, seq_lens: Optional[torch.Tensor] = None,
               k_cols_per_dim: int = 1) -> Shape:
    """k_cols_per_dim: K's last dimension per head-dim element (1, or 1/4 for packed 2-bit keys
    given as 4)."""
    B, Hq, D = q.shape
    B2, Hkv, T_max, D2 = K.shape
    if B != B2 or D != D2 * k_cols_per_dim:
        raise ValueError("q [B,Hq,D] and K [B,Hkv,T_max,D] disagree")
    if seq_lens is not None:
        _need(seq_lens, "seq_lens")
        if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
            raise ValueError("seq_lens must be int32 [B]")
    return Shape(B, Hq, Hkv, D, T_max, None if seq_lens is None else seq_lens.data_ptr())


def workspace_bytes(op: int, shape: Shape, kp: int = 0, kappa: int = 0) -> int:
    return int(load().prism_workspace_bytes(op, ctypes.byref(shape), kp, kappa))


def new_workspace(op: int, shape: Shape, kp: int = 0, kappa: int = 0, device=None, stream=None) -> torch.Tensor:
    """Allocate (through torch) and zero-fill (with the library's kernel) a workspace."""
    n = workspace_bytes(op, shape, kp, kappa)
    if n == 0:
        raise PrismError("prism_workspace_bytes", 1)
    return new_workspace_bytes(n, device=device, stream=stream)


def new_workspace_bytes(n: int, device=None, stream=None) -> torch.Tensor:
    """A zero-filled, 256-byte aligned workspace of n bytes (e.g. the larger of two ops' sizes,
    for a workspace that the two share)."""
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device or "cuda")
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    _check("prism_workspace_init", load().prism_workspace_init(_ptr(ws), n, _stream(stream)))
    return ws


def quantize_keys(K: torch.Tensor, seq_lens: Optional[torch.Tensor] = None, Kq: Optional[torch.Tensor] = None,
                  scales: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    _need(K, "K")
    B, Hkv, T_max, D = K.shape
    q_dummy = torch.empty((B, Hkv, D), device=K.device, dtype=K.dtype)
    shape = make_shape(q_dummy, K, seq_lens)
    if Kq is None:
        Kq = torch.zeros((B, Hkv, T_max, D), dtype=torch.int8, device=K.device)
    if scales is None:
        scales = torch.zeros((B, Hkv, T_max), dtype=torch.float32, device=K.device)
    _check("prism_quantize_keys", load().prism_quantize_keys(_ptr(K), _dtype_code(K), ctypes.byref(shape),
                                                             _ptr(Kq), _ptr(scales), _stream(stream)))
    return Kq, scales


def propose(q: torch.Tensor, Kq: torch.Tensor, scales: torch.Tensor, kp: int, agg: int = AGG_SUM,
            seq_lens: Optional[torch.Tensor] = None, pool: Optional[torch.Tensor] = None,
            scores: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """Proposal layer: returns pool [B,Hkv,kp] int32 (and fills `scores` if given)."""
    for t, n in ((q, "q"), (Kq, "Kq"), (scales, "scales")):
        _need(t, n)
    shape = make_shape(q, Kq, seq_lens)
    if pool is None:
        pool = torch.empty((shape.B, shape.Hkv, kp), dtype=torch.int32, device=q.device)
    if ws is None:
        ws = new_workspace(OP_PROPOSE, shape, kp, 0, device=q.device, stream=stream)
    _check("prism_propose", load().prism_propose(_ptr(q), _dtype_code(q), _ptr(Kq), _ptr(scales),
                                                 ctypes.byref(shape), kp, agg, _ptr(pool), _ptr(scores),
                                                 _ptr(ws), ws.numel(), _stream(stream)))
    return pool


def quantize_keys_int2(K: torch.Tensor, seq_lens: Optional[torch.Tensor] = None, Kq2: Optional[torch.Tensor] = None,
                       scales: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """INT2 key cache: returns (Kq2 [B,Hkv,T_max,D/4] uint8, four 2-bit codes per byte; scales)."""
    _need(K, "K")
    B, Hkv, T_max, D = K.shape
    q_dummy = torch.empty((B, Hkv, D), device=K.device, dtype=K.dtype)
    shape = make_shape(q_dummy, K, seq_lens)
    if Kq2 is None:
        Kq2 = torch.zeros((B, Hkv, T_max, D // 4), dtype=torch.uint8, device=K.device)
    if scales is None:
        scales = torch.zeros((B, Hkv, T_max), dtype=torch.float32, device=K.device)
    _check("prism_quantize_keys_int2", load().prism_quantize_keys_int2(_ptr(K), _dtype_code(K), ctypes.byref(shape),
                                                                       _ptr(Kq2), _ptr(scales), _stream(stream)))
    return Kq2, scales


def propose_int2(q: torch.Tensor, Kq2: torch.Tensor, scales: torch.Tensor, kp: int, agg: int = AGG_SUM,
                 seq_lens: Optional[torch.Tensor] = None, pool: Optional[torch.Tensor] = None,
                 scores: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """Proposal layer over the INT2 key cache: returns pool [B,Hkv,kp] int32."""
    for t, n in ((q, "q"), (Kq2, "Kq2"), (scales, "scales")):
        _need(t, n)
    shape = make_shape(q, Kq2, seq_lens, k_cols_per_dim=4)
    if pool is None:
        pool = torch.empty((shape.B, shape.Hkv, kp), dtype=torch.int32, device=q.device)
    if ws is None:
        ws = new_workspace(OP_PROPOSE, shape, kp, 0, device=q.device, stream=stream)
    _check("prism_propose_int2", load().prism_propose_int2(_ptr(q), _dtype_code(q), _ptr(Kq2), _ptr(scales),
                                                           ctypes.byref(shape), kp, agg, _ptr(pool), _ptr(scores),
                                                           _ptr(ws), ws.numel(), _stream(stream)))
    return pool


def refine_attend(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, pool: torch.Tensor, kappa: int,
                  agg: int = AGG_SUM, sm_scale: float = 0.0, seq_lens: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, want_lse: bool = True, ws: Optional[torch.Tensor] = None,
                  stream=None):
    """Refined layer: returns (out [B,Hq,D], idx [B,Hkv,kappa], lse [B,Hq] or None)."""
    for t, n in ((q, "q"), (K, "K"), (V, "V"), (pool, "pool")):
        _need(t, n)
    if not (q.dtype == K.dtype == V.dtype):
        raise TypeError("q, K and V must share one dtype")
    shape = make_shape(q, K, seq_lens)
    kp = pool.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    if idx is None:
        idx = torch.empty((shape.B, shape.Hkv, kappa), dtype=torch.int32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((shape.B, shape.Hq), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = new_workspace(OP_REFINE, shape, kp, kappa, device=q.device, stream=stream)
    _check("prism_refine_attend", load().prism_refine_attend(
        _ptr(q), _ptr(K), _ptr(V), _dtype_code(q), ctypes.byref(shape), _ptr(pool), kp, kappa, agg,
        float(sm_scale), _ptr(out), _ptr(idx), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return out, idx, lse


def refine_attend_static(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, pool: torch.Tensor, kappa: int,
                         agg: int = AGG_SUM, sm_scale: float = 0.0, seq_lens: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None, want_lse: bool = True, stream=None):
    """Refined layer through the allocation-free entry point (the library's static scratch, no
    workspace).  Pass out / idx / lse to keep this call free of allocations on the torch side too."""
    for t, n in ((q, "q"), (K, "K"), (V, "V"), (pool, "pool")):
        _need(t, n)
    if not (q.dtype == K.dtype == V.dtype):
        raise TypeError("q, K and V must share one dtype")
    shape = make_shape(q, K, seq_lens)
    kp = pool.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    if idx is None:
        idx = torch.empty((shape.B, shape.Hkv, kappa), dtype=torch.int32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((shape.B, shape.Hq), dtype=torch.float32, device=q.device)
    _check("prism_refine_attend_static", load().prism_refine_attend_static(
        _ptr(q), _ptr(K), _ptr(V), _dtype_code(q), ctypes.byref(shape), _ptr(pool), kp, kappa, agg,
        float(sm_scale), _ptr(out), _ptr(idx), _ptr(lse), _stream(stream)))
    return out, idx, lse


def _paged_shape(q: torch.Tensor, pool_rows: torch.Tensor, page_table: torch.Tensor, page_size: int,
                 T_max: Optional[int], seq_lens: Optional[torch.Tensor]) -> Tuple[Shape, Paging]:
    """Shape and page descriptor of a paged call: pools are [Hkv][num_slots][...]; T_max defaults to
    the table's capacity max_pages * page_size."""
    _need(page_table, "page_table")
    if page_table.dtype != torch.int32 or page_table.dim() != 2:
        raise ValueError("page_table must be int32 [B, max_pages]")
    B, Hq, D = q.shape
    Hkv, num_slots = pool_rows.shape[0], pool_rows.shape[1]
    if page_table.shape[0] != B:
        raise ValueError("page_table must have one row per sequence")
    T = int(T_max) if T_max is not None else page_table.shape[1] * page_size
    if seq_lens is not None:
        _need(seq_lens, "seq_lens")
        if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
            raise ValueError("seq_lens must be int32 [B]")
    shape = Shape(B, Hq, Hkv, D, T, None if seq_lens is None else seq_lens.data_ptr())
    return shape, Paging(page_table.data_ptr(), page_table.shape[1], int(page_size), int(num_slots))


def propose_paged(q: torch.Tensor, Kq_pool: torch.Tensor, scales_pool: torch.Tensor, page_table: torch.Tensor,
                  page_size: int, kp: int, agg: int = AGG_SUM, key_bits: int = 8, T_max: Optional[int] = None,
                  seq_lens: Optional[torch.Tensor] = None, pool: Optional[torch.Tensor] = None,
                  scores: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """Proposal layer over paged key pools (Kq_pool [Hkv, num_slots, D] int8, or [Hkv, num_slots, D/4]
    uint8 with key_bits=2; scales_pool [Hkv, num_slots]): returns pool [B,Hkv,kp] int32."""
    for t, n in ((q, "q"), (Kq_pool, "Kq_pool"), (scales_pool, "scales_pool")):
        _need(t, n)
    shape, pg = _paged_shape(q, Kq_pool, page_table, page_size, T_max, seq_lens)
    if pool is None:
        pool = torch.empty((shape.B, shape.Hkv, kp), dtype=torch.int32, device=q.device)
    if ws is None:
        ws = new_workspace(OP_PROPOSE, shape, kp, 0, device=q.device, stream=stream)
    _check("prism_propose_paged", load().prism_propose_paged(
        _ptr(q), _dtype_code(q), _ptr(Kq_pool), int(key_bits), _ptr(scales_pool), ctypes.byref(shape),
        ctypes.byref(pg), kp, agg, _ptr(pool), _ptr(scores), _ptr(ws), ws.numel(), _stream(stream)))
    return pool


def refine_attend_paged(q: torch.Tensor, K_pool: torch.Tensor, V_pool: torch.Tensor, page_table: torch.Tensor,
                        page_size: int, pool: torch.Tensor, kappa: int, agg: int = AGG_SUM, sm_scale: float = 0.0,
                        T_max: Optional[int] = None, seq_lens: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                        ws: Optional[torch.Tensor] = None, stream=None):
    """Refined layer over paged K / V pools [Hkv, num_slots, D]: returns (out, idx, lse)."""
    for t, n in ((q, "q"), (K_pool, "K_pool"), (V_pool, "V_pool"), (pool, "pool")):
        _need(t, n)
    if not (q.dtype == K_pool.dtype == V_pool.dtype):
        raise TypeError("q, K and V must share one dtype")
    shape, pg = _paged_shape(q, K_pool, page_table, page_size, T_max, seq_lens)
    kp = pool.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    if idx is None:
        idx = torch.empty((shape.B, shape.Hkv, kappa), dtype=torch.int32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((shape.B, shape.Hq), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = new_workspace(OP_REFINE, shape, kp, kappa, device=q.device, stream=stream)
    _check("prism_refine_attend_paged", load().prism_refine_attend_paged(
        _ptr(q), _ptr(K_pool), _ptr(V_pool), _dtype_code(q), ctypes.byref(shape), ctypes.byref(pg), _ptr(pool),
        kp, kappa, agg, float(sm_scale), _ptr(out), _ptr(idx), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return out, idx, lse


def dense_ref(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, sm_scale: float = 0.0,
              seq_lens: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """Dense decode attention: returns (out [B,Hq,D], lse [B,Hq])."""
    for t, n in ((q, "q"), (K, "K"), (V, "V")):
        _need(t, n)
    shape = make_shape(q, K, seq_lens)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((shape.B, shape.Hq), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = new_workspace(OP_DENSE, shape, device=q.device, stream=stream)
    _check("prism_dense_ref", load().prism_dense_ref(_ptr(q), _ptr(K), _ptr(V), _dtype_code(q),
                                                     ctypes.byref(shape), float(sm_scale), _ptr(out),
                                                     _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse


def read_probe(src: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One plain coalesced read of the whole of `src` (diagnostics: the read-stream ceiling)."""
    _need(src, "src")
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.zeros(4096, dtype=torch.int32, device=src.device)
    _check("prism_read_probe", load().prism_read_probe(_ptr(src), nbytes - nbytes % 16, _ptr(sink), _stream(stream)))
    return sink


def profile_enable(on: bool = True):
    """Bracket every kernel launch with HIP events on its stream (measurement passes only)."""
    load().prism_profile_enable(1 if on else 0)


def profile_reset():
    load().prism_profile_reset()


def profile_query(name: str) -> Tuple[int, float]:
    """(launches, total milliseconds) of kernel `name` since the last reset; synchronises."""
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _check("prism_profile_query", load().prism_profile_query(name.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


TL_KERNELS = ("k_scan", "k_cand", "k_compact", "k_rscore", "k_attend", "k_select", "k_rows", "k_attend_d")
TL_PHASES = 8


def timeline_clear():
    _check("prism_timeline_clear", load().prism_timeline_clear())


def timeline_read(kernel: str, max_wgs: int):
    """[max_wgs, 8] uint64 real-time stamps (100 MHz) of a kernel's last launch, 0 = not reached
    (timeline build only)."""
    import numpy as np
    out = np.zeros((max_wgs, TL_PHASES), dtype=np.uint64)
    _check("prism_timeline_read", load().prism_timeline_read(TL_KERNELS.index(kernel),
                                                             out.ctypes.data_as(ctypes.c_void_p), max_wgs))
    return out
