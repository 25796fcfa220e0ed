"""Python access to the CPU oracle (oracle/dro.c) through ctypes.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only tests/, the smoke check in
__graft_entry__ and bench.py's CPU-baseline leg import this package.  The
product library (deterministic_gemm_amd) never imports it and shares none of
its code.  Inputs and outputs are numpy arrays on the host.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


class Margin(ctypes.Structure):
    _fields_ = [
        ("sel_min", ctypes.c_float),
        ("rej_max", ctypes.c_float),
        ("sel_min_bf16", ctypes.c_uint16),
        ("rej_max_bf16", ctypes.c_uint16),
        ("ulps", ctypes.c_int32),
    ]


MARGIN_DTYPE = np.dtype(
    [("sel_min", "<f4"), ("rej_max", "<f4"), ("sel_min_bf16", "<u2"), ("rej_max_bf16", "<u2"), ("ulps", "<i4")]
)
assert MARGIN_DTYPE.itemsize == 16


def bind(path: str) -> ctypes.CDLL:
    """ctypes handle with the oracle's signatures for the library at `path`."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32, u32, c_int = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int
    L.dro_bf16_rne.argtypes = [ctypes.c_float]
    L.dro_bf16_rne.restype = ctypes.c_uint16
    L.dro_bf16_ord.argtypes = [ctypes.c_uint16]
    L.dro_bf16_ord.restype = i32
    L.dro_ulps.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
    L.dro_ulps.restype = i32
    L.dro_expf.argtypes = [ctypes.c_float]
    L.dro_expf.restype = ctypes.c_float
    L.dro_expf_array.argtypes = [P, P, i64]
    L.dro_expf_array.restype = None
    L.dro_logits.argtypes = [P, c_int, P, i64, i64, i64, i64, P, c_int]
    L.dro_logits.restype = None
    L.dro_route.argtypes = [P, c_int, P, i64, i64, i64, i32, i64, c_int, u32, P, P, P, P, c_int]
    L.dro_route.restype = c_int
    L.dro_select.argtypes = [P, i64, i64, i32, u32, P, P, P, c_int]
    L.dro_select.restype = c_int
    L.dro_route_split_by_m.argtypes = [P, c_int, P, i64, i64, i64, i32, c_int, u32, P, P, P, P, c_int]
    L.dro_route_split_by_m.restype = c_int
    L.dro_gate_dot.argtypes = [P, c_int, P, c_int, i64, i64, i64, P, P, c_int]
    L.dro_gate_dot.restype = None
    L.dro_gemm_bf16_ref.argtypes = [P, P, P, i64, i64, i64, c_int]
    L.dro_gemm_bf16_ref.restype = None
    L.dro_grouped_gemm_bf16_ref.argtypes = [P, i64, P, P, P, i64, i64, i64, i64, P, c_int]
    L.dro_grouped_gemm_bf16_ref.restype = c_int
    L.dro_moe_permute.argtypes = [P, i64, i32, i32, P, P, P]
    L.dro_moe_permute.restype = c_int
    L.dro_moe_gather.argtypes = [P, i64, P, i64, i64, P]
    L.dro_moe_gather.restype = None
    L.dro_moe_combine.argtypes = [P, c_int, P, P, P, i64, P, c_int, P, i64, i32, i64, P, c_int]
    L.dro_moe_combine.restype = c_int
    L.dro_default_threads.argtypes = []
    L.dro_default_threads.restype = c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = bind(_build.LIB)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _x_arg(x):
    """x as f32, or as bf16 bit patterns stored in uint16."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, 1
    if x.dtype != np.float32:
        raise TypeError("x must be float32 or uint16 (bf16 bits)")
    return x, 0


def default_threads() -> int:
    return lib().dro_default_threads()


def bf16_rne(v: float) -> int:
    return int(lib().dro_bf16_rne(float(v)))


def bf16_ord(b: int) -> int:
    return int(lib().dro_bf16_ord(int(b)))


def ulps(a: int, b: int) -> int:
    return int(lib().dro_ulps(int(a), int(b)))


def expf(t):
    t = np.ascontiguousarray(np.asarray(t, dtype=np.float32))
    out = np.empty_like(t)
    lib().dro_expf_array(_ptr(t), _ptr(out), t.size)
    return out


def logits(x, W, kblock: int = 256, nthreads: int = 0):
    x, xb = _x_arg(x)
    W = np.ascontiguousarray(W, dtype=np.float32)
    M, K = x.shape
    K2, E = W.shape
    assert K == K2
    out = np.empty((M, E), dtype=np.float32)
    lib().dro_logits(_ptr(x), xb, _ptr(W), M, K, E, kblock, _ptr(out), nthreads)
    return out


def route(x, W, k: int, kblock: int = 256, logits_bf16: bool = False, renormalize: bool = False,
          nthreads: int = 0, split_by_m: bool = False):
    """Returns (ids [M,k] int32, weights [M,k] f32, sel_logits [M,E] f32, margins [M] MARGIN_DTYPE).

    sel_logits are the values the selection saw (bf16-rounded and widened when
    logits_bf16)."""
    x, xb = _x_arg(x)
    W = np.ascontiguousarray(W, dtype=np.float32)
    M, K = x.shape
    K2, E = W.shape
    assert K == K2
    ids = np.empty((M, k), dtype=np.int32)
    w = np.empty((M, k), dtype=np.float32)
    lg = np.empty((M, E), dtype=np.float32)
    mg = np.empty((M,), dtype=MARGIN_DTYPE)
    flags = 1 if renormalize else 0
    if split_by_m:
        rc = lib().dro_route_split_by_m(_ptr(x), xb, _ptr(W), M, K, E, k, int(logits_bf16), flags,
                                        _ptr(ids), _ptr(w), _ptr(lg), _ptr(mg), nthreads)
    else:
        rc = lib().dro_route(_ptr(x), xb, _ptr(W), M, K, E, k, kblock, int(logits_bf16), flags,
                             _ptr(ids), _ptr(w), _ptr(lg), _ptr(mg), nthreads)
    if rc != 0:
        raise ValueError("dro_route rejected its arguments")
    return ids, w, lg, mg


def select(logits, k: int, renormalize: bool = False, nthreads: int = 0):
    """dro_select on logits [M,E] (fp32 values, used as given).  Returns
    (ids [M,k] int32, weights [M,k] f32, margins [M] MARGIN_DTYPE)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    M, E = lg.shape
    ids = np.empty((M, k), dtype=np.int32)
    w = np.empty((M, k), dtype=np.float32)
    mg = np.empty((M,), dtype=MARGIN_DTYPE)
    rc = lib().dro_select(_ptr(lg), M, E, k, 1 if renormalize else 0, _ptr(ids), _ptr(w), _ptr(mg), nthreads)
    if rc != 0:
        raise ValueError("dro_select rejected its arguments")
    return ids, w, mg


def gate_dot(x, w, kblock: int = 256, nthreads: int = 0):
    x, xb = _x_arg(x)
    w = np.ascontiguousarray(w)
    wb = 1 if w.dtype == np.uint16 else 0
    if not wb:
        w = w.astype(np.float32)
    M, K = x.shape
    assert w.shape == (K,)
    dot = np.empty((M,), dtype=np.float32)
    gate = np.empty((M,), dtype=np.float32)
    lib().dro_gate_dot(_ptr(x), xb, _ptr(w), wb, M, K, kblock, _ptr(dot), _ptr(gate), nthreads)
    return dot, gate


def gemm_bf16_ref(x_bits, W_bits, nthreads: int = 0):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    M, K = x.shape
    K2, N = W.shape
    assert K == K2
    out = np.empty((M, N), dtype=np.float32)
    lib().dro_gemm_bf16_ref(_ptr(x), _ptr(W), _ptr(out), M, K, N, nthreads)
    return out


def moe_permute(ids, E: int):
    """dro_moe_permute: ids [M,k] int32 -> (offsets [E+1], rows [M*k], pos [M,k]), all int32."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    M, k = ids.shape
    offsets = np.empty((E + 1,), dtype=np.int32)
    rows = np.empty((M * k,), dtype=np.int32)
    pos = np.empty((M, k), dtype=np.int32)
    if lib().dro_moe_permute(_ptr(ids), M, k, E, _ptr(offsets), _ptr(rows), _ptr(pos)) != 0:
        raise ValueError("dro_moe_permute rejected its arguments")
    return offsets, rows, pos


def moe_gather(x, rows):
    """dro_moe_gather: x [M,D] (any dtype) -> xp [P,D] with xp[p] = x[rows[p]]."""
    x = np.ascontiguousarray(x)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    D = x.shape[1]
    xp = np.empty((rows.size, D), dtype=x.dtype)
    lib().dro_moe_gather(_ptr(x), x.itemsize, _ptr(rows), rows.size, D, _ptr(xp))
    return xp


def _elem_arg(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return a, 1
    if a.dtype != np.float32:
        raise TypeError("expected float32 or uint16 (bf16 bits)")
    return a, 0


def moe_combine(y, weights, ids, pos, shared=None, gate=None, nthreads: int = 0):
    """dro_moe_combine: y [P,D] (f32 or bf16 bits), weights/ids/pos [M,k],
    optional shared [M,D] with gate [M] -> out [M,D] f32."""
    y, yb = _elem_arg(y)
    weights = np.ascontiguousarray(weights, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    M, k = ids.shape
    P, D = y.shape
    sb = 0
    if shared is not None:
        shared, sb = _elem_arg(shared)
        gate = np.ascontiguousarray(gate, dtype=np.float32)
    out = np.empty((M, D), dtype=np.float32)
    rc = lib().dro_moe_combine(_ptr(y), yb, _ptr(weights), _ptr(ids), _ptr(pos), P, _ptr(shared), sb,
                               _ptr(gate) if shared is not None else None, M, k, D, _ptr(out), nthreads)
    if rc != 0:
        raise ValueError("dro_moe_combine rejected its arguments")
    return out


def grouped_gemm_bf16_ref(x_bits, W_bits, offsets, rows=None, nthreads: int = 0):
    """dro_grouped_gemm_bf16_ref: x [Mx,K] bf16 bits, W [E,K,N] bf16 bits,
    offsets [E+1], optional rows [P] -> out [P,N] f32 (P = offsets[E])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    E, K, N = W.shape
    Mx = x.shape[0]
    P = int(offsets[-1])
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    out = np.empty((P, N), dtype=np.float32)
    rc = lib().dro_grouped_gemm_bf16_ref(_ptr(x), Mx, _ptr(r), _ptr(W), _ptr(offsets), E, P, K, N, _ptr(out),
                                         nthreads)
    if rc != 0:
        raise ValueError("dro_grouped_gemm_bf16_ref rejected its arguments")
    return out
