"""Python binding of libdr.so (include/dr.h): batch-invariant MoE routing on
MI355X.

Argument marshalling only.  torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: if the library is not built, or a tensor is not on
the GPU, the call raises.

    ids, weights, logits, margins = route(x, W, k)

x is [M,K] float32 or bfloat16 on the GPU, W is [K,E] float32.  The functions
mirror the C entry points: route -> dr_route, route_variant ->
dr_route_variant, route_logits -> dr_route_logits, route_select ->
dr_route_select, gate_dot -> dr_gate_dot, gemm_bf16 -> dr_gemm_bf16,
contract -> dr_contract.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdr.so")

DR_OK, DR_ERR_INVALID, DR_ERR_UNSUPPORTED, DR_ERR_DEVICE = 0, 1, 2, 3
DR_F32, DR_BF16 = 0, 1
VARIANTS = {"auto": 0, "rowwise": 1, "tiled": 2, "split": 3, "narrow": 4, "tiny": 5, "fused": 6}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}
DR_ROUTE_RENORMALIZE = 1

# dr_margin, 16 bytes per token
MARGIN_DTYPE = np.dtype(
    [("sel_min", "<f4"), ("rej_max", "<f4"), ("sel_min_bf16", "<u2"), ("rej_max_bf16", "<u2"), ("ulps", "<i4")]
)

EXPORTED = (
    "dr_route", "dr_route_noalloc", "dr_route_variant", "dr_route_auto_variant", "dr_route_logits", "dr_route_select",
    "dr_route_bf16_gemm", "dr_gate_dot", "dr_gemm_bf16", "dr_grouped_gemm_bf16", "dr_moe_permute", "dr_moe_gather", "dr_moe_combine", "dr_widen_bf16", "dr_contract",
    "dr_status_string", "dr_last_error",
)


class DrError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class _Contract(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("version", "kblock", "tree", "acc_bits", "fma", "exp_id", "tie_break", "max_k")]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdr.so (build it first with deterministic_gemm_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run python -m deterministic_gemm_amd.build")
    L = ctypes.CDLL(path)
    P, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
    L.dr_route.argtypes = [P, ctypes.c_int, P, i64, i64, i64, i32, ctypes.c_int, P, P, P, P, u32, P]
    L.dr_route.restype = ctypes.c_int
    L.dr_route_noalloc.argtypes = [P, ctypes.c_int, P, i64, i64, i64, i32, ctypes.c_int, P, P, P, P, u32, P]
    L.dr_route_noalloc.restype = ctypes.c_int
    L.dr_route_variant.argtypes = [P, ctypes.c_int, P, i64, i64, i64, i32, ctypes.c_int, P, P, P, P, u32,
                                   ctypes.c_int, P]
    L.dr_route_variant.restype = ctypes.c_int
    L.dr_route_auto_variant.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_int]
    L.dr_route_auto_variant.restype = ctypes.c_int
    L.dr_route_logits.argtypes = [P, P, i64, i64, i64, ctypes.c_int, P, P]
    L.dr_route_logits.restype = ctypes.c_int
    L.dr_route_select.argtypes = [P, ctypes.c_int, i64, i64, i32, P, P, P, u32, P]
    L.dr_route_select.restype = ctypes.c_int
    L.dr_gate_dot.argtypes = [P, ctypes.c_int, P, ctypes.c_int, P, P, i64, i64, P]
    L.dr_gate_dot.restype = ctypes.c_int
    L.dr_gemm_bf16.argtypes = [P, P, P, i64, i64, i64, P]
    L.dr_gemm_bf16.restype = ctypes.c_int
    L.dr_route_bf16_gemm.argtypes = [P, P, i64, i64, i64, i32, P, P, P, P, u32, P]
    L.dr_route_bf16_gemm.restype = ctypes.c_int
    L.dr_grouped_gemm_bf16.argtypes = [P, i64, P, P, P, i64, i64, i64, i64, P, P]
    L.dr_grouped_gemm_bf16.restype = ctypes.c_int
    L.dr_moe_permute.argtypes = [P, i64, i32, i32, P, P, P, P]
    L.dr_moe_permute.restype = ctypes.c_int
    L.dr_moe_gather.argtypes = [P, ctypes.c_int, i64, i64, P, i64, P, P]
    L.dr_moe_gather.restype = ctypes.c_int
    L.dr_widen_bf16.argtypes = [P, i64, P, P]
    L.dr_widen_bf16.restype = ctypes.c_int
    L.dr_moe_combine.argtypes = [P, ctypes.c_int, i64, P, P, P, P, ctypes.c_int, P, i64, i32, i64, P, P]
    L.dr_moe_combine.restype = ctypes.c_int
    L.dr_contract.argtypes = [ctypes.POINTER(_Contract)]
    L.dr_contract.restype = None
    L.dr_status_string.argtypes = [ctypes.c_int]
    L.dr_status_string.restype = ctypes.c_char_p
    L.dr_last_error.argtypes = []
    L.dr_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int, where: str):
    if status != DR_OK:
        L = load_library()
        detail = L.dr_last_error().decode() or L.dr_status_string(status).decode()
        raise DrError(status, where, detail)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_tensor(t, name, dtypes):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out_tensor(t, name, dtype, shape, device):
    """Checks a caller-supplied output (or extra input) tensor against exactly
    what the C call will write through its pointer: a torch tensor on
    `device`, of `dtype`, contiguous, of `shape`.  Raises TypeError or
    ValueError; the kernels would otherwise write past a smaller
    allocation."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _same_device(t, name, device):
    if t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device} (the device of the first operand), got {t.device}")
    return t


def contract() -> dict:
    c = _Contract()
    load_library().dr_contract(ctypes.byref(c))
    return {n: getattr(c, n) for n, _ in _Contract._fields_}


def auto_variant(M: int, K: int, E: int, x_dtype: str = "f32", logits: bool = True) -> str:
    """dr_route_auto_variant: the kernel family dr_route runs for this call shape."""
    xd = {"f32": DR_F32, "bf16": DR_BF16}[x_dtype]
    return VARIANT_NAMES[load_library().dr_route_auto_variant(M, K, E, xd, int(bool(logits)))]


def scratch_logits_used(M: int, K: int, E: int, x_dtype: str = "f32") -> bool:
    """Whether route(..., logits=False) passes a temporary logits buffer: when
    the library's dispatch with a logits buffer picks a two-kernel family
    (tiny, narrow or split), which the fused families do not match for speed."""
    return auto_variant(M, K, E, x_dtype, logits=True) in ("tiny", "narrow", "split")


def widen_bf16_used(M: int, K: int, E: int) -> bool:
    """Whether route(...) with bf16 x and variant "auto" widens x to fp32
    first (dr_widen_bf16): when the fp32 dispatch with a logits buffer picks
    an LDS-staged family (tiny, narrow or split) and the bf16 dispatch does
    not (the vector-ALU family reads bf16 itself).  The results are the same
    bits either way."""
    fast = ("tiny", "narrow", "split")
    return auto_variant(M, K, E, "f32", logits=True) in fast and auto_variant(M, K, E, "bf16", logits=True) not in fast


def route(x, W, k: int, *, logit_dtype: str = "f32", renormalize: bool = False, logits: bool = True,
          weights: bool = True, margins: bool = True, variant: str = "auto", out=None,
          scratch_logits: bool = True):
    """dr_route / dr_route_variant.  Returns (ids [M,k] int32, weights [M,k]
    float32 or None, logits [M,E] float32/bfloat16 or None, margins [M,4] int32
    raw dr_margin records or None).  `out` may pass preallocated tensors as a
    tuple in the same order.  With logits=False, variant "auto" and
    scratch_logits, a temporary logits tensor is passed (and dropped) when
    that lets the library pick a faster family (scratch_logits_used)."""
    L = load_library()
    _dev_tensor(x, "x", (torch.float32, torch.bfloat16))
    _dev_tensor(W, "W", (torch.float32,))
    if x.dim() != 2 or W.dim() != 2 or x.shape[1] != W.shape[0]:
        raise ValueError("x must be [M,K] and W [K,E]")
    M, K = x.shape
    E = W.shape[1]
    dev = x.device
    _same_device(W, "W", dev)
    ldt = {"f32": DR_F32, "bf16": DR_BF16}[logit_dtype]
    ldtype = torch.float32 if ldt == DR_F32 else torch.bfloat16
    if out is not None:
        ids_t, w_t, lg_t, mg_t = out
        _out_tensor(ids_t, "ids", torch.int32, (M, k), dev)
        if w_t is not None:
            _out_tensor(w_t, "weights", torch.float32, (M, k), dev)
        if lg_t is not None:
            _out_tensor(lg_t, "logits", ldtype, (M, E), dev)
        if mg_t is not None:
            _out_tensor(mg_t, "margins", torch.int32, (M, 4), dev)
    else:
        ids_t = torch.empty((M, k), dtype=torch.int32, device=dev)
        w_t = torch.empty((M, k), dtype=torch.float32, device=dev) if weights else None
        lg_t = (torch.empty((M, E), dtype=torch.float32 if ldt == DR_F32 else torch.bfloat16, device=dev)
                if logits else None)
        mg_t = torch.empty((M, 4), dtype=torch.int32, device=dev) if margins else None
    v = VARIANTS[variant]
    if x.dtype == torch.bfloat16 and v == 0 and widen_bf16_used(M, K, E):
        x = widen_bf16(x)
    xd = DR_F32 if x.dtype == torch.float32 else DR_BF16
    flags = DR_ROUTE_RENORMALIZE if renormalize else 0
    lg_pass = lg_t
    if (lg_t is None and v == 0 and scratch_logits
            and scratch_logits_used(M, K, E, "f32" if xd == DR_F32 else "bf16")):
        lg_pass = torch.empty((M, E), dtype=torch.float32 if ldt == DR_F32 else torch.bfloat16, device=dev)
    if v == 0:
        st = L.dr_route(_ptr(x), xd, _ptr(W), M, K, E, k, ldt, _ptr(ids_t), _ptr(w_t), _ptr(lg_pass), _ptr(mg_t),
                        flags, _stream(dev))
    else:
        st = L.dr_route_variant(_ptr(x), xd, _ptr(W), M, K, E, k, ldt, _ptr(ids_t), _ptr(w_t), _ptr(lg_t),
                                _ptr(mg_t), flags, v, _stream(dev))
    _check(st, "dr_route")
    return ids_t, w_t, lg_t, mg_t


def route_noalloc(x, W, k: int, out, *, logit_dtype: str = "f32", renormalize: bool = False):
    """dr_route_noalloc: dr_route that allocates nothing, for callers that
    cannot (graph capture, serving loops).  `out` = (ids [M,k] int32,
    weights [M,k] float32 or None, logits [M,E] or None, margins [M,4] int32
    or None), all preallocated; nothing is allocated here either.  With
    logits None the two-launch families keep their logits in the library's
    static 16 MiB device buffer (M*E*4 bytes at most).  Returns out."""
    L = load_library()
    _dev_tensor(x, "x", (torch.float32, torch.bfloat16))
    _dev_tensor(W, "W", (torch.float32,))
    if x.dim() != 2 or W.dim() != 2 or x.shape[1] != W.shape[0]:
        raise ValueError("x must be [M,K] and W [K,E]")
    M, K = x.shape
    E = W.shape[1]
    dev = x.device
    _same_device(W, "W", dev)
    ldt = {"f32": DR_F32, "bf16": DR_BF16}[logit_dtype]
    ids_t, w_t, lg_t, mg_t = out
    _out_tensor(ids_t, "ids", torch.int32, (M, k), dev)
    if w_t is not None:
        _out_tensor(w_t, "weights", torch.float32, (M, k), dev)
    if lg_t is not None:
        _out_tensor(lg_t, "logits", torch.float32 if ldt == DR_F32 else torch.bfloat16, (M, E), dev)
    if mg_t is not None:
        _out_tensor(mg_t, "margins", torch.int32, (M, 4), dev)
    xd = DR_F32 if x.dtype == torch.float32 else DR_BF16
    st = L.dr_route_noalloc(_ptr(x), xd, _ptr(W), M, K, E, k, ldt, _ptr(ids_t), _ptr(w_t), _ptr(lg_t), _ptr(mg_t),
                            DR_ROUTE_RENORMALIZE if renormalize else 0, _stream(dev))
    _check(st, "dr_route_noalloc")
    return out


def route_variant(x, W, k: int, variant: str, **kw):
    return route(x, W, k, variant=variant, **kw)


def route_logits(x, W, *, logit_dtype: str = "f32", out=None):
    """dr_route_logits: x [M,K] float32, W [K,E] float32 -> logits [M,E]
    float32 (or bfloat16 with logit_dtype="bf16")."""
    L = load_library()
    _dev_tensor(x, "x", (torch.float32,))
    _dev_tensor(W, "W", (torch.float32,))
    if x.dim() != 2 or W.dim() != 2 or x.shape[1] != W.shape[0]:
        raise ValueError("x must be [M,K] and W [K,E]")
    M, K = x.shape
    E = W.shape[1]
    _same_device(W, "W", x.device)
    ldt = {"f32": DR_F32, "bf16": DR_BF16}[logit_dtype]
    ldtype = torch.float32 if ldt == DR_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((M, E), dtype=ldtype, device=x.device)
    _out_tensor(out, "out", ldtype, (M, E), x.device)
    st = L.dr_route_logits(_ptr(x), _ptr(W), M, K, E, ldt, _ptr(out), _stream(x.device))
    _check(st, "dr_route_logits")
    return out


def route_select(logits, k: int, *, renormalize: bool = False, weights: bool = True, margins: bool = True,
                 out=None):
    """dr_route_select: logits [M,E] float32 or bfloat16 -> (ids [M,k] int32,
    weights [M,k] float32 or None, margins [M,4] int32 raw dr_margin records
    or None)."""
    L = load_library()
    _dev_tensor(logits, "logits", (torch.float32, torch.bfloat16))
    if logits.dim() != 2:
        raise ValueError("logits must be [M,E]")
    M, E = logits.shape
    dev = logits.device
    if out is not None:
        ids_t, w_t, mg_t = out
        _out_tensor(ids_t, "ids", torch.int32, (M, k), dev)
        if w_t is not None:
            _out_tensor(w_t, "weights", torch.float32, (M, k), dev)
        if mg_t is not None:
            _out_tensor(mg_t, "margins", torch.int32, (M, 4), dev)
    else:
        ids_t = torch.empty((M, k), dtype=torch.int32, device=dev)
        w_t = torch.empty((M, k), dtype=torch.float32, device=dev) if weights else None
        mg_t = torch.empty((M, 4), dtype=torch.int32, device=dev) if margins else None
    ldt = DR_F32 if logits.dtype == torch.float32 else DR_BF16
    st = L.dr_route_select(_ptr(logits), ldt, M, E, k, _ptr(ids_t), _ptr(w_t), _ptr(mg_t),
                           DR_ROUTE_RENORMALIZE if renormalize else 0, _stream(dev))
    _check(st, "dr_route_select")
    return ids_t, w_t, mg_t


def gate_dot(x, w, *, dot: bool = True, gate: bool = True):
    """dr_gate_dot: returns (dot [M] float32 or None, gate [M] float32 or None)."""
    L = load_library()
    _dev_tensor(x, "x", (torch.float32, torch.bfloat16))
    _dev_tensor(w, "w", (torch.float32, torch.bfloat16))
    if x.dim() != 2:
        raise ValueError("x must be [M,K]")
    M, K = x.shape
    if w.shape != (K,):
        raise ValueError("w must be [K]")
    _same_device(w, "w", x.device)
    d = torch.empty((M,), dtype=torch.float32, device=x.device) if dot else None
    g = torch.empty((M,), dtype=torch.float32, device=x.device) if gate else None
    st = L.dr_gate_dot(_ptr(x), DR_F32 if x.dtype == torch.float32 else DR_BF16, _ptr(w),
                       DR_F32 if w.dtype == torch.float32 else DR_BF16, _ptr(d), _ptr(g), M, K, _stream(x.device))
    _check(st, "dr_gate_dot")
    return d, g


def moe_permute(ids, E: int, out=None):
    """dr_moe_permute: ids [M,k] int32 -> (offsets [E+1], rows [M*k], pos [M,k]), int32 device tensors."""
    L = load_library()
    _dev_tensor(ids, "ids", (torch.int32,))
    if ids.dim() != 2:
        raise ValueError("ids must be [M,k]")
    M, k = ids.shape
    dev = ids.device
    if out is not None:
        offsets, rows, pos = out
        _out_tensor(offsets, "offsets", torch.int32, (E + 1,), dev)
        _out_tensor(rows, "rows", torch.int32, (M * k,), dev)
        _out_tensor(pos, "pos", torch.int32, (M, k), dev)
    else:
        offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        rows = torch.empty((M * k,), dtype=torch.int32, device=dev)
        pos = torch.empty((M, k), dtype=torch.int32, device=dev)
    st = L.dr_moe_permute(_ptr(ids), M, k, E, _ptr(offsets), _ptr(rows), _ptr(pos), _stream(dev))
    _check(st, "dr_moe_permute")
    return offsets, rows, pos


def widen_bf16(x, out=None):
    """dr_widen_bf16: a bfloat16 tensor widened exactly to float32 (same shape)."""
    L = load_library()
    _dev_tensor(x, "x", (torch.bfloat16,))
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _out_tensor(out, "out", torch.float32, x.shape, x.device)
    _check(L.dr_widen_bf16(_ptr(x), x.numel(), _ptr(out), _stream(x.device)), "dr_widen_bf16")
    return out


def moe_gather(x, rows, out=None):
    """dr_moe_gather: x [M,D] float32 or bfloat16, rows [P] int32 -> xp [P,D] with xp[p] = x[rows[p]]."""
    L = load_library()
    _dev_tensor(x, "x", (torch.float32, torch.bfloat16))
    _dev_tensor(rows, "rows", (torch.int32,))
    if x.dim() != 2 or rows.dim() != 1:
        raise ValueError("x must be [M,D] and rows [P]")
    _same_device(rows, "rows", x.device)
    M, D = x.shape
    P = rows.numel()
    xp = out if out is not None else torch.empty((P, D), dtype=x.dtype, device=x.device)
    _out_tensor(xp, "out", x.dtype, (P, D), x.device)
    st = L.dr_moe_gather(_ptr(x), DR_F32 if x.dtype == torch.float32 else DR_BF16, M, D, _ptr(rows), P,
                         _ptr(xp), _stream(x.device))
    _check(st, "dr_moe_gather")
    return xp


def moe_combine(y, weights, ids, pos, shared=None, gate=None, out=None):
    """dr_moe_combine: y [P,D] float32 or bfloat16, weights [M,k] float32, ids and
    pos [M,k] int32, optional shared [M,D] with gate [M] -> out [M,D] float32."""
    L = load_library()
    _dev_tensor(y, "y", (torch.float32, torch.bfloat16))
    _dev_tensor(weights, "weights", (torch.float32,))
    _dev_tensor(ids, "ids", (torch.int32,))
    _dev_tensor(pos, "pos", (torch.int32,))
    if y.dim() != 2 or ids.dim() != 2:
        raise ValueError("y must be [P,D] and ids [M,k]")
    P, D = y.shape
    M, k = ids.shape
    dev = y.device
    _out_tensor(weights, "weights", torch.float32, (M, k), dev)
    _out_tensor(ids, "ids", torch.int32, (M, k), dev)
    _out_tensor(pos, "pos", torch.int32, (M, k), dev)
    sdt = DR_F32
    if shared is not None:
        _dev_tensor(shared, "shared", (torch.float32, torch.bfloat16))
        _out_tensor(shared, "shared", shared.dtype, (M, D), dev)
        if gate is None:
            raise ValueError("gate is required with shared")
        _out_tensor(gate, "gate", torch.float32, (M,), dev)
        sdt = DR_F32 if shared.dtype == torch.float32 else DR_BF16
    o = out if out is not None else torch.empty((M, D), dtype=torch.float32, device=dev)
    _out_tensor(o, "out", torch.float32, (M, D), dev)
    st = L.dr_moe_combine(_ptr(y), DR_F32 if y.dtype == torch.float32 else DR_BF16, P, _ptr(weights), _ptr(ids),
                          _ptr(pos), _ptr(shared), sdt, _ptr(gate) if shared is not None else None, M, k, D,
                          _ptr(o), _stream(y.device))
    _check(st, "dr_moe_combine")
    return o


def route_bf16_gemm(x, W, k: int, *, renormalize: bool = False, weights: bool = True, margins: bool = True):
    """dr_route_bf16_gemm: x [M,K] bfloat16, W [K,E] bfloat16 -> (ids [M,k]
    int32, weights [M,k] float32 or None, logits [M,E] bfloat16, margins
    [M,4] int32 raw dr_margin records or None)."""
    L = load_library()
    _dev_tensor(x, "x", (torch.bfloat16,))
    _dev_tensor(W, "W", (torch.bfloat16,))
    if x.dim() != 2 or W.dim() != 2:
        raise ValueError("x must be [M,K] and W [K,E]")
    M, K = x.shape
    K2, E = W.shape
    if K != K2:
        raise ValueError("inner sizes differ")
    dev = x.device
    _same_device(W, "W", dev)
    ids_t = torch.empty((M, k), dtype=torch.int32, device=dev)
    w_t = torch.empty((M, k), dtype=torch.float32, device=dev) if weights else None
    lg_t = torch.empty((M, E), dtype=torch.bfloat16, device=dev)
    mg_t = torch.empty((M, 4), dtype=torch.int32, device=dev) if margins else None
    st = L.dr_route_bf16_gemm(_ptr(x), _ptr(W), M, K, E, k, _ptr(ids_t), _ptr(w_t), _ptr(lg_t), _ptr(mg_t),
                              DR_ROUTE_RENORMALIZE if renormalize else 0, _stream(dev))
    _check(st, "dr_route_bf16_gemm")
    return ids_t, w_t, lg_t, mg_t


def grouped_gemm_bf16(x, W, offsets, rows=None, out=None):
    """dr_grouped_gemm_bf16: x [Mx,K] bfloat16, W [E,K,N] bfloat16, offsets
    [E+1] int32, rows [P] int32 or None (then P = Mx) -> out [P,N] float32."""
    L = load_library()
    _dev_tensor(x, "x", (torch.bfloat16,))
    _dev_tensor(W, "W", (torch.bfloat16,))
    _dev_tensor(offsets, "offsets", (torch.int32,))
    if x.dim() != 2 or W.dim() != 3:
        raise ValueError("x must be [Mx,K] and W [E,K,N]")
    Mx, K = x.shape
    E, K2, N = W.shape
    if K != K2:
        raise ValueError("inner sizes differ")
    _same_device(W, "W", x.device)
    _out_tensor(offsets, "offsets", torch.int32, (E + 1,), x.device)
    if rows is not None:
        _dev_tensor(rows, "rows", (torch.int32,))
        if rows.dim() != 1:
            raise ValueError("rows must be [P]")
        _same_device(rows, "rows", x.device)
        P = rows.numel()
    else:
        P = Mx
    o = out if out is not None else torch.empty((P, N), dtype=torch.float32, device=x.device)
    _out_tensor(o, "out", torch.float32, (P, N), x.device)
    st = L.dr_grouped_gemm_bf16(_ptr(x), Mx, _ptr(rows), _ptr(W), _ptr(offsets), E, P, K, N, _ptr(o),
                                _stream(x.device))
    _check(st, "dr_grouped_gemm_bf16")
    return o


def gemm_bf16(x, W, out=None):
    """dr_gemm_bf16: x [M,K] bfloat16, W [K,N] bfloat16 -> out [M,N] float32."""
    L = load_library()
    _dev_tensor(x, "x", (torch.bfloat16,))
    _dev_tensor(W, "W", (torch.bfloat16,))
    if x.dim() != 2 or W.dim() != 2:
        raise ValueError("x must be [M,K] and W [K,N]")
    M, K = x.shape
    K2, N = W.shape
    if K != K2:
        raise ValueError("inner sizes differ")
    _same_device(W, "W", x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _out_tensor(out, "out", torch.float32, (M, N), x.device)
    st = L.dr_gemm_bf16(_ptr(x), _ptr(W), _ptr(out), M, K, N, _stream(x.device))
    _check(st, "dr_gemm_bf16")
    return out


def margins_to_numpy(mg: torch.Tensor) -> np.ndarray:
    """Raw [M,4] int32 dr_margin records -> numpy structured array."""
    return np.ascontiguousarray(mg.cpu().numpy()).view(MARGIN_DTYPE).reshape(-1)


dr_route = route
dr_route_noalloc = route_noalloc
dr_route_variant = route_variant
dr_route_logits = route_logits
dr_route_select = route_select
dr_gate_dot = gate_dot
dr_gemm_bf16 = gemm_bf16
dr_contract = contract
dr_widen_bf16 = widen_bf16
