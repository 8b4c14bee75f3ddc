"""Packed multi-head attention over live edges on AMD MI355X (gfx950).

A thin binding over ``libpma.so`` (declared in ``include/pma.h``): every
function here has the C entry point's name and only marshals arguments; all
of the computation runs in the library's HIP kernels. Device tensors are
passed as raw pointers; the stream defaults to torch's current stream.

There is no CPU fallback: when ``libpma.so`` is missing, the first call
raises ``ImportError`` (build it with ``python -m graph_sparse_head_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "PmaError", "Plan", "pma_create", "pma_forward", "pma_forward_masked", "pma_forward_static",
    "pma_destroy",
    "pma_train_bytes", "pma_forward_train", "pma_backward",
    "pma_create_graph", "pma_linear_forward", "pma_linear_backward",
    "pma_nnz", "pma_edges", "pma_edge_list",
    "pma_last_error", "pma_plan_info", "pma_csr", "pma_work_split", "pma_profile",
    "pma_profile_stages",
    "pma_profile_read", "pma_gather_probe", "pma_gather_ceiling", "STATUS", "STAGES", "library_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpma.so")
_lib = None

STATUS = {
    0: "PMA_OK", 1: "PMA_E_NULL", 2: "PMA_E_SIZE", 3: "PMA_E_INDEX_EMPTY",
    4: "PMA_E_INDEX_RANGE", 5: "PMA_E_INDEX_DUPLICATE", 6: "PMA_E_SELF_LOOPS",
    7: "PMA_E_DTYPE", 8: "PMA_E_ARG", 9: "PMA_E_OOM", 10: "PMA_E_DEVICE",
    11: "PMA_E_UNSUPPORTED",
}
STAGES = ("proj_in", "edge", "merge", "weights", "out")
_DTYPES = {"f32": 0, "bf16": 1}


class PmaError(RuntimeError):
    """A non-zero pma_status; ``name`` is its enum name."""

    def __init__(self, status: int, message: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {message}")


class _Info(ctypes.Structure):
    _fields_ = [("query_features", ctypes.c_int64), ("key_features", ctypes.c_int64),
                ("embed_dim", ctypes.c_int64), ("num_heads", ctypes.c_int64),
                ("nnz", ctypes.c_int64), ("dtype", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("n_tasks", ctypes.c_int64), ("n_split", ctypes.c_int64),
                ("n_slots", ctypes.c_int64), ("max_degree", ctypes.c_int64),
                ("kv_rows", ctypes.c_int64)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing; build it with "
                          "`python -m graph_sparse_head_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    st = ctypes.c_int
    sig = {
        "pma_create": (st, [ctypes.POINTER(P), P, P, I64, I64, I64, I64, I64, I32, I32, P]),
        "pma_forward": (st, [P, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, I32, P]),
        "pma_forward_masked": (st, [P, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, I32, P, I32,
                                    P]),
        "pma_forward_static": (st, [P, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, I32, P]),
        "pma_train_bytes": (ctypes.c_size_t, [P, I64]),
        "pma_forward_train": (st, [P, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, I32, P, I32, P,
                                   P]),
        "pma_backward": (st, [P, I64, P, P, P, P, P, P, P, I32, P, P, P, I32, P, P, P, P, P, P, P,
                              P, P, P, P, P]),
        "pma_create_graph": (st, [ctypes.POINTER(P), P, P, I64, I64, I64, I32, I32, P]),
        "pma_linear_forward": (st, [P, I64, I64, P, P, P, P, P]),
        "pma_linear_backward": (st, [P, I64, I64, P, P, P, P, P, P, P]),
        "pma_destroy": (st, [P]),
        "pma_nnz": (I64, [P]),
        "pma_edges": (st, [P, P, P]),
        "pma_last_error": (ctypes.c_char_p, []),
        "pma_plan_info": (st, [P, ctypes.POINTER(_Info)]),
        "pma_csr": (st, [P, P, P, P]),
        "pma_work_split": (st, [P] + [P] * 7),
        "pma_profile": (st, [P, I32]),
        "pma_profile_stages": (st, [P, ctypes.c_uint32]),
        "pma_profile_read": (st, [P, P, P]),
        "pma_gather_probe": (st, [P, P]),
        "pma_gather_ceiling": (st, [P, ctypes.c_uint64, P, I64, I64, P, P]),
        "pma_edge_list": (st, [P, P, I64, I64, I64, I32, I64, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise PmaError(status, pma_last_error())


def _host_i64(x, name: str) -> np.ndarray:
    """Host int64 copy of an index argument (tensor, ndarray or sequence)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.ndim != 1:
        raise PmaError(8, f"{name} must be 1-D")
    if a.size and (a.dtype == np.bool_ or not np.issubdtype(a.dtype, np.integer)):
        raise PmaError(8, f"{name} must hold integers")
    return np.ascontiguousarray(a, dtype=np.int64)


def _stream_ptr(stream):
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        return ctypes.c_void_p(None)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """Owner of a ``pma_plan *``; release it with ``pma_destroy``."""

    def __init__(self, handle: ctypes.c_void_p, dtype: str, L: int, S: int, E: int, H: int):
        self.handle = handle
        self.dtype, self.L, self.S, self.E, self.H = dtype, L, S, E, H

    @property
    def nnz(self) -> int:
        return pma_nnz(self)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        pma_destroy(self)


def pma_last_error() -> str:
    return _load().pma_last_error().decode()


def pma_create(source_index, target_index, query_features: int, key_features: int,
               embed_dim: int, num_heads: int, add_self_loops: bool = False,
               dtype: str = "f32", stream=None) -> Plan:
    """Build a plan for one graph (see ``pma_create`` in include/pma.h)."""
    lib = _load()
    src = _host_i64(source_index, "source_index")
    tgt = _host_i64(target_index, "target_index")
    if src.shape[0] != tgt.shape[0]:
        raise PmaError(8, "source_index and target_index differ in length")
    if dtype not in _DTYPES:
        raise PmaError(7, f"dtype must be one of {sorted(_DTYPES)}")
    if not isinstance(add_self_loops, (bool, np.bool_)):
        raise PmaError(8, "add_self_loops must be a bool")
    h = ctypes.c_void_p()
    st = lib.pma_create(ctypes.byref(h), src.ctypes.data, tgt.ctypes.data, src.shape[0],
                        int(query_features), int(key_features), int(embed_dim), int(num_heads),
                        int(bool(add_self_loops)), _DTYPES[dtype], _stream_ptr(stream))
    _check(st)
    return Plan(h, dtype, int(query_features), int(key_features), int(embed_dim), int(num_heads))


def _dptr(t, name: str, dtype, shape_tail: Optional[Sequence[int]] = None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise PmaError(8, f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise PmaError(7, f"{name} has dtype {t.dtype}, the plan uses {dtype}")
    if not t.is_contiguous():
        raise PmaError(8, f"{name} must be contiguous")
    if shape_tail is not None and tuple(t.shape[-len(shape_tail):]) != tuple(shape_tail):
        raise PmaError(2, f"{name} has shape {tuple(t.shape)}, expected (..., "
                          f"{', '.join(map(str, shape_tail))})")
    return t.data_ptr()


def _full_shape(t, name: str, shape) -> None:
    """A caller-supplied buffer must have exactly ``shape``: the kernels read
    or write that many elements through its pointer."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise PmaError(2, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _weights_shape(plan: "Plan", lead, average: bool):
    nnz = pma_nnz(plan)
    return tuple(lead) + ((nnz,) if average else (nnz, plan.H))


def pma_forward_static(plan: Plan, query, key, value, q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b,
                       out=None, weights=None, need_weights: bool = False,
                       average_attn_weights: bool = True, stream=None):
    """``pma_forward_static``: pma_forward without any device allocation in the
    library (its workspace is the library's fixed static scratch; see
    include/pma.h). ``out`` / ``weights`` are allocated here by torch when not
    given, before the call."""
    return pma_forward(plan, query, key, value, q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b, out=out,
                       weights=weights, need_weights=need_weights,
                       average_attn_weights=average_attn_weights, stream=stream,
                       _static=True)


def pma_forward(plan: Plan, query, key, value, q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b,
                out=None, weights=None, need_weights: bool = False,
                average_attn_weights: bool = True, stream=None, key_padding_mask=None,
                _static: bool = False):
    """One forward pass (see ``pma_forward`` / ``pma_forward_masked`` in
    include/pma.h).

    query (..., L, E), key / value (..., S, E) contiguous GPU tensors of the
    plan's dtype with equal leading axes. ``out`` and ``weights`` may be given
    (preallocated) or are allocated here. ``key_padding_mask``: None, or a
    boolean GPU tensor of shape (S,) (every sample) or (..., S) with the
    query's leading axes; True leaves that key out. Returns (out, weights or
    None).
    """
    import torch
    lib = _load()
    tdt = torch.float32 if plan.dtype == "f32" else torch.bfloat16
    L, S, E, H = plan.L, plan.S, plan.E, plan.H
    if query.dim() < 2 or key.dim() < 2 or value.dim() < 2:
        raise PmaError(2, "query, key and value need at least 2 dimensions")
    lead = tuple(query.shape[:-2])
    if tuple(key.shape[:-2]) != lead or tuple(value.shape[:-2]) != lead:
        raise PmaError(2, "the batch axes of query, key and value differ")
    B = int(np.prod(lead)) if lead else 1
    qp = _dptr(query, "query", tdt, (L, E))
    kp = _dptr(key, "key", tdt, (S, E))
    vp = _dptr(value, "value", tdt, (S, E))
    for w, n in ((q_w, "q_w"), (k_w, "k_w"), (v_w, "v_w"), (o_w, "o_w")):
        _full_shape(w, n, (E, E))
    for b, n in ((q_b, "q_b"), (k_b, "k_b"), (v_b, "v_b"), (o_b, "o_b")):
        _full_shape(b, n, (E,))
    wps = [_dptr(w, n, tdt, (E, E)) for w, n in ((q_w, "q_w"), (k_w, "k_w"), (v_w, "v_w"),
                                                  (o_w, "o_w"))]
    bps = [_dptr(b, n, tdt, (E,)) for b, n in ((q_b, "q_b"), (k_b, "k_b"), (v_b, "v_b"),
                                                (o_b, "o_b"))]
    if out is None:
        out = torch.empty(lead + (L, E), dtype=tdt, device=query.device)
    _full_shape(out, "out", lead + (L, E))
    op = _dptr(out, "out", tdt, (L, E))
    want_w = need_weights or weights is not None
    wshape = _weights_shape(plan, lead, average_attn_weights)
    if want_w and weights is None:
        weights = torch.empty(wshape, dtype=torch.float32, device=query.device)
    if want_w:
        _full_shape(weights, "weights", wshape)
    wp = _dptr(weights, "weights", torch.float32) if want_w else None
    if _static:
        if key_padding_mask is not None:
            raise PmaError(8, "pma_forward_static takes no key_padding_mask")
        st = lib.pma_forward_static(plan.handle, B, qp, kp, vp, wps[0], bps[0], wps[1], bps[1],
                                    wps[2], bps[2], wps[3], bps[3], op, wp,
                                    int(bool(average_attn_weights)), _stream_ptr(stream))
    elif key_padding_mask is None:
        st = lib.pma_forward(plan.handle, B, qp, kp, vp, wps[0], bps[0], wps[1], bps[1], wps[2],
                             bps[2], wps[3], bps[3], op, wp, int(bool(average_attn_weights)),
                             _stream_ptr(stream))
    else:
        m = key_padding_mask
        if tuple(m.shape) == (S,):
            per_sample = 0
        elif tuple(m.shape) == lead + (S,):
            per_sample = 1
        else:
            raise PmaError(2, f"key_padding_mask has shape {tuple(m.shape)}, expected ({S},) "
                              f"or {lead + (S,)}")
        mp = _dptr(m, "key_padding_mask", torch.bool)
        st = lib.pma_forward_masked(plan.handle, B, qp, kp, vp, wps[0], bps[0], wps[1], bps[1],
                                    wps[2], bps[2], wps[3], bps[3], op, wp,
                                    int(bool(average_attn_weights)), mp, per_sample,
                                    _stream_ptr(stream))
    _check(st)
    return out, (weights if want_w else None)


def pma_forward_masked(plan: Plan, query, key, value, q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b,
                       key_padding_mask, out=None, weights=None, need_weights: bool = False,
                       average_attn_weights: bool = True, stream=None):
    """``pma_forward`` with a required key_padding_mask (boolean GPU tensor,
    (S,) or the query's leading axes + (S,); True leaves that key out)."""
    if key_padding_mask is None:
        raise PmaError(1, "key_padding_mask is None")
    return pma_forward(plan, query, key, value, q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b, out=out,
                       weights=weights, need_weights=need_weights,
                       average_attn_weights=average_attn_weights, stream=stream,
                       key_padding_mask=key_padding_mask)


def pma_train_bytes(plan: Plan, batch: int) -> int:
    return int(_load().pma_train_bytes(plan.handle, int(batch)))


def _mask_args(m, lead, S):
    if m is None:
        return None, 0
    if tuple(m.shape) == (S,):
        per = 0
    elif tuple(m.shape) == tuple(lead) + (S,):
        per = 1
    else:
        raise PmaError(2, f"key_padding_mask has shape {tuple(m.shape)}, expected ({S},) or "
                          f"{tuple(lead) + (S,)}")
    import torch
    return _dptr(m, "key_padding_mask", torch.bool), per


def pma_forward_train(plan: Plan, query, key, value, q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b,
                      save=None, out=None, weights=None, need_weights: bool = False,
                      average_attn_weights: bool = True, key_padding_mask=None, stream=None):
    """``pma_forward_train``: returns (out, weights or None, save) where save
    is a uint8 GPU tensor holding what ``pma_backward`` needs."""
    import torch
    lib = _load()
    tdt = torch.float32 if plan.dtype == "f32" else torch.bfloat16
    L, S, E, H = plan.L, plan.S, plan.E, plan.H
    lead = tuple(query.shape[:-2])
    B = int(np.prod(lead)) if lead else 1
    if tuple(key.shape[:-2]) != lead or tuple(value.shape[:-2]) != lead:
        raise PmaError(2, "the batch axes of query, key and value differ")
    need = pma_train_bytes(plan, B)
    if save is None:
        save = torch.empty(need, dtype=torch.uint8, device=query.device)
    if save.numel() * save.element_size() < need:
        raise PmaError(2, f"save holds {save.numel() * save.element_size()} bytes, "
                          f"pma_train_bytes gives {need}")
    if out is None:
        out = torch.empty(lead + (L, E), dtype=tdt, device=query.device)
    _full_shape(out, "out", lead + (L, E))
    want_w = need_weights or weights is not None
    wshape = _weights_shape(plan, lead, average_attn_weights)
    if want_w and weights is None:
        weights = torch.empty(wshape, dtype=torch.float32, device=query.device)
    if want_w:
        _full_shape(weights, "weights", wshape)
    for w, n in ((q_w, "q_w"), (k_w, "k_w"), (v_w, "v_w"), (o_w, "o_w")):
        _full_shape(w, n, (E, E))
    for b, n in ((q_b, "q_b"), (k_b, "k_b"), (v_b, "v_b"), (o_b, "o_b")):
        _full_shape(b, n, (E,))
    mp, per = _mask_args(key_padding_mask, lead, S)
    st = lib.pma_forward_train(
        plan.handle, B, _dptr(query, "query", tdt, (L, E)), _dptr(key, "key", tdt, (S, E)),
        _dptr(value, "value", tdt, (S, E)), _dptr(q_w, "q_w", tdt, (E, E)), _dptr(q_b, "q_b", tdt, (E,)),
        _dptr(k_w, "k_w", tdt, (E, E)), _dptr(k_b, "k_b", tdt, (E,)), _dptr(v_w, "v_w", tdt, (E, E)),
        _dptr(v_b, "v_b", tdt, (E,)), _dptr(o_w, "o_w", tdt, (E, E)), _dptr(o_b, "o_b", tdt, (E,)),
        _dptr(out, "out", tdt, (L, E)),
        _dptr(weights, "weights", torch.float32) if want_w else None,
        int(bool(average_attn_weights)), mp, per, _dptr(save, "save", torch.uint8),
        _stream_ptr(stream))
    _check(st)
    return out, (weights if want_w else None), save


def pma_backward(plan: Plan, query, key, value, q_w, k_w, v_w, o_w, has_bias: bool, save,
                 grad_out, key_padding_mask=None, stream=None):
    """``pma_backward``: returns a dict of gradients ("query", "key", "value",
    "q_w", ..., "o_b"; bias entries only with has_bias). A token tensor given
    for several of query / key / value gets one gradient, the sum."""
    import torch
    lib = _load()
    tdt = torch.float32 if plan.dtype == "f32" else torch.bfloat16
    L, S, E = plan.L, plan.S, plan.E
    lead = tuple(query.shape[:-2])
    B = int(np.prod(lead)) if lead else 1
    if tuple(key.shape[:-2]) != lead or tuple(value.shape[:-2]) != lead:
        raise PmaError(2, "the batch axes of query, key and value differ")
    _full_shape(grad_out, "grad_out", lead + (L, E))
    for w, n in ((q_w, "q_w"), (k_w, "k_w"), (v_w, "v_w"), (o_w, "o_w")):
        _full_shape(w, n, (E, E))
    need = pma_train_bytes(plan, B)
    if save.numel() * save.element_size() < need:
        raise PmaError(2, f"save holds {save.numel() * save.element_size()} bytes, "
                          f"pma_train_bytes gives {need}")
    def new(x):
        return torch.empty(x.shape, dtype=tdt, device=x.device)
    gq = new(query)
    gk = gq if key is query else new(key)
    gv = gk if value is key else (gq if value is query else new(value))
    gw = {n: torch.empty(E, E, dtype=tdt, device=query.device) for n in ("q_w", "k_w", "v_w", "o_w")}
    gb = {n: (torch.empty(E, dtype=tdt, device=query.device) if has_bias else None)
          for n in ("q_b", "k_b", "v_b", "o_b")}
    mp, per = _mask_args(key_padding_mask, lead, S)
    st = lib.pma_backward(
        plan.handle, B, _dptr(query, "query", tdt, (L, E)), _dptr(key, "key", tdt, (S, E)),
        _dptr(value, "value", tdt, (S, E)), _dptr(q_w, "q_w", tdt, (E, E)),
        _dptr(k_w, "k_w", tdt, (E, E)), _dptr(v_w, "v_w", tdt, (E, E)),
        _dptr(o_w, "o_w", tdt, (E, E)), int(bool(has_bias)), _dptr(save, "save", torch.uint8),
        _dptr(grad_out, "grad_out", tdt, (L, E)), mp, per, gq.data_ptr(), gk.data_ptr(),
        gv.data_ptr(), gw["q_w"].data_ptr(), _dptr(gb["q_b"], "q_b", tdt),
        gw["k_w"].data_ptr(), _dptr(gb["k_b"], "k_b", tdt), gw["v_w"].data_ptr(),
        _dptr(gb["v_b"], "v_b", tdt), gw["o_w"].data_ptr(), _dptr(gb["o_b"], "o_b", tdt),
        _stream_ptr(stream))
    _check(st)
    res = {"query": gq, "key": gk, "value": gv}
    res.update(gw)
    if has_bias:
        res.update(gb)
    return res


def pma_create_graph(source_index, target_index, query_features: int, key_features: int,
                     add_self_loops: bool = False, dtype: str = "f32", stream=None) -> Plan:
    """A plan for the PackedLinear calls only (see ``pma_create_graph``)."""
    lib = _load()
    src = _host_i64(source_index, "source_index")
    tgt = _host_i64(target_index, "target_index")
    if src.shape[0] != tgt.shape[0]:
        raise PmaError(8, "source_index and target_index differ in length")
    if dtype not in _DTYPES:
        raise PmaError(7, f"dtype must be one of {sorted(_DTYPES)}")
    if not isinstance(add_self_loops, (bool, np.bool_)):
        raise PmaError(8, "add_self_loops must be a bool")
    h = ctypes.c_void_p()
    st = lib.pma_create_graph(ctypes.byref(h), src.ctypes.data, tgt.ctypes.data, src.shape[0],
                              int(query_features), int(key_features), int(bool(add_self_loops)),
                              _DTYPES[dtype], _stream_ptr(stream))
    _check(st)
    return Plan(h, dtype, int(query_features), int(key_features), 0, 0)


def pma_linear_forward(plan: Plan, x, weight, bias=None, out=None, stream=None):
    """``pma_linear_forward``: x (..., S, C) -> out (..., L, C)."""
    import torch
    lib = _load()
    tdt = torch.float32 if plan.dtype == "f32" else torch.bfloat16
    if x.dim() < 2 or x.shape[-2] != plan.S:
        raise PmaError(2, f"x has shape {tuple(x.shape)}, expected (..., {plan.S}, C)")
    C = int(x.shape[-1])
    lead = tuple(x.shape[:-2])
    B = int(np.prod(lead)) if lead else 1
    if out is None:
        out = torch.empty(*lead, plan.L, C, dtype=tdt, device=x.device)
    _full_shape(out, "out", lead + (plan.L, C))
    n = plan.nnz
    _full_shape(weight, "weight", (n,))
    _full_shape(bias, "bias", (plan.L,))
    st = lib.pma_linear_forward(plan.handle, B, C, _dptr(x, "x", tdt, (plan.S, C)),
                                _dptr(weight, "weight", tdt, (n,)),
                                _dptr(bias, "bias", tdt, (plan.L,)),
                                _dptr(out, "out", tdt, (plan.L, C)), _stream_ptr(stream))
    _check(st)
    return out


def pma_linear_backward(plan: Plan, x, weight, grad_out, has_bias: bool = True, stream=None):
    """``pma_linear_backward``: returns (grad_x, grad_weight, grad_bias or None)."""
    import torch
    lib = _load()
    tdt = torch.float32 if plan.dtype == "f32" else torch.bfloat16
    if x.dim() < 2 or x.shape[-2] != plan.S:
        raise PmaError(2, f"x has shape {tuple(x.shape)}, expected (..., {plan.S}, C)")
    C = int(x.shape[-1])
    lead = tuple(x.shape[:-2])
    B = int(np.prod(lead)) if lead else 1
    _full_shape(weight, "weight", (plan.nnz,))
    _full_shape(grad_out, "grad_out", lead + (plan.L, C))
    gx = torch.empty(x.shape, dtype=tdt, device=x.device)
    gw = torch.empty(plan.nnz, dtype=tdt, device=x.device)
    gb = torch.empty(plan.L, dtype=tdt, device=x.device) if has_bias else None
    st = lib.pma_linear_backward(plan.handle, B, C, _dptr(x, "x", tdt, (plan.S, C)),
                                 _dptr(weight, "weight", tdt, (plan.nnz,)),
                                 _dptr(grad_out, "grad_out", tdt, (plan.L, C)), gx.data_ptr(),
                                 gw.data_ptr(), _dptr(gb, "grad_bias", tdt), _stream_ptr(stream))
    _check(st)
    return gx, gw, gb


def pma_destroy(plan: Plan) -> None:
    if plan is None or plan.handle is None or not plan.handle.value:
        return
    _check(_load().pma_destroy(plan.handle))
    plan.handle = ctypes.c_void_p()


def pma_edge_list(source_index, target_index, query_features: int, key_features: int,
                  add_self_loops: bool = False):
    """``pma_edge_list``: the validated final edge list (given pairs, then the
    missing self loops), computed on the host by the library's index rules.
    Returns (src, tgt) int64 arrays."""
    lib = _load()
    src = _host_i64(source_index, "source_index")
    tgt = _host_i64(target_index, "target_index")
    if src.shape[0] != tgt.shape[0]:
        raise PmaError(8, "source_index and target_index differ in length")
    if not isinstance(add_self_loops, (bool, np.bool_)):
        raise PmaError(8, "add_self_loops must be a bool")
    cap = src.shape[0] + (max(int(query_features), 0) if add_self_loops else 0)
    so = np.empty(max(cap, 1), np.int64)
    to = np.empty(max(cap, 1), np.int64)
    n = ctypes.c_int64(0)
    _check(lib.pma_edge_list(src.ctypes.data if src.size else None,
                             tgt.ctypes.data if tgt.size else None, src.shape[0],
                             int(query_features), int(key_features), int(bool(add_self_loops)),
                             cap, so.ctypes.data, to.ctypes.data, ctypes.byref(n)))
    return so[:n.value].copy(), to[:n.value].copy()


def pma_nnz(plan: Plan) -> int:
    return int(_load().pma_nnz(plan.handle))


def pma_edges(plan: Plan):
    n = pma_nnz(plan)
    src = np.empty(n, np.int64)
    tgt = np.empty(n, np.int64)
    _check(_load().pma_edges(plan.handle, src.ctypes.data, tgt.ctypes.data))
    return src, tgt


def pma_plan_info(plan: Plan) -> dict:
    info = _Info()
    _check(_load().pma_plan_info(plan.handle, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in _Info._fields_}


def pma_csr(plan: Plan):
    info = pma_plan_info(plan)
    L, n = info["query_features"], info["nnz"]
    row_ptr = np.empty(L + 1, np.int64)
    src = np.empty(n, np.int64)
    eid = np.empty(n, np.int64)
    _check(_load().pma_csr(plan.handle, row_ptr.ctypes.data, src.ctypes.data, eid.ctypes.data))
    return row_ptr, src, eid


def pma_work_split(plan: Plan) -> dict:
    info = pma_plan_info(plan)
    nt, ns = info["n_tasks"], info["n_split"]
    out = {k: np.empty(nt, np.int64) for k in ("task_target", "task_begin", "task_end",
                                               "task_slot")}
    out.update({k: np.empty(max(ns, 1), np.int64) for k in ("split_target", "split_slot0",
                                                             "split_count")})
    _check(_load().pma_work_split(plan.handle, *(out[k].ctypes.data for k in (
        "task_target", "task_begin", "task_end", "task_slot", "split_target", "split_slot0",
        "split_count"))))
    for k in ("split_target", "split_slot0", "split_count"):
        out[k] = out[k][:ns]
    out["n_slots"] = info["n_slots"]
    return out


def pma_profile(plan: Plan, enable: bool) -> None:
    _check(_load().pma_profile(plan.handle, int(bool(enable))))


def pma_profile_stages(plan: Plan, stages) -> None:
    """Time only the named stages (an iterable of names from STAGES)."""
    mask = 0
    for name in stages:
        mask |= 1 << STAGES.index(name)
    _check(_load().pma_profile_stages(plan.handle, mask))


def pma_profile_read(plan: Plan) -> dict:
    """Per stage: (summed milliseconds, launches timed) since the last read."""
    ms = np.zeros(len(STAGES), np.float64)
    calls = np.zeros(len(STAGES), np.int64)
    _check(_load().pma_profile_read(plan.handle, ms.ctypes.data, calls.ctypes.data))
    return {name: (float(ms[i]), int(calls[i])) for i, name in enumerate(STAGES)}


def pma_gather_probe(plan: Plan, stream=None) -> None:
    """``pma_gather_probe``: the last forward's edge-kernel loads alone."""
    _check(_load().pma_gather_probe(plan.handle, _stream_ptr(stream)))


def pma_gather_ceiling(table, rows, rows_per_wave: int, sink, stream=None) -> None:
    """``pma_gather_ceiling``: 1 KB row gathers from ``table`` (a contiguous
    CUDA tensor of whole KiB) at the int32 CUDA tensor ``rows``; ``sink`` is a
    contiguous CUDA tensor of at least ceil(len(rows) / rows_per_wave) KiB."""
    import torch
    for name, t in (("table", table), ("rows", rows), ("sink", sink)):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
            raise PmaError(8, f"{name} must be a contiguous GPU tensor")
    if rows.dtype != torch.int32 or rows.dim() != 1:
        raise PmaError(7, "rows must be a 1-d int32 tensor")
    n = rows.numel()
    waves = -(-n // rows_per_wave) if rows_per_wave > 0 else 0
    if sink.numel() * sink.element_size() < waves * 1024:
        raise PmaError(2, "sink holds less than 1 KiB per wavefront")
    _check(_load().pma_gather_ceiling(table.data_ptr(), table.numel() * table.element_size(),
                                      rows.data_ptr(), n, rows_per_wave, sink.data_ptr(),
                                      _stream_ptr(stream)))


def __getattr__(name):
    # The nn.Module surface imports torch; load it on first use.
    if name in ("PackedMultiheadAttention", "PackedLinear", "ModuleArgError"):
        from . import module
        return getattr(module, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
