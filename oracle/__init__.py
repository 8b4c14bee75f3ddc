"""CPU oracle for packed multi-head attention over live edges.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg use it; the product path never does. It shares no
code with the GPU library and imports nothing from it.

What it computes follows the kpnn2 ``PackedMultiheadAttention`` page:
  * the constructor's index rules (parameter table: source_index,
    target_index, add_self_loops; "Raises" section) -> ``prepare_edges``;
  * the forward pass ("Notes", steps 1-5, and the paragraph on queries with
    no live keys) -> ``forward``, computed in double precision by the plain C
    loops in ``pma_oracle.c``;
  * ``need_weights`` / ``average_attn_weights`` (forward "Returns") ->
    ``average_heads``.
Two integer references describe the GPU plan's internal layout, so that the
index build can be compared bit for bit: ``csr`` (edges grouped by target,
sources ascending) and ``work_split`` (the plan's stated split of long
targets into pieces). Those two are this library's design, not the page's.

Parity pins for every function live in tests/test_oracle.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pma_oracle.c")
_LIB = os.path.join(_HERE, "_pma_oracle.so")
_lib = None


class OracleError(ValueError):
    """A rejected constructor argument; ``code`` names the rule."""

    def __init__(self, code: str, msg: str):
        super().__init__(msg)
        self.code = code


# --------------------------------------------------------------------------
# build / load


def build() -> str:
    """Compile pma_oracle.c with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_forward.argtypes = [i64] * 5 + [p] * 3 + [p] * 8 + [i64, p, p] + [i64, p, p] + \
        [p, p, p, p, i64, ctypes.c_int]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def num_threads(nthreads: int = 0) -> int:
    """Threads the oracle uses for ``nthreads`` (0: the OpenMP default)."""
    return int(_load().oracle_num_threads(int(nthreads)))


# --------------------------------------------------------------------------
# constructor rules


def _as_index(x, name: str) -> np.ndarray:
    if isinstance(x, (set, frozenset, dict)):
        raise OracleError("arg", f"{name}: a set or mapping has no pairing order")
    a = np.asarray(x)
    if a.ndim != 1:
        raise OracleError("arg", f"{name} must be 1-D")
    if a.shape[0] == 0:
        raise OracleError("index_empty", "indices must not be empty")
    if a.dtype == np.bool_ or not np.issubdtype(a.dtype, np.integer):
        raise OracleError("arg", f"{name} must hold integers")
    return a.astype(np.int64, copy=True)


def prepare_edges(source_index, target_index, query_features: int, key_features: int,
                  embed_dim: int, num_heads: int, add_self_loops: bool = False):
    """Validate the constructor arguments and return the final live edges.

    Rules (kpnn2 page, parameter table and "Raises"): 1-D integer indices of
    equal length nnz >= 1; 0 <= source < key_features and 0 <= target <
    query_features; no repeated (source, target) pair; positive sizes;
    embed_dim divisible by num_heads; add_self_loops requires query_features
    == key_features. With add_self_loops, every missing (i, i) is appended
    after the given pairs, in ascending i (the page says only "after the given
    pairs"; its example lists the added loops in node order). The inputs are
    copied, never modified.

    Returns (src, tgt) int64 arrays in edge-id order.
    """
    L, S, E, H = (int(v) for v in (query_features, key_features, embed_dim, num_heads))
    for v, nm in ((L, "query_features"), (S, "key_features"), (E, "embed_dim"), (H, "num_heads")):
        if v <= 0:
            raise OracleError("size", f"{nm} must be positive")
    if E % H != 0:
        raise OracleError("size", "embed_dim must be divisible by num_heads")
    src = _as_index(source_index, "source_index")
    tgt = _as_index(target_index, "target_index")
    if src.shape[0] == 0 or tgt.shape[0] == 0:
        raise OracleError("index_empty", "indices must not be empty")
    if src.shape[0] != tgt.shape[0]:
        raise OracleError("arg", "source_index and target_index differ in length")
    if src.min() < 0 or src.max() >= S:
        raise OracleError("index_range", "source_index out of range")
    if tgt.min() < 0 or tgt.max() >= L:
        raise OracleError("index_range", "target_index out of range")
    key = src * L + tgt                     # one integer per (source, target) pair
    uniq, counts = np.unique(key, return_counts=True)
    if (counts > 1).any():
        k = int(uniq[np.argmax(counts > 1)])
        raise OracleError("index_duplicate", f"repeated pair ({k // L}, {k % L})")
    if add_self_loops:
        if L != S:
            raise OracleError("self_loops", "add_self_loops needs query_features == key_features")
        has_loop = np.zeros(L, bool)
        has_loop[src[src == tgt]] = True
        extra = np.nonzero(~has_loop)[0].astype(np.int64)   # ascending node index
        src = np.concatenate([src, extra])
        tgt = np.concatenate([tgt, extra])
    return src, tgt


# --------------------------------------------------------------------------
# integer layout references (the GPU plan's design)


def csr(src: np.ndarray, tgt: np.ndarray, L: int):
    """Edges grouped by target, sources ascending within a target.

    row_ptr[t] counts the edges whose target is below t; within a row the
    edges are ordered by source (unique, since pairs do not repeat). Returns
    (row_ptr int64 (L+1,), csr_src int64 (nnz,), csr_eid int64 (nnz,)), where
    csr_eid is the position of each entry in the edge list.
    """
    src = np.asarray(src, np.int64)
    tgt = np.asarray(tgt, np.int64)
    order = np.lexsort((src, tgt))          # primary key target, then source
    row_ptr = np.zeros(L + 1, np.int64)
    row_ptr[1:] = np.cumsum(np.bincount(tgt, minlength=L))
    return row_ptr, src[order], order.astype(np.int64)


def work_split(row_ptr: np.ndarray, chunk: int):
    """The plan's split of targets into pieces of at most ``chunk`` edges.

    A target of degree g becomes n = max(1, ceil(g / chunk)) pieces; piece j
    covers CSR positions row_ptr[t] + floor(j g / n) .. row_ptr[t] +
    floor((j+1) g / n). Pieces are ordered by the bucket (chunk - length) // 16
    (longest bucket first), ties by ascending target then piece. Targets with
    n > 1 own n consecutive partial slots, numbered in ascending target order;
    a lone piece has slot -1.

    Returns dict of int64 arrays: task_target, task_begin, task_end,
    task_slot; split_target, split_slot0, split_count; and n_slots.
    """
    row_ptr = np.asarray(row_ptr, np.int64)
    L = row_ptr.shape[0] - 1
    items = []                          # (length, t, j, begin, end)
    split_t, split_s0, split_n = [], [], []
    slot = 0
    first_slot = {}
    for t in range(L):
        g = int(row_ptr[t + 1] - row_ptr[t])
        n = max(1, -(-g // chunk))
        if n > 1:
            first_slot[t] = slot
            split_t.append(t)
            split_s0.append(slot)
            split_n.append(n)
            slot += n
        for j in range(n):
            b = int(row_ptr[t]) + (j * g) // n
            e = int(row_ptr[t]) + ((j + 1) * g) // n
            items.append((e - b, t, j, b, e))
    items.sort(key=lambda it: ((chunk - it[0]) // 16, it[1], it[2]))
    tt = np.array([it[1] for it in items], np.int64)
    tb = np.array([it[3] for it in items], np.int64)
    te = np.array([it[4] for it in items], np.int64)
    ts = np.array([first_slot[it[1]] + it[2] if it[1] in first_slot else -1 for it in items],
                  np.int64)
    return {
        "task_target": tt, "task_begin": tb, "task_end": te, "task_slot": ts,
        "split_target": np.array(split_t, np.int64), "split_slot0": np.array(split_s0, np.int64),
        "split_count": np.array(split_n, np.int64), "n_slots": slot,
    }


# --------------------------------------------------------------------------
# forward


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored inputs: fp32 values, or bfloat16 bit
    patterns (a bfloat16 is the top 16 bits of a float32)."""
    if a is None:
        return None
    if dtype == "bf16":
        u = np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float64)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward(B: int, L: int, S: int, E: int, H: int, xq, xk, xv, params: Dict[str, Optional[np.ndarray]],
            src, tgt, rows: Optional[np.ndarray] = None, want_weights: bool = False,
            want_mixed: bool = False, nthreads: int = 0, key_padding_mask=None):
    """Packed multi-head attention forward in double precision.

    xq (B, L, E), xk / xv (B, S, E) float64; params wq bq wk bk wv bv wo bo
    (biases all present or all None); src / tgt the final edge list (see
    ``prepare_edges``). ``rows`` is an (n, 2) array of (sample, target) pairs
    to compute, or None for every row.

    ``key_padding_mask``: None, or a boolean (S,) mask shared by every sample
    or (B, S) per sample; True leaves that key out of the sample's softmax.

    Returns dict: "out" (n, E) or (B, L, E) when rows is None; "mixed" the
    joined heads before out_proj (same shape) if asked; "weights" (B, nnz, H)
    per-head edge weights if asked (NaN for edges into rows not computed).
    """
    lib = _load()
    B, L, S, E, H = (int(v) for v in (B, L, S, E, H))
    if E % H:
        raise OracleError("size", "embed_dim must be divisible by num_heads")
    xq, xk, xv = _f64(xq), _f64(xk), _f64(xv)
    assert xq.shape == (B, L, E) and xk.shape == (B, S, E) and xv.shape == (B, S, E)
    w = {k: _f64(params.get(k)) for k in ("wq", "bq", "wk", "bk", "wv", "bv", "wo", "bo")}
    for k in ("wq", "wk", "wv", "wo"):
        assert w[k] is not None and w[k].shape == (E, E), k
    nb = sum(w[k] is None for k in ("bq", "bk", "bv", "bo"))
    assert nb in (0, 4), "biases are all present or all absent"
    src = np.ascontiguousarray(src, np.int64)
    tgt = np.ascontiguousarray(tgt, np.int64)
    nnz = src.shape[0]
    if rows is None:
        nrows = B * L
        rb = rt = None
    else:
        rows = np.asarray(rows, np.int64).reshape(-1, 2)
        nrows = rows.shape[0]
        rb = np.ascontiguousarray(rows[:, 0])
        rt = np.ascontiguousarray(rows[:, 1])
        assert (rb >= 0).all() and (rb < B).all() and (rt >= 0).all() and (rt < L).all()
    kpm, kstride = None, 0
    if key_padding_mask is not None:
        km = np.asarray(key_padding_mask)
        if km.dtype != np.bool_:
            raise OracleError("arg", "key_padding_mask must be boolean")
        if km.shape == (S,):
            kstride = 0
        elif km.shape == (B, S):
            kstride = S
        else:
            raise OracleError("arg", f"key_padding_mask shape {km.shape} is not ({S},) or ({B}, {S})")
        kpm = np.ascontiguousarray(km, np.uint8)
    out = np.empty((nrows, E), np.float64)
    mixed = np.empty((nrows, E), np.float64) if want_mixed else None
    weights = np.full((B, nnz, H), np.nan, np.float64) if want_weights else None
    rc = lib.oracle_forward(B, L, S, E, H, _ptr(xq), _ptr(xk), _ptr(xv),
                            _ptr(w["wq"]), _ptr(w["bq"]), _ptr(w["wk"]), _ptr(w["bk"]),
                            _ptr(w["wv"]), _ptr(w["bv"]), _ptr(w["wo"]), _ptr(w["bo"]),
                            nnz, _ptr(src), _ptr(tgt), nrows, _ptr(rb), _ptr(rt),
                            _ptr(out), _ptr(mixed), _ptr(weights), _ptr(kpm), int(kstride),
                            int(nthreads))
    if rc != 0:
        raise MemoryError("oracle_forward ran out of memory")
    res = {"out": out if rows is not None else out.reshape(B, L, E)}
    if want_mixed:
        res["mixed"] = mixed if rows is not None else mixed.reshape(B, L, E)
    if want_weights:
        res["weights"] = weights
    return res


def average_heads(weights: np.ndarray) -> np.ndarray:
    """``average_attn_weights=True``: the mean of the per-head weights."""
    return weights.mean(axis=-1)


def case_forward(case, rows=None, want_weights=False, want_mixed=False, nthreads=0,
                 key_padding_mask=None):
    """``forward`` on a synthetic case (validates and appends loops first)."""
    src, tgt = prepare_edges(case.src, case.tgt, case.L, case.S, case.E, case.H,
                             case.add_self_loops)
    params = {k: widen(v, case.dtype) for k, v in case.params.items()}
    xq = widen(case.xq, case.dtype)
    xk = xq if case.xk is case.xq else widen(case.xk, case.dtype)
    xv = xk if case.xv is case.xk else widen(case.xv, case.dtype)
    res = forward(case.B, case.L, case.S, case.E, case.H, xq, xk, xv, params, src, tgt,
                  rows=rows, want_weights=want_weights, want_mixed=want_mixed,
                  nthreads=nthreads, key_padding_mask=key_padding_mask)
    res["src"], res["tgt"] = src, tgt
    return res
