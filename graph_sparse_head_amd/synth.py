"""Seeded synthetic inputs for packed multi-head attention over live edges.

This module draws graphs, tokens and parameters. It holds none of the
method's arithmetic: no projection, score, softmax or mix happens here. Both
the CPU oracle (through the tests) and the GPU path consume what it returns.

The shapes and distributions follow the workloads motivated on the kpnn2
``PackedMultiheadAttention`` page (class docstring: gene-regulatory priors of
about 20,000 nodes, bipartite pathway -> gene maps). Real priors are not
available, so seeded synthetic graphs of the same shape stand in for them.

Storage convention: fp32 arrays are ``float32``; bf16 arrays are ``uint16``
bit patterns, rounded to nearest-even from the fp32 draw.

Seeds: graph 0, tokens 1, parameters 2 (numpy PCG64 ``default_rng``), unless a
caller passes others.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Case", "f32_to_bf16_bits", "bf16_bits_to_f32", "tiny", "complete",
    "gene", "bipartite", "large", "worked_example", "random_graph", "CONFIGS",
    "make_config",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns. Finite inputs only (the generators draw
    finite values).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Case:
    """One workload: a graph, a batch of tokens and the four projections."""

    name: str
    B: int
    L: int
    S: int
    E: int
    H: int
    dtype: str                      # "f32" or "bf16"
    src: np.ndarray                 # int64 (nnz0,), given pairs (no appended loops)
    tgt: np.ndarray                 # int64 (nnz0,)
    add_self_loops: bool
    need_weights: bool
    average: bool
    xq: np.ndarray                  # (B, L, E) float32 or uint16 bits
    xk: np.ndarray                  # (B, S, E)
    xv: np.ndarray                  # (B, S, E); may be the same object as xk / xq
    params: Dict[str, Optional[np.ndarray]]  # wq bq wk bk wv bv wo bo ([out][in] weights)
    note: str = ""

    @property
    def nnz0(self) -> int:
        return int(self.src.shape[0])


# --------------------------------------------------------------------------
# small helpers


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _params(rng: np.random.Generator, E: int, dtype: str, w_bound: float,
            bias: str) -> Dict[str, Optional[np.ndarray]]:
    """Four (E, E) weights U(-w_bound, w_bound) and biases.

    bias: "normal" -> N(0, 0.02); "zero" -> zeros; "none" -> no bias arrays.
    """
    out: Dict[str, Optional[np.ndarray]] = {}
    for name in ("q", "k", "v", "o"):
        w = rng.uniform(-w_bound, w_bound, size=(E, E)).astype(np.float32)
        if bias == "normal":
            b = rng.normal(0.0, 0.02, size=(E,)).astype(np.float32)
        elif bias == "zero":
            b = np.zeros((E,), np.float32)
        else:
            b = None
        out["w" + name] = _store(w, dtype)
        out["b" + name] = None if b is None else _store(b, dtype)
    return out


def _xavier_bound(E: int) -> float:
    # Xavier-uniform for a square (E, E) map: sqrt(6 / (fan_in + fan_out)).
    return math.sqrt(6.0 / (2 * E))


def _tokens(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return _store(rng.standard_normal(size=shape, dtype=np.float32), dtype)


def _distinct_weighted(rng: np.random.Generator, deg: np.ndarray, node_of_rank: np.ndarray,
                       cdf: np.ndarray, allow_self: bool):
    """Draw deg[t] distinct sources for every target t.

    Sources are drawn one after another from the popularity distribution given
    by ``cdf`` over ranks (``node_of_rank`` maps a rank to a node id); a repeat
    of an already chosen source, or the target itself when ``allow_self`` is
    False, is discarded and redrawn. Draws are made in vectorised rounds.

    Returns (src, tgt) int64, grouped by ascending target, each target's
    sources in draw order.
    """
    n_t = deg.shape[0]
    deg = deg.astype(np.int64)
    need = deg.copy()
    ts = np.empty(0, np.int64)
    ss = np.empty(0, np.int64)
    qs = np.empty(0, np.int64)
    seq0 = 0
    factor = 2
    for _ in range(200):
        act = np.nonzero(need > 0)[0]
        if act.size == 0:
            break
        m = need[act] * factor + 8
        tt = np.repeat(act, m)
        u = rng.random(tt.shape[0])
        rank = np.minimum(np.searchsorted(cdf, u, side="right"), cdf.shape[0] - 1)
        sn = node_of_rank[rank]
        qq = seq0 + np.arange(tt.shape[0], dtype=np.int64)
        seq0 += tt.shape[0]
        if not allow_self:
            keep = sn != tt
            tt, sn, qq = tt[keep], sn[keep], qq[keep]
        # keep the entries of the still-active targets plus the new draws
        old_act = need[ts] > 0
        done_t, done_s, done_q = ts[~old_act], ss[~old_act], qs[~old_act]
        at = np.concatenate([ts[old_act], tt])
        as_ = np.concatenate([ss[old_act], sn])
        aq = np.concatenate([qs[old_act], qq])
        # first draw of each (target, source) pair
        o = np.lexsort((aq, as_, at))
        at, as_, aq = at[o], as_[o], aq[o]
        first = np.ones(at.shape[0], bool)
        first[1:] = (at[1:] != at[:-1]) | (as_[1:] != as_[:-1])
        at, as_, aq = at[first], as_[first], aq[first]
        # per target, keep the first deg[t] distinct sources in draw order
        o = np.lexsort((aq, at))
        at, as_, aq = at[o], as_[o], aq[o]
        start = np.searchsorted(at, at, side="left")
        rank_in_t = np.arange(at.shape[0]) - start
        keep = rank_in_t < deg[at]
        at, as_, aq = at[keep], as_[keep], aq[keep]
        ts = np.concatenate([done_t, at])
        ss = np.concatenate([done_s, as_])
        qs = np.concatenate([done_q, aq])
        cnt = np.bincount(ts, minlength=n_t)
        need = deg - cnt
        factor = min(factor * 2, 64)
    else:  # pragma: no cover - the loop always finishes for feasible degrees
        raise RuntimeError("source sampling did not converge")
    o = np.lexsort((qs, ts))
    return ss[o].astype(np.int64), ts[o].astype(np.int64)


def _zipf_cdf(n: int, s: float) -> np.ndarray:
    p = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(p)
    return c / c[-1]


# --------------------------------------------------------------------------
# the workloads


def tiny(seed_graph=0, seed_tok=1, seed_par=2) -> Case:
    """n = 8, B = 2, E = 8, H = 2, fp32. Each target gets 0..4 distinct
    sources chosen uniformly (self allowed); the pairs are listed shuffled.
    Weights U(-1/sqrt(8), 1/sqrt(8)), biases N(0, 0.02); need_weights."""
    n, B, E, H = 8, 2, 8, 2
    g = np.random.default_rng(seed_graph)
    src, tgt = [], []
    for t in range(n):
        d = int(g.integers(0, 5))
        for s in g.choice(n, size=d, replace=False):
            src.append(int(s))
            tgt.append(t)
    src = np.array(src, np.int64)
    tgt = np.array(tgt, np.int64)
    perm = g.permutation(src.shape[0])
    src, tgt = src[perm], tgt[perm]
    x = _tokens(np.random.default_rng(seed_tok), (B, n, E), "f32")
    params = _params(np.random.default_rng(seed_par), E, "f32", 1.0 / math.sqrt(8.0), "normal")
    return Case("tiny", B, n, n, E, H, "f32", src, tgt, False, True, True, x, x, x, params)


def complete(bias: str = "normal", seed_graph=0, seed_tok=1, seed_par=2) -> Case:
    """n = 64, every node sources every node including itself (nnz = 4096),
    pairs shuffled; B = 4, E = 64, H = 4, fp32, Xavier-uniform weights.
    bias "normal" draws N(0, 0.02), "zero" zeros."""
    n, B, E, H = 64, 4, 64, 4
    g = np.random.default_rng(seed_graph)
    s, t = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    src, tgt = s.ravel().astype(np.int64), t.ravel().astype(np.int64)
    perm = g.permutation(src.shape[0])
    src, tgt = src[perm], tgt[perm]
    x = _tokens(np.random.default_rng(seed_tok), (B, n, E), "f32")
    params = _params(np.random.default_rng(seed_par), E, "f32", _xavier_bound(E), bias)
    return Case("complete", B, n, n, E, H, "f32", src, tgt, False, False, True, x, x, x, params)


def gene(n: int = 20000, B: int = 32, E: int = 64, H: int = 4, dtype: str = "bf16",
         max_deg: int = 1000, seed_graph=0, seed_tok=1, seed_par=2) -> Case:
    """Gene-regulatory prior. In-degree min(max_deg, round(LogNormal(1.243,
    1.456))) (mean 10, about 9% of targets without an incoming edge); sources
    drawn distinct and different from the target with Zipf(1.5) popularity
    over a seeded ranking of the nodes. Tokens N(0, 1), Xavier weights, biases
    N(0, 0.02), all in ``dtype``. The same tokens serve as query, key and value."""
    g = np.random.default_rng(seed_graph)
    deg = np.minimum(max_deg, np.rint(g.lognormal(1.243, 1.456, size=n))).astype(np.int64)
    deg = np.minimum(deg, n - 1)
    node_of_rank = g.permutation(n).astype(np.int64)
    src, tgt = _distinct_weighted(g, deg, node_of_rank, _zipf_cdf(n, 1.5), allow_self=False)
    x = _tokens(np.random.default_rng(seed_tok), (B, n, E), dtype)
    params = _params(np.random.default_rng(seed_par), E, dtype, _xavier_bound(E), "normal")
    return Case("gene", B, n, n, E, H, dtype, src, tgt, False, False, True, x, x, x, params)


def bipartite(L: int = 2000, S: int = 20000, B: int = 16, E: int = 128, H: int = 8,
              dtype: str = "f32", lo: int = 5, hi: int = 500,
              seed_graph=0, seed_tok=1, seed_par=2) -> Case:
    """Bipartite pathway -> gene map. Pathway p has round(exp(U(ln lo, ln hi)))
    member genes chosen uniformly without replacement; each member is an edge
    gene -> pathway. Query tokens (B, L, E), key = value tokens (B, S, E)."""
    g = np.random.default_rng(seed_graph)
    m = np.rint(np.exp(g.uniform(math.log(lo), math.log(hi), size=L))).astype(np.int64)
    m = np.clip(m, lo, min(hi, S))
    src = np.concatenate([g.choice(S, size=int(k), replace=False) for k in m]).astype(np.int64)
    tgt = np.repeat(np.arange(L, dtype=np.int64), m)
    rt = np.random.default_rng(seed_tok)
    xq = _tokens(rt, (B, L, E), dtype)
    xkv = _tokens(rt, (B, S, E), dtype)
    params = _params(np.random.default_rng(seed_par), E, dtype, _xavier_bound(E), "normal")
    return Case("bipartite", B, L, S, E, H, dtype, src, tgt, False, True, True,
                xq, xkv, xkv, params)


def large(n: int = 100000, nnz0: int = 5_000_000, B: int = 8, E: int = 128, H: int = 8,
          dtype: str = "bf16", seed_graph=0, seed_tok=1, seed_par=2) -> Case:
    """Large graph. In-degree proportional to r**-0.5 over a seeded ranking of
    the targets, rounded by largest remainder to sum to nnz0; sources distinct
    with Zipf(1.2) popularity (self allowed, so some loops exist already);
    add_self_loops appends the rest."""
    g = np.random.default_rng(seed_graph)
    w = np.arange(1, n + 1, dtype=np.float64) ** -0.5
    share = w / w.sum() * nnz0
    d = np.floor(share).astype(np.int64)
    rem = nnz0 - int(d.sum())
    if rem > 0:
        order = np.argsort(-(share - d), kind="stable")
        d[order[:rem]] += 1
    d = np.minimum(d, n)
    target_of_rank = g.permutation(n).astype(np.int64)
    deg = np.empty(n, np.int64)
    deg[target_of_rank] = d
    node_of_rank = g.permutation(n).astype(np.int64)
    src, tgt = _distinct_weighted(g, deg, node_of_rank, _zipf_cdf(n, 1.2), allow_self=True)
    x = _tokens(np.random.default_rng(seed_tok), (B, n, E), dtype)
    params = _params(np.random.default_rng(seed_par), E, dtype, _xavier_bound(E), "normal")
    return Case("large", B, n, n, E, H, dtype, src, tgt, True, False, True, x, x, x, params)


def worked_example(B: int = 2, add_self_loops: bool = True, seed_tok=1, seed_par=2) -> Case:
    """The four-node example of the kpnn2 page (Examples): x feeds a two-node
    loop a <-> b, which feeds y. Nodes indexed a=0, b=1, x=2, y=3; edges listed
    a->b, a->y, b->a, x->a; E = 8, H = 2."""
    src = np.array([0, 0, 1, 2], np.int64)
    tgt = np.array([1, 3, 0, 0], np.int64)
    E, H, n = 8, 2, 4
    x = _tokens(np.random.default_rng(seed_tok), (B, n, E), "f32")
    params = _params(np.random.default_rng(seed_par), E, "f32", _xavier_bound(E), "normal")
    return Case("worked_example", B, n, n, E, H, "f32", src, tgt, add_self_loops, True, True,
                x, x, x, params)


def random_graph(rng: np.random.Generator, L: int, S: int, p: float, *,
                 shuffle: bool = True) -> tuple:
    """Every (s, t) pair independently with probability p; pairs shuffled."""
    mask = rng.random((S, L)) < p
    s, t = np.nonzero(mask)
    src, tgt = s.astype(np.int64), t.astype(np.int64)
    if shuffle:
        perm = rng.permutation(src.shape[0])
        src, tgt = src[perm], tgt[perm]
    return src, tgt


def random_case(seed: int, B: int, L: int, S: int, E: int, H: int, p: float,
                dtype: str = "f32", bias: str = "normal", same_kv: bool = True,
                same_qkv: Optional[bool] = None, add_self_loops: bool = False,
                name: str = "random") -> Case:
    """A random graph with Bernoulli(p) pairs and N(0, 1) tokens."""
    g = np.random.default_rng(seed)
    src, tgt = random_graph(g, L, S, p)
    if same_qkv is None:
        same_qkv = (L == S) and same_kv
    xq = _tokens(g, (B, L, E), dtype)
    if same_qkv:
        xk = xv = xq
    else:
        xk = _tokens(g, (B, S, E), dtype)
        xv = xk if same_kv else _tokens(g, (B, S, E), dtype)
    params = _params(g, E, dtype, _xavier_bound(E), bias)
    return Case(name, B, L, S, E, H, dtype, src, tgt, add_self_loops, True, True,
                xq, xk, xv, params)


def wide(seed: int, dtype: str, B: int, E: int, H: int, L: int, S: int, deg: int,
         hub: int, need_weights: bool = True, name: str = "wide") -> Case:
    """Few targets over many sources, so that the key / value rows of the
    batch pass 2 GiB: every target has ``deg`` distinct uniform sources, except
    targets 0 and 1 (``hub`` each), every 97th from 3 (none) and every 89th
    from 5 (one). Query tokens distinct from key = value tokens."""
    g = np.random.default_rng(seed)
    src, tgt = [], []
    for t in range(L):
        d = hub if t < 2 else 0 if t % 97 == 3 else 1 if t % 89 == 5 else deg
        src.append(g.choice(S, size=d, replace=False))
        tgt.append(np.full(d, t, np.int64))
    src = np.concatenate(src).astype(np.int64)
    tgt = np.concatenate(tgt)
    perm = g.permutation(src.shape[0])
    xq = _tokens(g, (B, L, E), dtype)
    xk = _tokens(g, (B, S, E), dtype)
    params = _params(g, E, dtype, _xavier_bound(E), "normal")
    return Case(name, B, L, S, E, H, dtype, src[perm], tgt[perm], False, need_weights, True,
                xq, xk, xk, params)


CONFIGS = ("tiny", "complete", "gene", "bipartite", "large")


def make_config(name: str) -> Case:
    """The five named workloads at their full sizes."""
    return {"tiny": tiny, "complete": complete, "gene": gene, "bipartite": bipartite,
            "large": large}[name]()


def to_torch(case: Case, device: str = "cuda") -> Dict[str, object]:
    """Move a case's tokens and parameters to ``device`` as torch tensors of
    its dtype (bf16 bit patterns are reinterpreted, not converted). Tensors
    that were one array stay one tensor."""
    import torch

    def conv(a):
        if a is None:
            return None
        if case.dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return t.to(device)

    out: Dict[str, object] = {}
    out["xq"] = conv(case.xq)
    out["xk"] = out["xq"] if case.xk is case.xq else conv(case.xk)
    out["xv"] = out["xk"] if case.xv is case.xk else conv(case.xv)
    for k, v in case.params.items():
        out[k] = conv(v)
    return out
