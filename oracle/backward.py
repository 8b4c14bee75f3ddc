"""Gradients of packed multi-head attention over live edges, in float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): only the tests, the smoke
check and the bench's CPU-baseline leg use it. It shares no code with the GPU
library.

The forward below is written from the kpnn2 PackedMultiheadAttention page,
"Notes" steps 1-5 (and key_padding_mask, forward parameter table), with
plain torch CPU float64 operations: gather the query row of each edge's
target and the key / value rows of its source, score, softmax over the edges
into each target (segment maximum and sum by index), mix by index-add, join
heads, out_proj. torch.autograd differentiates it; the gradient of a
function is the definition here, and the pins in tests/test_oracle_backward.py
tie it to finite differences of the C oracle and to torch's own
nn.MultiheadAttention.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch


def _t(a):
    return torch.as_tensor(np.ascontiguousarray(a, np.float64))


def forward_torch(E: int, H: int, xq, xk, xv, params: Dict[str, Optional[torch.Tensor]], src, tgt,
                  key_padding_mask=None, L: Optional[int] = None):
    """xq (B, L, E), xk / xv (B, S, E) float64 tensors; params torch float64
    (wq bq wk bk wv bv wo bo; biases may be None); src / tgt int64 edge
    lists. Returns out (B, L, E) and per-head weights (B, nnz, H)."""
    B, Lq, _ = xq.shape
    L = Lq if L is None else L
    d = E // H
    src = torch.as_tensor(np.asarray(src), dtype=torch.int64)
    tgt = torch.as_tensor(np.asarray(tgt), dtype=torch.int64)
    nnz = src.shape[0]

    def lin(x, w, b):
        y = x @ w.T
        return y if b is None else y + b

    # step 1: projections, split into H slices of d channels
    q = lin(xq, params["wq"], params["bq"]).reshape(B, L, H, d)
    k = lin(xk, params["wk"], params["bk"]).reshape(B, -1, H, d)
    v = lin(xv, params["wv"], params["bv"]).reshape(B, -1, H, d)
    # step 2: one score per live edge and head
    score = (q[:, tgt] * k[:, src]).sum(-1) / math.sqrt(d)          # (B, nnz, H)
    live = torch.ones(B, nnz, dtype=torch.bool)
    if key_padding_mask is not None:
        km = torch.as_tensor(np.asarray(key_padding_mask, dtype=bool))
        km = km.expand(B, km.shape[-1]) if km.dim() == 1 else km
        live = ~km[:, src]
    score = score.masked_fill(~live[..., None], -math.inf)
    # step 3: softmax over the edges into each target (segment max and sum)
    idx = tgt[None, :, None].expand(B, nnz, H)
    mx = torch.full((B, L, H), -math.inf, dtype=torch.float64)
    mx = mx.scatter_reduce(1, idx, score, reduce="amax", include_self=True)
    shifted = score - mx.gather(1, idx).detach()
    ex = torch.where(live[..., None], torch.exp(torch.where(live[..., None], shifted,
                                                            torch.zeros_like(shifted))),
                     torch.zeros_like(shifted))
    den = torch.zeros(B, L, H, dtype=torch.float64).index_add(1, tgt, ex)
    den_e = den.gather(1, idx)
    w = torch.where(den_e > 0, ex / torch.where(den_e > 0, den_e, torch.ones_like(den_e)),
                    torch.zeros_like(ex))
    # step 4: mix the sources' values into each target (zeros with no live edge)
    contrib = w[..., None] * v[:, src]                                 # (B, nnz, H, d)
    mixed = torch.zeros(B, L, H, d, dtype=torch.float64).index_add(1, tgt, contrib)
    # step 5: join heads, out_proj
    out = lin(mixed.reshape(B, L, E), params["wo"], params["bo"])
    return out, w


def gradients(B: int, L: int, S: int, E: int, H: int, xq, xk, xv, params, src, tgt, grad_out,
              key_padding_mask=None, shared: str = "none"):
    """Gradients of sum(out * grad_out) with respect to the tokens and the
    eight projection parameters, float64 numpy.

    shared: "none" (query, key, value separate tensors), "kv" (key is value)
    or "qkv" (one tensor for all three): a shared tensor gets the sum of its
    uses' gradients, returned under each of its names."""
    P = {k: (None if v is None else _t(v).requires_grad_(True)) for k, v in params.items()}
    xq_t = _t(xq).requires_grad_(True)
    xk_t = xq_t if shared == "qkv" else _t(xk).requires_grad_(True)
    xv_t = xk_t if shared in ("kv", "qkv") else _t(xv).requires_grad_(True)
    out, _ = forward_torch(E, H, xq_t, xk_t, xv_t, P, src, tgt, key_padding_mask, L)
    leaves = {"query": xq_t, "key": xk_t, "value": xv_t}
    leaves.update({k: v for k, v in P.items() if v is not None})
    names = list(leaves)
    uniq, seen = [], {}
    for n in names:
        if id(leaves[n]) not in seen:
            seen[id(leaves[n])] = len(uniq)
            uniq.append(leaves[n])
    g = torch.autograd.grad((out * _t(grad_out)).sum(), uniq, allow_unused=True)
    res = {}
    for n in names:
        gi = g[seen[id(leaves[n])]]
        res[n] = (torch.zeros_like(leaves[n]) if gi is None else gi).detach().numpy()
    return res
