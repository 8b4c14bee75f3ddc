"""torch.nn.Module surface over the C-ABI (kpnn2 0.3.0 API reference,
PackedMultiheadAttention: constructor parameter table, attributes, "Raises",
reset_parameters and forward; and PackedLinear from its "See also").

Every step of the computation runs in libpma's kernels; this module only
validates arguments, keeps the four projections as nn.Linear parameters,
moves layouts (sequence-first <-> batch-first, leading axes) and hands
pointers to ``pma_forward`` / ``pma_forward_masked``. Plans are built per
(device, dtype) on first use and cached.

Gradients flow through pma_forward_train / pma_backward (a torch.autograd
Function). Not covered: dropout in training mode (the kernels compute the
eval-mode softmax; a training-mode call with dropout > 0 raises), attn_mask
and is_causal (must be None / False, as on the page), checkpoint identity
and index digests.
"""
from __future__ import annotations

import math
import numbers
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

from . import (PmaError, pma_backward, pma_create, pma_create_graph, pma_destroy, pma_edge_list,
               pma_edges, pma_forward, pma_forward_train, pma_linear_backward,
               pma_linear_forward)

__all__ = ["PackedMultiheadAttention", "PackedLinear", "ModuleArgError"]


class ModuleArgError(ValueError):
    """An argument the layer rejects (the page's Kpnn2Error cases)."""


def _is_int(x) -> bool:
    return isinstance(x, (numbers.Integral, np.integer)) and not isinstance(x, (bool, np.bool_))


def _pos_int(x, name: str) -> int:
    if not _is_int(x) or int(x) <= 0:
        raise ModuleArgError(f"{name} must be a positive integer, got {x!r}")
    return int(x)


def _index(x, name: str) -> np.ndarray:
    """1-D integer indices from a tensor, ndarray or sequence (copied)."""
    if isinstance(x, (set, frozenset, dict)):
        raise ModuleArgError(f"{name} must be ordered (a set or mapping is rejected)")
    if isinstance(x, torch.Tensor):
        if x.is_complex() or x.is_floating_point() or x.dtype == torch.bool:
            raise ModuleArgError(f"{name} must be an integer tensor")
        a = x.detach().cpu().numpy()
    else:
        a = np.asarray(x)
        if a.size and (a.dtype == np.bool_ or not np.issubdtype(a.dtype, np.integer)):
            if a.dtype == object and all(_is_int(v) for v in a.ravel()):
                a = a.astype(np.int64)
            else:
                raise ModuleArgError(f"{name} must hold integers")
    if a.ndim != 1:
        raise ModuleArgError(f"{name} must be 1-D")
    return np.array(a, dtype=np.int64, copy=True)


def _bool(x, name: str) -> bool:
    if not isinstance(x, (bool, np.bool_)):
        raise ModuleArgError(f"{name} must be a bool, got {x!r}")
    return bool(x)


def _edges(source_index, target_index, L: int, S: int, add_self_loops: bool):
    """Validated edge arrays in the layer's edge order: the given pairs, then
    the missing (i, i) in ascending i when add_self_loops. The index rules
    (kpnn2 page, constructor parameter table and "Raises") are the library's
    own (pma_edge_list, host only); its rejections surface here as
    ModuleArgError."""
    src = _index(source_index, "source_index")
    tgt = _index(target_index, "target_index")
    try:
        return pma_edge_list(src, tgt, L, S, add_self_loops)
    except PmaError as e:
        raise ModuleArgError(str(e)) from None


def _named_edges(sources: Sequence, targets: Sequence, nodes: Optional[Sequence]):
    """Node order and integer edges from a named edge list: ``nodes`` when
    given, else order of first appearance (sources and targets interleaved
    edge by edge)."""
    if len(sources) != len(targets):
        raise ModuleArgError("sources and targets differ in length")
    order: Dict[object, int] = {}
    if nodes is None:
        for s, t in zip(sources, targets):
            order.setdefault(s, len(order))
            order.setdefault(t, len(order))
    else:
        for n in nodes:
            if n in order:
                raise ModuleArgError(f"node {n!r} listed twice")
            order[n] = len(order)
    try:
        src = [order[s] for s in sources]
        tgt = [order[t] for t in targets]
    except KeyError as e:
        raise ModuleArgError(f"edge endpoint {e.args[0]!r} is not in nodes") from None
    return order, src, tgt


def _plan_dtype(dtype: torch.dtype) -> str:
    if dtype == torch.float32:
        return "f32"
    if dtype == torch.bfloat16:
        return "bf16"
    raise ModuleArgError(f"parameters of dtype {dtype} are not supported (float32, bfloat16)")


class PackedMultiheadAttention(torch.nn.Module):
    """Multi-head attention in which each target token attends only to its
    listed source tokens (kpnn2 page, class docstring and "Notes")."""

    def __init__(self, source_index, target_index, query_features, key_features, embed_dim,
                 num_heads, dropout: float = 0.0, bias: bool = True, kdim=None, vdim=None,
                 batch_first: bool = True, add_self_loops: bool = False, *,
                 generator: Optional[torch.Generator] = None, device=None, dtype=None):
        super().__init__()
        L = _pos_int(query_features, "query_features")
        S = _pos_int(key_features, "key_features")
        E = _pos_int(embed_dim, "embed_dim")
        H = _pos_int(num_heads, "num_heads")
        if E % H:
            raise ModuleArgError(f"embed_dim {E} is not divisible by num_heads {H}")
        if isinstance(dropout, (bool, np.bool_)) or not isinstance(dropout, (numbers.Real, np.floating)):
            raise ModuleArgError(f"dropout must be a number, got {dropout!r}")
        dropout = float(dropout)
        if not math.isfinite(dropout) or not 0.0 <= dropout <= 1.0:
            raise ModuleArgError(f"dropout must lie in [0, 1], got {dropout}")
        bias = _bool(bias, "bias")
        batch_first = _bool(batch_first, "batch_first")
        add_self_loops = _bool(add_self_loops, "add_self_loops")
        for n, v in (("kdim", kdim), ("vdim", vdim)):
            if v is not None and (not _is_int(v) or int(v) != E):
                raise ModuleArgError(f"{n} must be None or equal to embed_dim ({E}), got {v!r}")
        if generator is not None and not isinstance(generator, torch.Generator):
            raise ModuleArgError("generator must be a torch.Generator or None")
        src, tgt = _edges(source_index, target_index, L, S, add_self_loops)

        self.query_features, self.key_features = L, S
        self.embed_dim, self.num_heads, self.head_dim = E, H, E // H
        self.dropout, self.batch_first, self.add_self_loops = dropout, batch_first, add_self_loops
        self.register_buffer("source_index", torch.from_numpy(src), persistent=True)
        self.register_buffer("target_index", torch.from_numpy(tgt), persistent=True)
        kw = {"device": device, "dtype": dtype}
        self.q_proj = torch.nn.Linear(E, E, bias=bias, **kw)
        self.k_proj = torch.nn.Linear(E, E, bias=bias, **kw)
        self.v_proj = torch.nn.Linear(E, E, bias=bias, **kw)
        self.out_proj = torch.nn.Linear(E, E, bias=bias, **kw)
        self._plans: Dict[Tuple[str, int, str], object] = {}
        self.reset_parameters(generator)

    # ------------------------------------------------------------------
    @classmethod
    def from_edgelist(cls, sources: Sequence, targets: Sequence, embed_dim: int, num_heads: int,
                      nodes: Optional[Sequence] = None, **kwargs) -> "PackedMultiheadAttention":
        """Attention within one node set from a named edge list (source ->
        target). Node i of the token sequence is ``nodes[i]``; without
        ``nodes`` the order is that of first appearance, sources and targets
        interleaved edge by edge."""
        order, src, tgt = _named_edges(sources, targets, nodes)
        n = len(order)
        layer = cls(src, tgt, n, n, embed_dim, num_heads, **kwargs)
        layer.nodes = list(order)
        return layer

    @property
    def nnz(self) -> int:
        return int(self.source_index.shape[0])

    def reset_parameters(self, generator: Optional[torch.Generator] = None) -> None:
        """Xavier-uniform projection weights; biases zeroed (kpnn2 page,
        reset_parameters)."""
        with torch.no_grad():
            for lin in (self.q_proj, self.k_proj, self.v_proj, self.out_proj):
                bound = math.sqrt(6.0 / (lin.in_features + lin.out_features))
                w = torch.empty(lin.weight.shape, dtype=torch.float32)
                w.uniform_(-bound, bound, generator=generator)
                lin.weight.copy_(w)
                if lin.bias is not None:
                    lin.bias.zero_()

    # ------------------------------------------------------------------
    def _plan(self, device: torch.device, dtype: torch.dtype):
        dt = _plan_dtype(dtype)
        key = (device.type, device.index if device.index is not None else torch.cuda.current_device(), dt)
        plan = self._plans.get(key)
        if plan is None:
            with torch.cuda.device(key[1]):
                plan = pma_create(self.source_index.cpu().numpy(), self.target_index.cpu().numpy(),
                                  self.query_features, self.key_features, self.embed_dim,
                                  self.num_heads, add_self_loops=False, dtype=dt)
            s, t = pma_edges(plan)
            assert (s == self.source_index.cpu().numpy()).all() and \
                (t == self.target_index.cpu().numpy()).all()
            self._plans[key] = plan
        return plan

    def _drop_plans(self):
        for plan in self._plans.values():
            try:
                pma_destroy(plan)
            except Exception:   # pragma: no cover - interpreter shutdown
                pass
        self._plans = {}

    def __del__(self):
        try:
            self._drop_plans()
        except Exception:   # pragma: no cover
            pass

    def _apply(self, fn, *args, **kwargs):
        # Changing device or dtype invalidates nothing in the plans (they are
        # keyed by device and dtype), but buffers must stay int64.
        out = super()._apply(fn, *args, **kwargs)
        for n in ("source_index", "target_index"):
            b = getattr(self, n)
            if b.dtype != torch.int64:
                setattr(self, n, b.to(torch.int64))
        return out

    # ------------------------------------------------------------------
    def _check_tokens(self, x, name: str, seq: int):
        E = self.embed_dim
        if not isinstance(x, torch.Tensor):
            raise ModuleArgError(f"{name} must be a tensor")
        if not x.is_floating_point():
            raise ModuleArgError(f"{name} must be floating-point, got {x.dtype}")
        if x.dim() < 2:
            raise ModuleArgError(f"{name} needs at least 2 dimensions")
        if x.shape[-1] != E:
            raise ModuleArgError(f"{name} has width {x.shape[-1]}, embed_dim is {E}")
        seq_axis = -2 if (self.batch_first or x.dim() == 2) else 0
        if x.shape[seq_axis] != seq:
            raise ModuleArgError(f"{name} has sequence length {x.shape[seq_axis]}, expected {seq}")
        if not self.batch_first and x.dim() != 2 and x.dim() != 3:
            raise ModuleArgError(f"batched {name} must be 3-D (seq, batch, E) with batch_first=False")

    def forward(self, query, key, value, key_padding_mask=None, need_weights: bool = False,
                attn_mask=None, average_attn_weights: bool = True, is_causal: bool = False):
        """Returns (output in query's layout, weights or None); weights are
        one per live edge in edge order, (..., nnz) averaged or (..., nnz, H)."""
        if attn_mask is not None:
            raise ModuleArgError("attn_mask must be None: the edge list is the mask")
        if is_causal is not False:
            raise ModuleArgError("is_causal must be False")
        need_weights = _bool(need_weights, "need_weights")
        average_attn_weights = _bool(average_attn_weights, "average_attn_weights")
        if self.training and self.dropout > 0:
            raise ModuleArgError("dropout in training mode is not supported; call eval() "
                                 "or set dropout=0")
        L, S, E, H = self.query_features, self.key_features, self.embed_dim, self.num_heads
        self._check_tokens(query, "query", L)
        self._check_tokens(key, "key", S)
        self._check_tokens(value, "value", S)
        if key.shape != value.shape:
            raise ModuleArgError("key and value shapes differ")
        unbatched = query.dim() == 2
        seq_first = not self.batch_first and not unbatched

        def to_bf(x):
            return x.transpose(0, 1) if seq_first else x

        q, k, v = to_bf(query), to_bf(key), to_bf(value)
        lead = tuple(q.shape[:-2])
        if tuple(k.shape[:-2]) != lead or tuple(v.shape[:-2]) != lead:
            raise ModuleArgError("the batch axes of query, key and value differ")
        if key_padding_mask is not None:
            m = key_padding_mask
            if not isinstance(m, torch.Tensor) or m.dtype != torch.bool:
                raise ModuleArgError("key_padding_mask must be a boolean tensor")
            if tuple(m.shape) != (S,) and tuple(m.shape) != lead + (S,):
                raise ModuleArgError(f"key_padding_mask has shape {tuple(m.shape)}, expected "
                                     f"({S},) or {lead + (S,)}")
        w = self.q_proj.weight
        if query.device != w.device or query.device.type != "cuda":
            raise ModuleArgError("query, key, value and the layer must be on the same GPU")
        dt = w.dtype
        plan = self._plan(w.device, dt)

        def prep(x):
            return x.to(dt).contiguous()

        same_kv = key is value
        same_qkv = query is key and same_kv
        qc = prep(q)
        kc = qc if same_qkv else prep(k)
        vc = kc if same_kv else prep(v)
        mask = None if key_padding_mask is None else key_padding_mask.to(device=qc.device).contiguous()
        if torch.is_grad_enabled() and (q.requires_grad or k.requires_grad or v.requires_grad or
                                        any(p.requires_grad for p in self.parameters())):
            out, weights = _PackedAttnFn.apply(plan, qc, kc, vc, mask, need_weights,
                                               average_attn_weights, same_qkv, same_kv,
                                               *self._params())
        else:
            out, weights = self._run(plan, qc, kc, vc, mask, need_weights, average_attn_weights)
        return self._finish(out, weights, seq_first, lead)

    def _params(self):
        ps = []
        for lin in (self.q_proj, self.k_proj, self.v_proj, self.out_proj):
            ps += [lin.weight, lin.bias]
        return ps

    def _run(self, plan, qc, kc, vc, mask, need_weights, average):
        def c(t):
            return None if t is None else t.detach().contiguous()
        return pma_forward(plan, qc.detach(), kc.detach(), vc.detach(),
                           c(self.q_proj.weight), c(self.q_proj.bias),
                           c(self.k_proj.weight), c(self.k_proj.bias),
                           c(self.v_proj.weight), c(self.v_proj.bias),
                           c(self.out_proj.weight), c(self.out_proj.bias),
                           need_weights=need_weights, average_attn_weights=average,
                           key_padding_mask=mask)

    @staticmethod
    def _finish(out, weights, seq_first, lead):
        if seq_first:
            out = out.transpose(0, 1)
            if weights is not None:
                weights = weights.transpose(0, 1)   # (nnz, batch[, H])
        return out, weights


class _PackedAttnFn(torch.autograd.Function):
    """Forward through pma_forward_train (which keeps what the backward
    needs in a save area), backward through pma_backward."""

    @staticmethod
    def forward(ctx, plan, q, k, v, mask, need_weights, average, same_qkv, same_kv,
                q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b):
        def c(t):
            return None if t is None else t.detach().contiguous()
        ws = [c(t) for t in (q_w, q_b, k_w, k_b, v_w, v_b, o_w, o_b)]
        out, weights, save = pma_forward_train(plan, q, k, v, *ws, need_weights=need_weights,
                                               average_attn_weights=average,
                                               key_padding_mask=mask)
        ctx.plan = plan
        ctx.has_bias = q_b is not None
        ctx.same = (same_qkv, same_kv)
        ctx.mask = mask
        ctx.save_for_backward(q, k, v, save, ws[0], ws[2], ws[4], ws[6])
        if weights is not None:
            ctx.mark_non_differentiable(weights)
        return out, weights

    @staticmethod
    def backward(ctx, grad_out, grad_weights):
        q, k, v, save, q_w, k_w, v_w, o_w = ctx.saved_tensors
        same_qkv, same_kv = ctx.same
        # the forward received one tensor object per shared role; the
        # gradient of a shared tensor is returned once (autograd sums per use)
        kk = q if same_qkv else k
        vv = kk if (same_qkv or same_kv) else v
        g = pma_backward(ctx.plan, q, kk, vv, q_w, k_w, v_w, o_w, ctx.has_bias, save,
                         grad_out.contiguous(), key_padding_mask=ctx.mask)
        gq = g["query"]
        gk = None if same_qkv else g["key"]
        gv = None if (same_qkv or same_kv) else g["value"]
        gb = [g.get(n) for n in ("q_b", "k_b", "v_b", "o_b")]
        return (None, gq, gk, gv, None, None, None, None, None,
                g["q_w"], gb[0], g["k_w"], gb[1], g["v_w"], gb[2], g["o_w"], gb[3])


class PackedLinear(torch.nn.Module):
    """One trained scalar per edge on the packed pairs (kpnn2
    PackedMultiheadAttention page, "See also": PackedLinear; information flows
    from source to target). Input (..., in_features) -> output
    (..., out_features) with

        out[..., t] = bias[t] + sum over edges e into t of weight[e] input[..., s_e],

    weight in the layer's edge order (given pairs, then appended loops).
    The product and its gradients run in libpma (pma_linear_forward /
    pma_linear_backward)."""

    def __init__(self, source_index, target_index, in_features, out_features, bias: bool = True,
                 add_self_loops: bool = False, *, generator: Optional[torch.Generator] = None,
                 device=None, dtype=None):
        super().__init__()
        S = _pos_int(in_features, "in_features")
        L = _pos_int(out_features, "out_features")
        bias = _bool(bias, "bias")
        add_self_loops = _bool(add_self_loops, "add_self_loops")
        if generator is not None and not isinstance(generator, torch.Generator):
            raise ModuleArgError("generator must be a torch.Generator or None")
        src, tgt = _edges(source_index, target_index, L, S, add_self_loops)
        self.in_features, self.out_features, self.add_self_loops = S, L, add_self_loops
        self.register_buffer("source_index", torch.from_numpy(src), persistent=True)
        self.register_buffer("target_index", torch.from_numpy(tgt), persistent=True)
        kw = {"device": device, "dtype": dtype}
        self.weight = torch.nn.Parameter(torch.empty(src.shape[0], **kw))
        if bias:
            self.bias = torch.nn.Parameter(torch.empty(L, **kw))
        else:
            self.register_parameter("bias", None)
        self._plans: Dict[Tuple[str, int, str], object] = {}
        self.reset_parameters(generator)

    @classmethod
    def from_edgelist(cls, sources: Sequence, targets: Sequence, nodes: Optional[Sequence] = None,
                      **kwargs) -> "PackedLinear":
        """A layer over one node set from a named edge list (source -> target),
        node order as for PackedMultiheadAttention.from_edgelist."""
        order, src, tgt = _named_edges(sources, targets, nodes)
        n = len(order)
        layer = cls(src, tgt, n, n, **kwargs)
        layer.nodes = list(order)
        return layer

    @property
    def nnz(self) -> int:
        return int(self.source_index.shape[0])

    def reset_parameters(self, generator: Optional[torch.Generator] = None) -> None:
        """nn.Linear's default draw with each target's in-degree as its fan-in:
        weight[e] and bias[t] uniform in +-1 / sqrt(in-degree of t) (zero
        bias for a target with no edge)."""
        deg = np.bincount(self.target_index.cpu().numpy(), minlength=self.out_features)
        bt = torch.from_numpy(np.where(deg > 0, 1.0 / np.sqrt(np.maximum(deg, 1)), 0.0))
        with torch.no_grad():
            u = torch.rand(self.nnz, dtype=torch.float64, generator=generator)
            self.weight.copy_((2 * u - 1) * bt[self.target_index.cpu()])
            if self.bias is not None:
                u = torch.rand(self.out_features, dtype=torch.float64, generator=generator)
                self.bias.copy_((2 * u - 1) * bt)

    def _plan(self, device: torch.device, dtype: torch.dtype):
        dt = _plan_dtype(dtype)
        key = (device.type, device.index if device.index is not None else torch.cuda.current_device(), dt)
        plan = self._plans.get(key)
        if plan is None:
            with torch.cuda.device(key[1]):
                plan = pma_create_graph(self.source_index.cpu().numpy(),
                                        self.target_index.cpu().numpy(), self.out_features,
                                        self.in_features, add_self_loops=False, dtype=dt)
            s, t = pma_edges(plan)
            assert (s == self.source_index.cpu().numpy()).all() and \
                (t == self.target_index.cpu().numpy()).all()
            self._plans[key] = plan
        return plan

    def __del__(self):
        try:
            for plan in self._plans.values():
                pma_destroy(plan)
            self._plans = {}
        except Exception:   # pragma: no cover
            pass

    def _apply(self, fn, *args, **kwargs):
        out = super()._apply(fn, *args, **kwargs)
        for n in ("source_index", "target_index"):
            b = getattr(self, n)
            if b.dtype != torch.int64:
                setattr(self, n, b.to(torch.int64))
        return out

    def forward(self, input):
        if not isinstance(input, torch.Tensor) or not input.is_floating_point():
            raise ModuleArgError("input must be a floating-point tensor")
        if input.dim() < 1 or input.shape[-1] != self.in_features:
            raise ModuleArgError(f"input has width {input.shape[-1] if input.dim() else None}, "
                                 f"in_features is {self.in_features}")
        w = self.weight
        if input.device != w.device or input.device.type != "cuda":
            raise ModuleArgError("input and the layer must be on the same GPU")
        plan = self._plan(w.device, w.dtype)
        lead = tuple(input.shape[:-1])
        x = input.to(w.dtype).reshape(-1, self.in_features, 1).contiguous()
        if torch.is_grad_enabled() and (x.requires_grad or w.requires_grad or
                                        (self.bias is not None and self.bias.requires_grad)):
            y = _PackedLinearFn.apply(plan, x, w, self.bias)
        else:
            b = None if self.bias is None else self.bias.detach().contiguous()
            y = pma_linear_forward(plan, x.detach(), w.detach().contiguous(), b)
        return y.reshape(lead + (self.out_features,))


class _PackedLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, plan, x, weight, bias):
        w = weight.detach().contiguous()
        b = None if bias is None else bias.detach().contiguous()
        ctx.plan, ctx.has_bias = plan, bias is not None
        ctx.save_for_backward(x.detach(), w)
        return pma_linear_forward(plan, x.detach(), w, b)

    @staticmethod
    def backward(ctx, grad_out):
        x, w = ctx.saved_tensors
        gx, gw, gb = pma_linear_backward(ctx.plan, x, w, grad_out.contiguous(),
                                         has_bias=ctx.has_bias)
        return None, gx, gw, gb
