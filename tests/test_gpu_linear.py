"""PackedLinear on the GPU (pma_create_graph, pma_linear_forward,
pma_linear_backward) against the oracle (oracle/linear.py): one trained
scalar per edge on the packed pairs, for single and multi-channel inputs,
both dtypes, split targets and sources, targets without edges, and the
full-size gene and bipartite graphs."""
import numpy as np
import pytest
import torch

import graph_sparse_head_amd as pma
import oracle
from oracle import linear as ol
from graph_sparse_head_amd import synth
from gpu_helpers import TOL, max_abs_rel, to_f64

pytestmark = pytest.mark.gpu


def _round(a, dt):
    a = np.asarray(a, np.float32)
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a)) if dt == "bf16" else a


def _dev(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return t.to(torch.bfloat16) if dt == "bf16" else t


def _check(src, tgt, L, S, B, C, dt, bias=True, loops=False, seed=0, grads=True):
    print(f"[linear] L={L} S={S} B={B} C={C} {dt} bias={bias} loops={loops} nnz0={len(src)}",
          flush=True)
    rng = np.random.default_rng(seed)
    s2, t2 = oracle.prepare_edges(src, tgt, L, S, 1, 1, loops)
    nnz = len(s2)
    x = _round(rng.standard_normal((B, S, C)), dt)
    w = _round(rng.uniform(-1, 1, nnz), dt)
    b = _round(rng.normal(0, 0.5, L), dt) if bias else None
    G = _round(rng.standard_normal((B, L, C)), dt)
    plan = pma.pma_create_graph(src, tgt, L, S, add_self_loops=loops, dtype=dt)
    try:
        assert plan.nnz == nnz
        xd, wd, gd = _dev(x, dt), _dev(w, dt), _dev(G, dt)
        bd = None if b is None else _dev(b, dt)
        y = pma.pma_linear_forward(plan, xd, wd, bd)
        torch.cuda.synchronize()
        ref = ol.forward(x, w, b, s2, t2, L)
        assert max_abs_rel(to_f64(y, dt), ref) <= TOL[dt]
        deg = np.bincount(t2, minlength=L)
        if (deg == 0).any():
            # a target with no edge gets its bias exactly (zero without bias)
            want = np.zeros(L) if b is None else b.astype(np.float64)
            got = to_f64(y, dt)[:, deg == 0, :]
            assert (got == want[deg == 0][None, :, None]).all()
        if grads:
            gx, gw, gb = pma.pma_linear_backward(plan, xd, wd, gd, has_bias=bias)
            torch.cuda.synchronize()
            dx, dw, db = ol.gradients(x, w, s2, t2, L, G)
            assert max_abs_rel(to_f64(gx, dt), dx) <= TOL[dt]
            assert max_abs_rel(to_f64(gw, dt), dw) <= TOL[dt]
            if bias:
                assert max_abs_rel(to_f64(gb, dt), db) <= TOL[dt]
            else:
                assert gb is None
            # a source no edge reads gets a zero gradient
            unread = np.bincount(s2, minlength=S) == 0
            assert (to_f64(gx, dt)[:, unread, :] == 0).all()
    finally:
        pma.pma_destroy(plan)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("C", [1, 3, 8, 16])
@pytest.mark.parametrize("bias", [True, False])
def test_linear_random(dt, C, bias):
    rng = np.random.default_rng(C * 10 + int(bias))
    src, tgt = synth.random_graph(rng, 90, 70, 0.08)
    _check(src, tgt, 90, 70, 5, C, dt, bias=bias, seed=C)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("C", [1, 8])
def test_linear_pieces(dt, C, monkeypatch):
    # PMA_CHUNK / PMA_BWD_CHUNK = 3: most targets and sources are split
    monkeypatch.setenv("PMA_CHUNK", "3")
    monkeypatch.setenv("PMA_BWD_CHUNK", "3")
    rng = np.random.default_rng(31 + C)
    src, tgt = synth.random_graph(rng, 60, 60, 0.2)
    _check(src, tgt, 60, 60, 64, C, dt, seed=C, loops=True)


def test_linear_hub_source_and_target():
    rng = np.random.default_rng(40)
    src, tgt = synth.random_graph(rng, 400, 400, 0.01)
    keep = (src != 5) & (tgt != 9)
    src = np.concatenate([src[keep], np.full(390, 5), np.arange(10, 400)])
    tgt = np.concatenate([tgt[keep], np.arange(10, 400), np.full(390, 9)])
    _check(src, tgt, 400, 400, 64, 1, "f32", seed=41)


@pytest.mark.parametrize("cfg", ["gene", "bipartite"])
def test_linear_full_graph(cfg):
    c = synth.gene() if cfg == "gene" else synth.bipartite()
    _check(c.src, c.tgt, c.L, c.S, c.B, 1, c.dtype, seed=42)


def test_graph_plan_rejects_attention_calls():
    plan = pma.pma_create_graph([0, 1], [1, 0], 2, 2)
    try:
        lib = pma._load()
        z = torch.zeros(64, device="cuda").data_ptr()
        st = lib.pma_forward(plan.handle, 1, z, z, z, z, None, z, None, z, None, z, None, z, None,
                             0, None)
        assert pma.STATUS[st] == "PMA_E_ARG"
        assert lib.pma_train_bytes(plan.handle, 1) == 0
        assert pma.pma_plan_info(plan)["embed_dim"] == 0
    finally:
        pma.pma_destroy(plan)


def test_attention_plan_serves_linear_calls():
    rng = np.random.default_rng(43)
    src, tgt = synth.random_graph(rng, 30, 30, 0.1)
    plan = pma.pma_create(src, tgt, 30, 30, 8, 2)
    try:
        s2, t2 = oracle.prepare_edges(src, tgt, 30, 30, 8, 2, False)
        x = rng.standard_normal((2, 30, 4)).astype(np.float32)
        w = rng.standard_normal(len(s2)).astype(np.float32)
        y = pma.pma_linear_forward(plan, _dev(x, "f32"), _dev(w, "f32"))
        assert max_abs_rel(to_f64(y, "f32"), ol.forward(x, w, None, s2, t2, 30)) <= TOL["f32"]
    finally:
        pma.pma_destroy(plan)
