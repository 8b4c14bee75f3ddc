"""Tensors past 2 GiB. Once any tensor the edge kernels address reaches
2 GiB (here the key / value rows of the batch) they switch from 32-bit to
64-bit offsets: the q projection, out_proj, the merge of split targets and the
per-edge weights then run in those variants. Checked against the oracle on
sampled (sample, target) rows that include two split hub targets,
zero-degree targets and lone edges, for outputs and per-edge weights; and
the backward at the same sizes (its save area and key / value gradients past
2 GiB) against the gradient oracle."""
import functools

import numpy as np
import pytest
import torch

import graph_sparse_head_amd as pma
import oracle
from oracle import backward as ob
from graph_sparse_head_amd import synth
from gpu_helpers import TOL, max_abs_rel, record, run, to_f64

pytestmark = pytest.mark.gpu

# (dtype, B, E, H, L, S, deg, hub): bf16 at embed_dim 64 (q projection and
# out_proj inside the edge kernel), fp32 at 128 (separate launches)
WIDE = [("bf16", 64, 64, 4, 3000, 150_000, 200, 6000),
        ("f32", 32, 128, 8, 3000, 75_000, 100, 3000)]


def _rows(c, deg, rng):
    """Sampled (sample, target) rows: both hubs, zero-degree and one-edge
    targets, random others; the first, last and random samples."""
    t = np.concatenate([[0, 1], np.flatnonzero(deg == 0)[:4], np.flatnonzero(deg == 1)[:4],
                        rng.choice(c.L, size=40, replace=False)])
    b = np.unique(np.concatenate([[0, c.B - 1], rng.choice(c.B, size=4, replace=False)]))
    return np.array([(bb, tt) for bb in b for tt in np.unique(t)], np.int64)


@functools.lru_cache(maxsize=2)
def _case(spec):
    dt, B, E, H, L, S, d, hub = spec
    return synth.wide(71, dt, B, E, H, L, S, d, hub)     # ~15 s of token generation


@pytest.mark.parametrize("spec,need_weights", [(s, w) for s in WIDE for w in (False, True)],
                         ids=lambda v: (f"{v[0]}_E{v[2]}_B{v[1]}_S{v[5]}" if isinstance(v, tuple)
                                        else ("weights" if v else "out")))
def test_past_2gib(spec, need_weights):
    dt, B, E, H, L, S, d, hub = spec
    c = _case(spec)
    print(f"[wide] {dt} B={B} E={E} H={H} L={L} S={S} nnz={c.nnz0} w={need_weights}",
          flush=True)
    out, w, plan = run(c, need_weights=need_weights, average=True)
    try:
        info = pma.pma_plan_info(plan)
        src, tgt = pma.pma_edges(plan)
    finally:
        pma.pma_destroy(plan)
    es = 2 if dt == "bf16" else 4
    assert info["kv_rows"] * 2 * B * E * es >= 1 << 31      # past 2 GiB: 64-bit offsets
    assert info["n_split"] >= 2                             # both hubs split
    deg = np.bincount(tgt, minlength=L)
    rows = _rows(c, deg, np.random.default_rng(72))
    ref = oracle.case_forward(c, rows=rows, want_weights=need_weights)
    assert (ref["src"] == src).all() and (ref["tgt"] == tgt).all()
    got = out[rows[:, 0], rows[:, 1]]
    err = max_abs_rel(got, ref["out"])
    record(f"wide {dt}", "out (sampled rows)", err, TOL[dt])
    assert err <= TOL[dt], err
    bo = oracle.widen(c.params["bo"], dt)
    assert (out[:, deg == 0] == bo).all()
    if need_weights:
        rw = oracle.average_heads(ref["weights"])
        m = ~np.isnan(rw)
        assert m.sum() > 0
        werr = max_abs_rel(w[m], rw[m])
        record(f"wide {dt}", "weights (sampled rows)", werr, TOL[dt])
        assert werr <= TOL[dt], werr
        assert (w[:, deg[tgt] == 1] == 1.0).all()
        sums = np.stack([np.bincount(tgt, weights=w[b], minlength=L) for b in range(B)])
        assert np.abs(sums[:, deg > 0] - 1).max() <= TOL[dt]


NAMES = {"query": None, "key": None, "q_w": "wq", "k_w": "wk", "v_w": "wv", "o_w": "wo",
         "q_b": "bq", "v_b": "bv", "o_b": "bo"}


@pytest.mark.parametrize("spec", WIDE, ids=lambda s: f"{s[0]}_E{s[2]}_B{s[1]}_S{s[5]}")
def test_past_2gib_backward(spec):
    """The upstream gradient is zero except at the first and the last sample,
    so every parameter gradient is those two samples' contribution and every
    other sample's token gradients are exactly zero: the oracle runs on the
    two samples alone while the GPU runs the whole batch."""
    dt, B, E, H, L, S, d, hub = spec
    c = _case(spec)
    print(f"[wide backward] {dt} B={B} E={E} H={H} L={L} S={S} nnz={c.nnz0}", flush=True)
    picked = [0, B - 1]
    rng = np.random.default_rng(73)
    G = np.zeros((B, L, E), np.float32)
    G[picked] = rng.standard_normal((2, L, E)).astype(np.float32)
    if dt == "bf16":
        G = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(G))
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    dev = synth.to_torch(c)
    plan = pma.pma_create(c.src, c.tgt, L, S, E, H, dtype=dt)
    try:
        args = (dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["bq"], dev["wk"], dev["bk"],
                dev["wv"], dev["bv"], dev["wo"], dev["bo"])
        _, _, save = pma.pma_forward_train(plan, *args)
        assert save.numel() >= 1 << 31                      # save area past 2 GiB
        gr = pma.pma_backward(plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["wk"],
                              dev["wv"], dev["wo"], True, save,
                              torch.from_numpy(G).to(tdt).cuda())
        torch.cuda.synchronize()
        got = {n: to_f64(gr[n], dt) for n in NAMES}
        got["k_b"] = to_f64(gr["k_b"], dt)
    finally:
        pma.pma_destroy(plan)
        del dev
    src, tgt = oracle.prepare_edges(c.src, c.tgt, L, S, E, H, False)
    params = {k: oracle.widen(v, dt) for k, v in c.params.items()}
    par, tok = None, {"query": [], "key": []}
    for b in picked:
        xq = oracle.widen(c.xq[b:b + 1], dt)
        xk = oracle.widen(c.xk[b:b + 1], dt)
        r = ob.gradients(1, L, S, E, H, xq, xk, xk, params, src, tgt,
                         G[b:b + 1].astype(np.float64), shared="kv")
        tok["query"].append(r["query"][0])
        tok["key"].append(r["key"][0])
        p = {k: r[k] for k in ("wq", "wk", "wv", "wo", "bq", "bk", "bv", "bo")}
        par = p if par is None else {k: par[k] + p[k] for k in par}
    tol = TOL[dt]
    rows = {"query": L, "key": S}
    for n in ("query", "key"):
        have = got[n].reshape(B, rows[n], E)
        others = np.ones(B, bool)
        others[picked] = False
        assert (have[others] == 0).all(), n               # zero upstream gradient
        err = max_abs_rel(have[picked], np.stack(tok[n]))
        record(f"wide backward {dt}", n + " (two samples)", err, tol)
        assert err <= tol, (n, err)
    for n, o in NAMES.items():
        if o is None:
            continue
        err = max_abs_rel(got[n].reshape(par[o].shape), par[o])
        record(f"wide backward {dt}", n, err, tol)
        assert err <= tol, (n, err)
    assert np.abs(got["k_b"]).max() <= tol * np.abs(par["wk"]).max()
