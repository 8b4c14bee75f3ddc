"""Tensors past 2 GiB. Once any tensor the edge kernels address reaches
2 GiB (here the key / value rows of the batch) they switch from 32-bit to
64-bit offsets: the q projection, out_proj, the merge of split targets and the
per-edge weights then run in those variants. Checked against the oracle on
sampled (sample, target) rows that include two split hub targets,
zero-degree targets and lone edges, for outputs and per-edge weights."""
import functools

import numpy as np
import pytest

import graph_sparse_head_amd as pma
import oracle
from graph_sparse_head_amd import synth
from gpu_helpers import TOL, max_abs_rel, record, run

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


@functools.lru_cache(maxsize=1)
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
