"""GPU index build: the target-grouped edges and the work split must equal the
oracle's integer references bit for bit; repeated pairs must be rejected."""
import numpy as np
import pytest

import graph_sparse_head_amd as pma
import oracle
from graph_sparse_head_amd import synth

pytestmark = pytest.mark.gpu


def _check_plan(src0, tgt0, L, S, E=8, H=2, loops=False):
    print(f"[index] L={L} S={S} nnz0={len(src0)} loops={loops}", flush=True)
    plan = pma.pma_create(src0, tgt0, L, S, E, H, add_self_loops=loops)
    try:
        src, tgt = oracle.prepare_edges(src0, tgt0, L, S, E, H, loops)
        es, et = pma.pma_edges(plan)
        assert (es == src).all() and (et == tgt).all()
        assert pma.pma_nnz(plan) == src.shape[0]
        rp, cs, ce = pma.pma_csr(plan)
        orp, ocs, oce = oracle.csr(src, tgt, L)
        assert (rp == orp).all()
        assert (cs == ocs).all()
        assert (ce == oce).all()
        info = pma.pma_plan_info(plan)
        ws = pma.pma_work_split(plan)
        ows = oracle.work_split(orp, info["chunk"])
        for k in ("task_target", "task_begin", "task_end", "task_slot", "split_target",
                  "split_slot0", "split_count"):
            assert (ws[k] == ows[k]).all(), k
        assert ws["n_slots"] == ows["n_slots"]
        assert info["max_degree"] == int(np.diff(orp).max())
        assert info["kv_rows"] == np.unique(src).shape[0]
    finally:
        pma.pma_destroy(plan)


@pytest.mark.parametrize("name", ["tiny", "complete", "gene", "bipartite", "large"])
def test_csr_configs(name):
    c = synth.make_config(name)
    _check_plan(c.src, c.tgt, c.L, c.S, c.E, c.H, c.add_self_loops)


def test_csr_shuffled_gene():
    c = synth.gene()
    perm = np.random.default_rng(9).permutation(c.nnz0)
    _check_plan(c.src[perm], c.tgt[perm], c.L, c.S, c.E, c.H)


@pytest.mark.parametrize("case", ["single", "hub", "hub_huge", "L_ne_S", "loops_partial",
                                  "loops_all", "L1", "S1", "many_small"])
def test_csr_edge_cases(case):
    rng = np.random.default_rng(1)
    if case == "single":
        _check_plan([3], [1], 5, 7)
    elif case == "hub":
        s = rng.permutation(3000)[:2000]
        _check_plan(s, np.full(2000, 4), 10, 3000)
    elif case == "hub_huge":
        s = rng.permutation(300000)
        _check_plan(s, np.zeros(300000, np.int64), 3, 300000)
    elif case == "L_ne_S":
        s, t = synth.random_graph(rng, 37, 300, 0.2)
        _check_plan(s, t, 37, 300)
    elif case == "loops_partial":
        s, t = synth.random_graph(rng, 50, 50, 0.1)
        _check_plan(s, t, 50, 50, loops=True)
    elif case == "loops_all":
        n = 40
        _check_plan(np.arange(n)[::-1].copy(), np.arange(n)[::-1].copy(), n, n, loops=True)
    elif case == "L1":
        _check_plan(rng.permutation(500), np.zeros(500, np.int64), 1, 500)
    elif case == "S1":
        _check_plan(np.zeros(300, np.int64), rng.permutation(300), 300, 1)
    elif case == "many_small":
        s, t = synth.random_graph(rng, 4000, 4000, 0.002)
        _check_plan(s, t, 4000, 4000, loops=True)


@pytest.mark.parametrize("where", ["first", "middle", "last", "far"])
def test_duplicate_rejected_on_device(where):
    c = synth.gene(n=3000, B=1, max_deg=200, dtype="f32")
    src, tgt = c.src.copy(), c.tgt.copy()
    n = src.shape[0]
    i, j = {"first": (0, 1), "middle": (n // 2, n // 2 + 7), "last": (n - 2, n - 1),
            "far": (3, n - 5)}[where]
    src[j], tgt[j] = src[i], tgt[i]
    print(f"[index] duplicate at {i}, {j}", flush=True)
    with pytest.raises(pma.PmaError) as e:
        pma.pma_create(src, tgt, c.L, c.S, c.E, c.H)
    assert e.value.name == "PMA_E_INDEX_DUPLICATE"


@pytest.mark.parametrize("chunk", ["1", "7", "65535"])
def test_work_split_chunk_knob(chunk, monkeypatch):
    monkeypatch.setenv("PMA_CHUNK", chunk)
    c = synth.gene(n=3000, B=1, max_deg=400, dtype="f32")
    _check_plan(c.src, c.tgt, c.L, c.S, c.E, c.H)
