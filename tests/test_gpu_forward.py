"""GPU forward parity with the oracle (fp32 <= 1e-5, bf16 <= 2e-2 max-abs-rel,
the tolerance measured over the whole output / weights tensor), plus the
exact special cases: a target without edges outputs exactly the out_proj bias,
a target with one edge gives it weight exactly 1."""
import numpy as np
import pytest
import torch

import graph_sparse_head_amd as pma
import oracle
from graph_sparse_head_amd import synth
from gpu_helpers import TOL, make_plan, max_abs_rel, record, run

pytestmark = pytest.mark.gpu


def _full_check(case, need_weights=True, average=True, lead=None):
    print(f"[forward] {case.name} B={case.B} L={case.L} S={case.S} E={case.E} H={case.H} "
          f"{case.dtype} w={need_weights} avg={average}", flush=True)
    out, w, plan = run(case, need_weights=need_weights, average=average, lead=lead)
    try:
        ref = oracle.case_forward(case, want_weights=need_weights)
        err = max_abs_rel(out, ref["out"])
        if case.name in ("tiny", "complete"):
            record(f"forward {case.name}", "out", err, TOL[case.dtype])
        assert err <= TOL[case.dtype], err
        deg = np.bincount(ref["tgt"], minlength=case.L)
        bo = case.params["bo"]
        bo64 = np.zeros(case.E) if bo is None else oracle.widen(bo, case.dtype)
        assert (out[:, deg == 0] == bo64).all()               # exactly the bias
        if need_weights:
            rw = ref["weights"]
            rw = oracle.average_heads(rw) if average else rw
            werr = max_abs_rel(w, rw)
            assert werr <= TOL[case.dtype], werr
            one = deg[ref["tgt"]] == 1
            assert (w[:, one] == 1.0).all()                     # lone edge: weight 1
            assert (w >= 0).all()
        return out, w
    finally:
        pma.pma_destroy(plan)


def test_tiny_averaged():
    _full_check(synth.tiny(), need_weights=True, average=True)


def test_tiny_per_head():
    _full_check(synth.tiny(), need_weights=True, average=False)


@pytest.mark.parametrize("bias", ["normal", "zero", "none"])
def test_complete(bias):
    _full_check(synth.complete(bias=bias), need_weights=True, average=True)


def test_complete_without_weights():
    _full_check(synth.complete(), need_weights=False)


@pytest.mark.parametrize("loops", [True, False])
def test_worked_example(loops):
    c = synth.worked_example(add_self_loops=loops)
    out, w = _full_check(c, need_weights=True, average=False)
    assert w.shape == (2, 8 if loops else 4, 2)


# fast paths (16-byte chunks) and the generic kernels, several tiles + ragged tails
SMALL = [
    # (name, seed, B, L, S, E, H, p, dtype, same_kv, same_qkv, loops)
    ("f32_d16", 1, 3, 300, 300, 64, 4, 0.03, "f32", True, True, False),
    ("f32_d16_bip", 2, 5, 70, 410, 128, 8, 0.05, "f32", True, False, False),
    ("f32_d32_sep", 3, 2, 130, 170, 128, 4, 0.04, "f32", False, False, False),
    ("f32_d4", 4, 4, 90, 90, 64, 16, 0.05, "f32", True, True, True),
    ("f32_d8", 5, 3, 100, 100, 64, 8, 0.05, "f32", True, True, False),
    ("bf16_d16", 6, 7, 333, 333, 64, 4, 0.03, "bf16", True, True, False),
    ("bf16_d16_E128", 7, 3, 250, 250, 128, 8, 0.04, "bf16", True, True, True),
    ("bf16_d32_sep", 8, 2, 120, 260, 128, 4, 0.05, "bf16", False, False, False),
    ("bf16_d8", 9, 5, 100, 100, 64, 8, 0.05, "bf16", True, True, False),
    ("bf16_d64", 10, 2, 80, 80, 128, 2, 0.08, "bf16", True, True, False),
    ("f32_generic_d12", 11, 3, 60, 70, 48, 4, 0.1, "f32", True, False, False),
    ("bf16_generic_d4", 12, 2, 50, 50, 16, 4, 0.1, "bf16", True, True, False),
    ("f32_odd_E", 13, 2, 40, 40, 20, 5, 0.2, "f32", True, True, True),
    ("f32_B1", 14, 1, 200, 200, 64, 4, 0.05, "f32", True, True, False),
    ("bf16_B1", 15, 1, 200, 200, 64, 4, 0.05, "bf16", True, True, False),
    ("f32_bigB", 16, 40, 60, 60, 64, 4, 0.1, "f32", True, True, False),
]


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("avg", [True, False])
def test_small_random(spec, avg):
    name, seed, B, L, S, E, H, p, dt, same_kv, same_qkv, loops = spec
    c = synth.random_case(seed, B, L, S, E, H, p, dtype=dt, same_kv=same_kv, same_qkv=same_qkv,
                          add_self_loops=loops, name=name)
    _full_check(c, need_weights=True, average=avg)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_no_bias_no_weights(dt):
    c = synth.random_case(21, 3, 150, 150, 64, 4, 0.05, dtype=dt, bias="none", name="nobias")
    _full_check(c, need_weights=False)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_leading_axes(dt):
    c = synth.random_case(22, 6, 100, 100, 64, 4, 0.05, dtype=dt, name="lead")
    _full_check(c, need_weights=True, average=False, lead=(2, 3))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("deg", [65, 300, 1500])
def test_split_targets(dt, deg, monkeypatch):
    """Targets above the plan's chunk are split into pieces and merged."""
    monkeypatch.setenv("PMA_CHUNK", "256")
    rng = np.random.default_rng(deg)
    L, S, B, E, H = 40, 2000, 3, 64, 4
    src, tgt = [], []
    for t in range(L):
        d = deg if t % 3 == 0 else int(rng.integers(0, 70))
        s = rng.choice(S, size=d, replace=False)
        src += s.tolist()
        tgt += [t] * d
    c = synth.random_case(30, B, L, S, E, H, 0.0, dtype=dt, name=f"split{deg}")
    c.src, c.tgt = np.array(src, np.int64), np.array(tgt, np.int64)
    perm = rng.permutation(c.src.shape[0])
    c.src, c.tgt = c.src[perm], c.tgt[perm]
    _full_check(c, need_weights=True, average=False)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_split_merge_repeated_calls(dt, monkeypatch):
    """Repeated forwards on one plan with split targets, with batches of
    different sample-group counts in between (the partial slots are reused),
    give the oracle's result and bit-identical repeats."""
    monkeypatch.setenv("PMA_CHUNK", "3")
    big = synth.random_case(41, 37, 120, 120, 64, 4, 0.1, dtype=dt, name="merge_big")
    small = synth.random_case(41, 5, 120, 120, 64, 4, 0.1, dtype=dt, name="merge_small")
    small.src, small.tgt = big.src, big.tgt
    plan = make_plan(big)
    try:
        first, w_first, _ = run(big, plan=plan, need_weights=True, average=False)
        for case in (small, big, small):
            out, w, _ = run(case, plan=plan, need_weights=True, average=False)
            ref = oracle.case_forward(case, want_weights=True)
            assert max_abs_rel(out, ref["out"]) <= TOL[dt]
            assert max_abs_rel(w, ref["weights"]) <= TOL[dt]
        again, w_again, _ = run(big, plan=plan, need_weights=True, average=False)
        assert (again == first).all() and (w_again == w_first).all()
    finally:
        pma.pma_destroy(plan)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_deterministic(dt):
    c = synth.random_case(40, 4, 300, 300, 64, 4, 0.05, dtype=dt, name="det")
    out1, w1, plan = run(c, need_weights=True, average=False)
    try:
        out2, w2, _ = run(c, plan=plan, need_weights=True, average=False)
        assert (out1 == out2).all() and (w1 == w2).all()
    finally:
        pma.pma_destroy(plan)


def test_plan_reuse_growing_batch():
    """One plan, a small batch then a larger one (the workspace grows)."""
    base = synth.random_case(41, 2, 120, 120, 64, 4, 0.06, dtype="f32", name="grow")
    big = synth.random_case(41, 9, 120, 120, 64, 4, 0.06, dtype="f32", name="grow")
    big.src, big.tgt = base.src, base.tgt
    out, _, plan = run(base, need_weights=False)
    try:
        assert max_abs_rel(out, oracle.case_forward(base)["out"]) <= TOL["f32"]
        out, w, _ = run(big, plan=plan, need_weights=True, average=True)
        ref = oracle.case_forward(big, want_weights=True)
        assert max_abs_rel(out, ref["out"]) <= TOL["f32"]
        assert max_abs_rel(w, oracle.average_heads(ref["weights"])) <= TOL["f32"]
    finally:
        pma.pma_destroy(plan)


def test_forward_rejects():
    c = synth.tiny()
    plan = pma.pma_create(c.src, c.tgt, c.L, c.S, c.E, c.H)
    dev = synth.to_torch(c)
    try:
        with pytest.raises(pma.PmaError) as e:
            pma.pma_forward(plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["bq"],
                            dev["wk"], None, dev["wv"], dev["bv"], dev["wo"], dev["bo"])
        assert e.value.name == "PMA_E_ARG"
        with pytest.raises(pma.PmaError) as e:
            pma.pma_forward(plan, dev["xq"].double(), dev["xk"], dev["xv"], dev["wq"], dev["bq"],
                            dev["wk"], dev["bk"], dev["wv"], dev["bv"], dev["wo"], dev["bo"])
        assert e.value.name == "PMA_E_DTYPE"
        with pytest.raises(pma.PmaError) as e:
            pma.pma_forward(plan, dev["xq"][:, :5].contiguous(), dev["xk"], dev["xv"], dev["wq"], dev["bq"],
                            dev["wk"], dev["bk"], dev["wv"], dev["bv"], dev["wo"], dev["bo"])
        assert e.value.name == "PMA_E_SIZE"
    finally:
        pma.pma_destroy(plan)


def test_binding_rejects_buffers_of_the_wrong_size():
    """Preallocated outputs, save areas and gradients are checked against the
    plan's sizes before any launch (a smaller buffer would be written past its
    end on the device)."""
    c = synth.tiny()
    plan = pma.pma_create(c.src, c.tgt, c.L, c.S, c.E, c.H)
    dev = synth.to_torch(c)
    args = (plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["bq"], dev["wk"], dev["bk"],
            dev["wv"], dev["bv"], dev["wo"], dev["bo"])
    n = plan.nnz
    f32 = dict(dtype=torch.float32, device="cuda")
    try:
        for kw in (dict(out=torch.empty(1, c.L, c.E, **f32)),
                   dict(weights=torch.empty(c.B, n - 1, **f32)),
                   dict(weights=torch.empty(c.B, n, **f32), average_attn_weights=False),
                   dict(weights=torch.empty(1, n, **f32))):
            with pytest.raises(pma.PmaError) as e:
                pma.pma_forward(*args, **kw)
            assert e.value.name == "PMA_E_SIZE", kw
        with pytest.raises(pma.PmaError) as e:
            pma.pma_forward(plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"][:4].contiguous(),
                            dev["bq"], dev["wk"], dev["bk"], dev["wv"], dev["bv"], dev["wo"],
                            dev["bo"])
        assert e.value.name == "PMA_E_SIZE"
        small = torch.empty(pma.pma_train_bytes(plan, c.B) - 256, dtype=torch.uint8,
                            device="cuda")
        with pytest.raises(pma.PmaError) as e:
            pma.pma_forward_train(*args, save=small)
        assert e.value.name == "PMA_E_SIZE"
        out, _, save = pma.pma_forward_train(*args)
        g = torch.empty(1, c.L, c.E, **f32)
        with pytest.raises(pma.PmaError) as e:
            pma.pma_backward(plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["wk"],
                             dev["wv"], dev["wo"], True, save, g)
        assert e.value.name == "PMA_E_SIZE"
        with pytest.raises(pma.PmaError) as e:
            pma.pma_backward(plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["wk"],
                             dev["wv"], dev["wo"], True, save[:64],
                             torch.zeros(c.B, c.L, c.E, **f32))
        assert e.value.name == "PMA_E_SIZE"
        torch.cuda.synchronize()
    finally:
        pma.pma_destroy(plan)


# fp32 at embed_dim 128: projections as split-bf16 matrix-core products
# (default) or on the fp32 matrix cores (PMA_F32_SPLIT=0); ragged row tiles
# (B * L and B * S not multiples of 256), separate query / key / value tokens,
# with and without biases, per-head weights.
@pytest.mark.parametrize("split", ["1", "0"])
@pytest.mark.parametrize("bias", ["normal", "none"])
def test_fp32_embed128_projections(split, bias, monkeypatch):
    monkeypatch.setenv("PMA_F32_SPLIT", split)
    c = synth.random_case(101, 3, 171, 203, 128, 8, 0.05, dtype="f32", bias=bias, same_kv=False,
                          same_qkv=False, name="f32_e128")
    print(f"[forward] fp32 E=128 split={split} bias={bias}", flush=True)
    out, w, plan = run(c, need_weights=True, average=False)
    pma.pma_destroy(plan)
    ref = oracle.case_forward(c, want_weights=True)
    assert max_abs_rel(out, ref["out"]) <= TOL["f32"]
    assert max_abs_rel(w, ref["weights"]) <= TOL["f32"]


# ---------------------------------------------------------------------------
# full-size workloads in the launch configuration the benchmark times: every
# output element (and every per-edge weight) against the oracle


@pytest.mark.parametrize("name", ["gene", "bipartite", "large"])
def test_full_size(name):
    c = synth.make_config(name)
    print(f"[forward] full {name} nnz0={c.nnz0}", flush=True)
    out, w, plan = run(c)
    try:
        src, tgt = pma.pma_edges(plan)
    finally:
        pma.pma_destroy(plan)
    ref = oracle.case_forward(c, want_weights=c.need_weights)
    assert (ref["src"] == src).all() and (ref["tgt"] == tgt).all()
    err = max_abs_rel(out, ref["out"])
    record(f"forward {name}", "out", err, TOL[c.dtype])
    assert err <= TOL[c.dtype], err
    deg = np.bincount(tgt, minlength=c.L)
    bo = oracle.widen(c.params["bo"], c.dtype)
    assert (out[:, deg == 0] == bo).all()                       # exactly the bias
    if c.need_weights:
        rw = oracle.average_heads(ref["weights"])
        werr = max_abs_rel(w, rw)
        record(f"forward {name}", "weights", werr, TOL[c.dtype])
        assert werr <= TOL[c.dtype], werr
        assert (w >= 0).all()
        assert (w[:, deg[tgt] == 1] == 1.0).all()               # lone edge: weight 1
        # every target's weights sum to 1 at every sample
        sums = np.zeros((c.B, c.L))
        np.add.at(sums, (slice(None), tgt), w)
        serr = np.abs(sums[:, deg > 0] - 1).max()
        record(f"forward {name}", "weight sums", serr, TOL[c.dtype])
        assert serr <= TOL[c.dtype], serr


# ---------------------------------------------------------------------------
# every tuning knob gives the same results (read at plan creation)

KNOBS = [
    {},
    {"PMA_COMPACT": "0"},
    {"PMA_COMPACT": "1", "PMA_LAYOUT": "batch"},
    {"PMA_PERSIST": "1"},
    {"PMA_NT": "1", "PMA_PERSIST": "0"},
    {"PMA_FUSE_OUT": "0"},
    {"PMA_LAYOUT": "batch"},
    {"PMA_LAYOUT": "batch", "PMA_FUSE_OUT": "0"},
    {"PMA_CHUNK": "3"},
    {"PMA_CHUNK": "3", "PMA_FUSE_OUT": "0"},
    {"PMA_XCD_MAP": "1"},
    {"PMA_XCD_MAP": "0", "PMA_NT": "0"},
    {"PMA_NT": "2", "PMA_CHUNK": "3"},
    {"PMA_NT": "3", "PMA_FUSE_OUT": "0"},
    {"PMA_FUSE_IN": "0"},
    {"PMA_FUSE_IN": "0", "PMA_CHUNK": "3"},
    {"PMA_HOT": "1"},
    {"PMA_XCD_MAP": "2"},
    {"PMA_XCD_MAP": "2", "PMA_PERSIST": "1", "PMA_CHUNK": "3"},
]


@pytest.mark.parametrize("knobs", KNOBS, ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
@pytest.mark.parametrize("shape", [("f32", 64, 4), ("bf16", 64, 4), ("bf16", 128, 8)])
def test_tuning_knobs(knobs, shape, monkeypatch):
    for k, v in knobs.items():
        monkeypatch.setenv(k, v)
    dt, E, H = shape
    c = synth.random_case(50, 5, 220, 220, E, H, 0.04, dtype=dt, name="knobs")
    # two hub targets so that small chunks split them; sources 120.. are never
    # read, so that keys and values are projected for the read ones only
    rng = np.random.default_rng(51)
    hub_src = rng.choice(120, size=100, replace=False)
    keep = ~np.isin(c.tgt, [3, 17]) & (c.src < 120)
    c.src = np.concatenate([c.src[keep], hub_src, hub_src[:60]])
    c.tgt = np.concatenate([c.tgt[keep], np.full(100, 3), np.full(60, 17)])
    _full_check(c, need_weights=True, average=False)


@pytest.mark.parametrize("fuse_in", ["0", "1"])
@pytest.mark.parametrize("compact", ["0", "1"])
@pytest.mark.parametrize("shared", ["none", "kv", "qkv"])
@pytest.mark.parametrize("B", [5, 37])
@pytest.mark.parametrize("H", [1, 2, 4, 8])
def test_q_projection_in_edge_kernel(fuse_in, compact, shared, B, H, monkeypatch):
    # bf16 at embed_dim 64: the edge kernel projects q from the query rows
    # itself (PMA_FUSE_IN=1, the default) or reads a separately projected q;
    # with shared tokens the key/value projection then runs on its own. B = 5
    # leaves lanes without a sample, B = 37 a partial sample group; H = 1..8
    # puts a head on 8, 4, 2 or 1 lanes.
    monkeypatch.setenv("PMA_FUSE_IN", fuse_in)
    monkeypatch.setenv("PMA_COMPACT", compact)
    c = synth.random_case(93, B, 300, 300, 64, H, 0.02, dtype="bf16", same_kv=shared != "none",
                          same_qkv=shared == "qkv", name="fuse_in")
    keep = c.src < 200   # sources 200.. are never read
    c.src, c.tgt = c.src[keep], c.tgt[keep]
    _full_check(c, need_weights=True, average=False)


# Hot-row cache (PMA_HOT=1; bf16 inference with the q projection in the edge
# kernel, no weights, no mask): each workgroup keeps the key/value rows of the 64
# most-read sources in LDS and a target row lists those sources first, so a
# piece runs all-cached steps, all-memory steps and at most one step across
# the boundary. Zipf-popular sources, split targets (PMA_CHUNK=5), compacted
# key/value rows, one and four sample groups and partial ones.
@pytest.mark.parametrize("hot", ["0", "1"])
@pytest.mark.parametrize("chunk", ["auto", "5"])
@pytest.mark.parametrize("compact", ["0", "1"])
@pytest.mark.parametrize("B,H", [(3, 4), (8, 4), (32, 4), (8, 1), (8, 8), (20, 2)])
def test_hot_row_cache(hot, chunk, compact, B, H, monkeypatch):
    monkeypatch.setenv("PMA_HOT", hot)
    monkeypatch.setenv("PMA_COMPACT", compact)
    if chunk != "auto":
        monkeypatch.setenv("PMA_CHUNK", chunk)
    c = synth.gene(n=3000, B=B, H=H, max_deg=400)
    keep = c.src % 7 != 3   # some sources never read (compaction renumbers the rest)
    c.src, c.tgt = c.src[keep], c.tgt[keep]
    _full_check(c, need_weights=False)


@pytest.mark.parametrize("knobs", [{"PMA_PERSIST": "1"}, {"PMA_PERSIST": "1", "PMA_XCD_MAP": "1"},
                                   {"PMA_PERSIST": "1", "PMA_XCD_MAP": "2"},
                                   {"PMA_PERSIST": "2", "PMA_CHUNK": "5"}],
                         ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_wavefront_walks_pieces(knobs, dt, monkeypatch):
    # More pieces than wavefronts: each wavefront of the edge kernel walks
    # several pieces (its next piece's bounds and query fetched ahead).
    for k, v in knobs.items():
        monkeypatch.setenv(k, v)
    c = synth.random_case(52, 4, 6000, 6000, 64, 4, 0.0015, dtype=dt, name="walk")
    _full_check(c, need_weights=True, average=True)


@pytest.mark.parametrize("name", ["tiny", "complete", "gene", "bipartite", "large"])
def test_automatic_piece_length(name):
    # a target is split only above 16x the average in-degree (a power of two,
    # at least 256)
    c = synth.make_config(name)
    plan = pma.pma_create(c.src, c.tgt, c.L, c.S, c.E, c.H, add_self_loops=c.add_self_loops,
                          dtype=c.dtype)
    try:
        info = pma.pma_plan_info(plan)
        want = 256
        while want < 16 * plan.nnz / c.L:
            want *= 2
        assert info["chunk"] == min(want, 65535)
    finally:
        pma.pma_destroy(plan)
