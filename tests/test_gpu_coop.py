"""Split targets merged inside the edge kernel (opt-in, PMA_COOP=1). Where
every split target has at most four pieces, the sample groups are pinned to
XCDs and there is no key_padding_mask, one workgroup per (split target,
sample group) walks the target's pieces, one per wavefront, and merges them
after a workgroup barrier, so no merge launch follows. Checked here: parity with the oracle, outputs, weights, softmax
statistics and gradients bit-identical to the separate merge launch
(PMA_COOP=0), and which of the two a plan takes (the merge stage's launch
count)."""
import numpy as np
import pytest
import torch

import graph_sparse_head_amd as pma
import oracle
from graph_sparse_head_amd import synth
from gpu_helpers import TOL, make_plan, max_abs_rel, run, to_f64

pytestmark = pytest.mark.gpu


def _hub_case(seed, B, E, H, dt, hub_degrees, L=60, S=400, name="coop"):
    """Targets 0, 5, 10, ... have the given in-degrees (cycled); the others
    0-15 sources. With PMA_CHUNK=16 a hub of degree g has ceil(g / 16)
    pieces."""
    rng = np.random.default_rng(seed)
    src, tgt = [], []
    hubs = iter(hub_degrees * L)
    for t in range(L):
        d = next(hubs) if t % 5 == 0 else int(rng.integers(0, 16))
        src += rng.choice(S, size=d, replace=False).tolist()
        tgt += [t] * d
    c = synth.random_case(seed, B, L, S, E, H, 0.0, dtype=dt, same_kv=True, same_qkv=False,
                          name=name)
    perm = rng.permutation(len(src))
    c.src = np.array(src, np.int64)[perm]
    c.tgt = np.array(tgt, np.int64)[perm]
    return c


def _merge_launches(plan, case, dev, kpm=None, need_weights=True, average=False):
    """The forward's merge-stage launches (0 when the edge kernel merged)."""
    lib = pma._load()
    lib.pma_profile_stages(plan.handle, (1 << len(pma.STAGES)) - 1)
    pma.pma_profile_read(plan)
    run(case, plan=plan, dev=dev, need_weights=need_weights, average=average, kpm=kpm)
    st = pma.pma_profile_read(plan)
    lib.pma_profile_stages(plan.handle, 0)
    return st["merge"][1]


def _pair(case, monkeypatch, kpm=None, need_weights=True, average=False, expect_coop=True):
    """Forwards of one case on a plan that merges in the edge kernel and on
    one that launches the merge; both against the oracle, and against each
    other bit for bit."""
    print(f"[coop] {case.name} B={case.B} E={case.E} H={case.H} {case.dtype} "
          f"w={need_weights} mask={kpm is not None}", flush=True)
    dev = synth.to_torch(case)
    monkeypatch.setenv("PMA_CHUNK", "16")
    monkeypatch.setenv("PMA_COOP", "1")
    p_coop = make_plan(case)
    monkeypatch.setenv("PMA_COOP", "0")
    p_launch = make_plan(case)
    try:
        got = {}
        for name, plan in (("coop", p_coop), ("launch", p_launch)):
            got[name] = run(case, plan=plan, dev=dev, need_weights=need_weights,
                            average=average, kpm=kpm)[:2]
            launches = _merge_launches(plan, case, dev, kpm, need_weights, average)
            assert launches == (0 if name == "coop" and expect_coop else 1), (name, launches)
        ref = oracle.case_forward(case, want_weights=need_weights, key_padding_mask=kpm)
        out, w = got["coop"]
        assert max_abs_rel(out, ref["out"]) <= TOL[case.dtype]
        assert (out == got["launch"][0]).all()
        if need_weights:
            rw = ref["weights"] if not average else oracle.average_heads(ref["weights"])
            assert max_abs_rel(w, rw) <= TOL[case.dtype]
            assert (w == got["launch"][1]).all()
    finally:
        pma.pma_destroy(p_coop)
        pma.pma_destroy(p_launch)


# (dtype, E, H, B): one sample group; two, four and eight groups pinned to
# XCDs; E = 64 with out_proj (and for bf16 the q projection) in the edge
# kernel, E = 128 with both as launches of their own; heads of 1-4 lanes.
SHAPES = [("bf16", 64, 4, 5), ("bf16", 64, 4, 32), ("bf16", 64, 8, 16), ("f32", 64, 4, 3),
          ("f32", 64, 4, 32), ("f32", 64, 16, 8), ("bf16", 128, 8, 8), ("f32", 128, 8, 16),
          ("f32", 128, 4, 2)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}_E{s[1]}_H{s[2]}_B{s[3]}")
@pytest.mark.parametrize("hubs", [[20], [40], [60, 64], [17, 33, 49, 64]],
                         ids=["2pieces", "3pieces", "4pieces", "mixed"])
def test_coop_matches_merge_launch(shape, hubs, monkeypatch):
    dt, E, H, B = shape
    c = _hub_case(61, B, E, H, dt, hubs)
    _pair(c, monkeypatch, need_weights=True, average=False)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_coop_without_weights_and_averaged(dt, monkeypatch):
    c = _hub_case(62, 32, 64, 4, dt, [64, 30])
    _pair(c, monkeypatch, need_weights=False)
    _pair(c, monkeypatch, need_weights=True, average=True)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_masked_forward_uses_the_merge_launch(dt, monkeypatch):
    # with a key_padding_mask split targets keep the merge launch; sample 1
    # masks every key of the first hub (its pieces then carry m = -inf, l = 0
    # and the target outputs the bias)
    c = _hub_case(63, 8, 64, 4, dt, [50, 64])
    kpm = np.random.default_rng(64).random((c.B, c.S)) < 0.3
    kpm[1, c.src[c.tgt == 0]] = True
    _pair(c, monkeypatch, kpm=kpm, need_weights=True, average=False, expect_coop=False)


def test_five_pieces_use_the_merge_launch(monkeypatch):
    # a target of 5 pieces: the whole plan keeps the merge launch
    c = _hub_case(65, 32, 64, 4, "bf16", [70, 20])
    _pair(c, monkeypatch, need_weights=True, average=False, expect_coop=False)


def test_unpinned_groups_use_the_merge_launch(monkeypatch):
    # five sample groups do not divide the 8 XCDs: no pinning, merge launch
    c = _hub_case(66, 37, 64, 4, "bf16", [40])
    _pair(c, monkeypatch, need_weights=True, average=False, expect_coop=False)


@pytest.mark.parametrize("shape", [("bf16", 64, 4, 32), ("f32", 64, 4, 8), ("bf16", 128, 8, 8)],
                         ids=lambda s: f"{s[0]}_E{s[1]}_B{s[3]}")
def test_coop_training_bit_identical(shape, monkeypatch):
    """The training forward's saved softmax statistics of split targets come
    from the in-kernel merge: the backward's gradients equal those of a plan
    with the merge launch bit for bit."""
    dt, E, H, B = shape
    c = _hub_case(67, B, E, H, dt, [64, 40, 20])
    print(f"[coop train] B={B} E={E} H={H} {dt}", flush=True)
    dev = synth.to_torch(c)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    g_dev = torch.from_numpy(np.random.default_rng(68).standard_normal((B, c.L, E))
                             .astype(np.float32)).to(tdt).cuda()
    args = (dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["bq"], dev["wk"], dev["bk"],
            dev["wv"], dev["bv"], dev["wo"], dev["bo"])
    monkeypatch.setenv("PMA_CHUNK", "16")
    res = {}
    for coop in ("1", "0"):
        monkeypatch.setenv("PMA_COOP", coop)
        plan = make_plan(c)
        try:
            out, _, save = pma.pma_forward_train(plan, *args)
            gr = pma.pma_backward(plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["wk"],
                                  dev["wv"], dev["wo"], True, save, g_dev)
            torch.cuda.synchronize()
            res[coop] = {"out": to_f64(out, dt),
                         **{k: to_f64(v, dt) for k, v in gr.items() if v is not None}}
        finally:
            pma.pma_destroy(plan)
    ref = oracle.case_forward(c)
    assert max_abs_rel(res["1"]["out"], ref["out"]) <= TOL[dt]
    for k in res["0"]:
        assert (res["1"][k] == res["0"][k]).all(), k
