"""The memory-path calibration entry point (pma_gather_ceiling): wavefront w
folds with XOR the 1 KB rows rows[w * per .. w * per + per - 1] of the table,
lane l holding bytes 16 l .. 16 l + 15 of each row, and row indices outside
the table read its last row. Checked bit for bit against the same fold on
the host."""
import numpy as np
import pytest
import torch

import graph_sparse_head_amd as pma

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,per", [(103, 5), (64, 64), (1, 1), (1000, 8), (999, 7)])
def test_gather_ceiling_folds_the_rows(n, per):
    print(f"[calibrate] n={n} per={per}", flush=True)
    rng = np.random.default_rng(n + per)
    n_tab = 37
    table = rng.integers(0, 2**32, size=(n_tab, 256), dtype=np.uint64).astype(np.uint32)
    rows = rng.integers(-3, n_tab + 5, size=n).astype(np.int32)   # some past either end
    waves = -(-n // per)
    t_dev = torch.from_numpy(table.view(np.int32)).cuda()
    r_dev = torch.from_numpy(rows).cuda()
    sink = torch.full((waves * 256,), -1, dtype=torch.int32, device="cuda")
    pma.pma_gather_ceiling(t_dev, r_dev, per, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32).reshape(waves, 256)
    clamped = np.where((rows < 0) | (rows >= n_tab), n_tab - 1, rows)
    for w in range(waves):
        want = np.bitwise_xor.reduce(table[clamped[w * per:(w + 1) * per]], axis=0)
        assert np.array_equal(got[w], want), w


def test_gather_ceiling_binding_rejects():
    t = torch.zeros(256, dtype=torch.int32, device="cuda")
    r = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(pma.PmaError) as e:
        pma.pma_gather_ceiling(t, r.to(torch.int64), 2, torch.zeros(512, dtype=torch.int32, device="cuda"))
    assert e.value.name == "PMA_E_DTYPE"
    with pytest.raises(pma.PmaError) as e:
        pma.pma_gather_ceiling(t, r, 2, torch.zeros(256, dtype=torch.int32, device="cuda"))
    assert e.value.name == "PMA_E_SIZE"                     # 2 wavefronts need 2 KiB
    with pytest.raises(pma.PmaError) as e:
        pma.pma_gather_ceiling(t[:100], r, 2, torch.zeros(512, dtype=torch.int32, device="cuda"))
    assert e.value.name == "PMA_E_ARG"                      # 400 bytes: not whole KiB


def _case(dt, E, H, seed=600):
    from graph_sparse_head_amd import synth
    c = synth.random_case(seed, 5, 120, 120, E, H, 0.05, dtype=dt, name="probe")
    # a hub target, so that short chunks split it into pieces
    keep = c.tgt != 9
    c.src = np.concatenate([c.src[keep], np.arange(0, 100)])
    c.tgt = np.concatenate([c.tgt[keep], np.full(100, 9)])
    return c


def test_gather_probe_needs_a_forward():
    from gpu_helpers import make_plan
    c = _case("bf16", 64, 4)
    plan = make_plan(c)
    try:
        with pytest.raises(pma.PmaError) as e:
            pma.pma_gather_probe(plan)
        assert e.value.name == "PMA_E_ARG"
    finally:
        pma.pma_destroy(plan)


@pytest.mark.parametrize("shape", [("bf16", 64, 4), ("f32", 64, 4), ("bf16", 128, 8), ("f32", 128, 8)],
                         ids=lambda s: f"{s[0]}_E{s[1]}_H{s[2]}")
@pytest.mark.parametrize("mask", [False, True])
def test_gather_probe_leaves_the_forward_intact(shape, mask, monkeypatch):
    # The probe walks the last forward's pieces (split targets included) and
    # writes into the plan's workspace only: the next forward on the same
    # plan still matches the oracle and repeats the first bit for bit.
    import oracle
    from gpu_helpers import TOL, make_plan, max_abs_rel, run
    monkeypatch.setenv("PMA_CHUNK", "16")
    dt, E, H = shape
    c = _case(dt, E, H)
    kpm = None
    if mask:
        kpm = np.random.default_rng(601).random((c.B, c.S)) < 0.3
    plan = make_plan(c)
    try:
        out1, w1, _ = run(c, plan=plan, need_weights=True, average=False, kpm=kpm)
        for _ in range(2):
            pma.pma_gather_probe(plan)
        torch.cuda.synchronize()
        out2, w2, _ = run(c, plan=plan, need_weights=True, average=False, kpm=kpm)
        assert np.array_equal(out1, out2) and np.array_equal(w1, w2)
        ref = oracle.case_forward(c, want_weights=True, key_padding_mask=kpm)
        assert max_abs_rel(out2, ref["out"]) <= TOL[dt]
    finally:
        pma.pma_destroy(plan)


def test_gather_probe_refuses_the_per_channel_kernel():
    # head size 6 in fp32 is not a whole number of 16-byte chunks: those
    # forwards run the per-channel kernel, which the probe does not mirror
    from gpu_helpers import make_plan, run
    c = _case("f32", 12, 2)
    plan = make_plan(c)
    try:
        run(c, plan=plan, need_weights=False)
        with pytest.raises(pma.PmaError) as e:
            pma.pma_gather_probe(plan)
        assert e.value.name == "PMA_E_UNSUPPORTED"
    finally:
        pma.pma_destroy(plan)
