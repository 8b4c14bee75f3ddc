"""key_padding_mask on the GPU (kpnn2 PackedMultiheadAttention page, forward
parameter table and "Notes" step 3): parity with the oracle under the same
mask, masked edges weigh exactly 0, and targets whose keys are all masked
output exactly the out_proj bias."""
import numpy as np
import pytest

import graph_sparse_head_amd as pma
import oracle
from graph_sparse_head_amd import synth
from gpu_helpers import TOL, max_abs_rel, record, run

pytestmark = pytest.mark.gpu


def _live(kpm, src, tgt, B, L):
    """(B, L): whether (sample, target) keeps some unmasked edge."""
    live = np.zeros((B, L), bool)
    for b in range(B):
        keep = ~(kpm[b] if kpm.ndim == 2 else kpm)[src]
        live[b, np.unique(tgt[keep])] = True
    return live


def _check(case, kpm, need_weights=True, average=True, lead=None):
    print(f"[mask] {case.name} B={case.B} L={case.L} S={case.S} E={case.E} H={case.H} "
          f"{case.dtype} mask{kpm.shape} frac={kpm.mean():.2f}", flush=True)
    out, w, plan = run(case, need_weights=need_weights, average=average, lead=lead, kpm=kpm)
    try:
        ref = oracle.case_forward(case, want_weights=need_weights, key_padding_mask=kpm)
        err = max_abs_rel(out, ref["out"])
        assert err <= TOL[case.dtype], err
        src, tgt = ref["src"], ref["tgt"]
        live = _live(kpm, src, tgt, case.B, case.L)
        bo = case.params["bo"]
        bo64 = np.zeros(case.E) if bo is None else oracle.widen(bo, case.dtype)
        assert (out[~live] == bo64).all()                        # exactly the bias
        if need_weights:
            rw = ref["weights"]
            rw = oracle.average_heads(rw) if average else rw
            assert max_abs_rel(w, rw) <= TOL[case.dtype]
            for b in range(case.B):
                m = (kpm[b] if kpm.ndim == 2 else kpm)[src]
                assert (w[b][m] == 0).all()                      # masked: weight 0
        return out, w
    finally:
        pma.pma_destroy(plan)


SHAPES = [("f32", 8, 2), ("f32", 64, 4), ("bf16", 64, 4), ("bf16", 128, 8), ("f32", 12, 4),
          ("bf16", 48, 2)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}_E{s[1]}_H{s[2]}")
@pytest.mark.parametrize("frac", [0.2, 0.6])
def test_mask_per_sample(shape, frac):
    dt, E, H = shape
    c = synth.random_case(70, 6, 90, 90, E, H, 0.08, dtype=dt, name="mask")
    kpm = np.random.default_rng(71).random((c.B, c.S)) < frac
    kpm[2] = True                                                # one sample fully masked
    _check(c, kpm, need_weights=True, average=False)


# Samples per wavefront of the fast kernel: 64 / (E / chunk). One 32-bit mask
# word per edge covers them up to 32 samples; embed_dim = chunk (fp32 E = 4,
# bf16 E = 8) puts 64 samples on a wavefront and two words; B = 70 leaves a
# partial last group; bf16 E = 16 has 32 samples per wavefront.
@pytest.mark.parametrize("shape", [("f32", 4, 1), ("bf16", 8, 1), ("bf16", 16, 2), ("f32", 8, 2)],
                         ids=lambda s: f"{s[0]}_E{s[1]}_H{s[2]}")
def test_mask_many_samples_per_wavefront(shape):
    dt, E, H = shape
    c = synth.random_case(79, 70, 60, 60, E, H, 0.1, dtype=dt, name="mask_wide")
    kpm = np.random.default_rng(80).random((c.B, c.S)) < 0.3
    kpm[33] = True                                               # a sample of the second word
    kpm[64] = True                                               # and of the third
    _check(c, kpm, need_weights=True, average=True)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_mask_shared_and_leading_axes(dt):
    c = synth.random_case(72, 6, 70, 110, 64, 4, 0.1, dtype=dt, same_kv=True, name="mask_kv")
    kpm = np.random.default_rng(73).random(c.S) < 0.4
    _check(c, kpm, need_weights=True, average=True)
    kpm2 = np.random.default_rng(74).random((c.B, c.S)) < 0.4
    _check(c, kpm2, need_weights=True, average=True, lead=(2, 3))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_mask_all_false_is_unmasked(dt):
    c = synth.random_case(75, 3, 60, 60, 64, 4, 0.1, dtype=dt, name="mask0")
    plan = pma.pma_create(c.src, c.tgt, c.L, c.S, c.E, c.H, dtype=c.dtype)
    try:
        a, wa, _ = run(c, plan=plan, need_weights=True, average=False,
                       kpm=np.zeros((c.B, c.S), bool))
        b, wb, _ = run(c, plan=plan, need_weights=True, average=False)
        assert np.abs(a - b).max() == 0 and np.abs(wa - wb).max() == 0
    finally:
        pma.pma_destroy(plan)


@pytest.mark.parametrize("knobs", [{"PMA_CHUNK": "3"}, {"PMA_CHUNK": "3", "PMA_FUSE_OUT": "0"},
                                   {"PMA_CHUNK": "3", "PMA_FUSE_IN": "0"},
                                   {"PMA_PERSIST": "1"}, {"PMA_COMPACT": "0"},
                                   {"PMA_XCD_MAP": "0"}],
                         ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_mask_split_targets_and_knobs(knobs, dt, monkeypatch):
    # A hub target split into pieces, some of them entirely masked.
    for k, v in knobs.items():
        monkeypatch.setenv(k, v)
    c = synth.random_case(76, 4, 150, 150, 64, 4, 0.03, dtype=dt, name="mask_split")
    keep = c.tgt != 5
    c.src = np.concatenate([c.src[keep], np.arange(0, 120)])
    c.tgt = np.concatenate([c.tgt[keep], np.full(120, 5)])
    kpm = np.random.default_rng(77).random((c.B, c.S)) < 0.3
    kpm[1, :60] = True                                           # leading pieces of the hub
    kpm[3, :120] = True                                          # the whole hub
    _check(c, kpm, need_weights=True, average=True)


# Rows of 3 chunks (3 heads of one 16-byte chunk each): wavefronts cover
# 21-22 samples starting mid-row, so above 32 samples some wavefronts hold
# samples on both sides of a multiple of 32 and need both mask words of an
# edge (B = 64 and B = 70 both have such wavefronts).
@pytest.mark.parametrize("shape", [("bf16", 24, 3), ("f32", 12, 3)],
                         ids=lambda s: f"{s[0]}_E{s[1]}_H{s[2]}")
@pytest.mark.parametrize("B", [64, 70])
@pytest.mark.parametrize("need_weights", [False, True])
def test_mask_rows_of_three_chunks(shape, B, need_weights):
    dt, E, H = shape
    c = synth.random_case(90 + B, B, 60, 60, E, H, 0.1, dtype=dt, name="mask_cpr3")
    kpm = np.random.default_rng(91).random((c.B, c.S)) < 0.3
    kpm[40] = True                                               # a fully masked sample past 32
    _check(c, kpm, need_weights=need_weights, average=False)


def test_mask_rejects():
    import torch
    c = synth.random_case(78, 2, 20, 20, 8, 2, 0.2, name="mask_bad")
    dev = synth.to_torch(c)
    plan = pma.pma_create(c.src, c.tgt, c.L, c.S, c.E, c.H)
    try:
        args = (plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["bq"], dev["wk"], dev["bk"],
                dev["wv"], dev["bv"], dev["wo"], dev["bo"])
        with pytest.raises(pma.PmaError):
            pma.pma_forward(*args, key_padding_mask=torch.zeros(c.S + 1, dtype=torch.bool,
                                                                device="cuda"))
        with pytest.raises(pma.PmaError):
            pma.pma_forward(*args, key_padding_mask=torch.zeros(c.S, dtype=torch.float32,
                                                                device="cuda"))
        lib = pma._load()
        st = lib.pma_forward_masked(plan.handle, c.B, dev["xq"].data_ptr(), dev["xk"].data_ptr(),
                                    dev["xv"].data_ptr(), dev["wq"].data_ptr(), None,
                                    dev["wk"].data_ptr(), None, dev["wv"].data_ptr(), None,
                                    dev["wo"].data_ptr(), None, dev["xq"].data_ptr(), None, 1,
                                    None, 1, None)
        assert pma.STATUS[st] == "PMA_E_NULL"
    finally:
        pma.pma_destroy(plan)


@pytest.mark.parametrize("name", ["gene", "bipartite", "large"])
def test_mask_full_size(name):
    # every output element and every per-edge weight, a quarter of the keys
    # masked per sample
    c = synth.make_config(name)
    kpm = np.random.default_rng(79).random((c.B, c.S)) < 0.25
    print(f"[mask] full {name}", flush=True)
    out, w, plan = run(c, kpm=kpm)
    try:
        src, tgt = pma.pma_edges(plan)
    finally:
        pma.pma_destroy(plan)
    ref = oracle.case_forward(c, want_weights=c.need_weights, key_padding_mask=kpm)
    err = max_abs_rel(out, ref["out"])
    record(f"masked forward {name}", "out", err, TOL[c.dtype])
    assert err <= TOL[c.dtype], err
    live = _live(kpm, src, tgt, c.B, c.L)
    bo = oracle.widen(c.params["bo"], c.dtype)
    assert (out[~live] == bo).all()
    if c.need_weights:
        rw = oracle.average_heads(ref["weights"])
        werr = max_abs_rel(w, rw)
        record(f"masked forward {name}", "weights", werr, TOL[c.dtype])
        assert werr <= TOL[c.dtype], werr
        assert (w[kpm[:, src]] == 0).all()                       # masked: weight 0
