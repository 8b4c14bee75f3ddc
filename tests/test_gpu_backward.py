"""Backward pass on the GPU (pma_forward_train + pma_backward) against the
gradient oracle (oracle/backward.py): gradients of every token tensor and of
the eight projection parameters, for separate, key=value and shared
query/key/value tokens, with and without biases and key_padding_mask."""
import numpy as np
import pytest
import torch

import graph_sparse_head_amd as pma
import oracle
from oracle import backward as ob
from graph_sparse_head_amd import synth
from gpu_helpers import TOL, max_abs_rel, record, to_f64

pytestmark = pytest.mark.gpu

NAMES = ["query", "key", "value", "q_w", "k_w", "v_w", "o_w", "q_b", "k_b", "v_b", "o_b"]
ORACLE = {"q_w": "wq", "k_w": "wk", "v_w": "wv", "o_w": "wo", "q_b": "bq", "k_b": "bk",
          "v_b": "bv", "o_b": "bo"}


def _grad_check(c, shared, kpm=None, rows=None):
    print(f"[backward] {c.name} B={c.B} L={c.L} S={c.S} E={c.E} H={c.H} {c.dtype} "
          f"shared={shared} mask={kpm is not None}", flush=True)
    dev = synth.to_torch(c)
    tdt = torch.float32 if c.dtype == "f32" else torch.bfloat16
    rng = np.random.default_rng(5)
    G = rng.standard_normal((c.B, c.L, c.E)).astype(np.float32)
    if c.dtype == "bf16":
        G = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(G))
    g_dev = torch.from_numpy(G).to(tdt).cuda()
    plan = pma.pma_create(c.src, c.tgt, c.L, c.S, c.E, c.H, add_self_loops=c.add_self_loops,
                          dtype=c.dtype)
    try:
        mask = None if kpm is None else torch.from_numpy(kpm).cuda()
        args = (dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["bq"], dev["wk"], dev["bk"],
                dev["wv"], dev["bv"], dev["wo"], dev["bo"])
        out, _, save = pma.pma_forward_train(plan, *args, key_padding_mask=mask)
        # the training forward computes the same output as the plain one
        out2, _ = pma.pma_forward(plan, *args, key_padding_mask=mask)
        torch.cuda.synchronize()
        assert max_abs_rel(to_f64(out, c.dtype), to_f64(out2, c.dtype)) <= TOL[c.dtype]
        has_bias = dev["bq"] is not None
        gr = pma.pma_backward(plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["wk"],
                              dev["wv"], dev["wo"], has_bias, save, g_dev, key_padding_mask=mask)
        torch.cuda.synchronize()
        src, tgt = oracle.prepare_edges(c.src, c.tgt, c.L, c.S, c.E, c.H, c.add_self_loops)
        params = {k: oracle.widen(v, c.dtype) for k, v in c.params.items()}
        xq = oracle.widen(c.xq, c.dtype)
        xk = xq if shared == "qkv" else oracle.widen(c.xk, c.dtype)
        xv = xk if shared in ("qkv", "kv") else oracle.widen(c.xv, c.dtype)
        ref = ob.gradients(c.B, c.L, c.S, c.E, c.H, xq, xk, xv, params, src, tgt,
                           G.astype(np.float64), kpm, shared=shared)
        for n in NAMES:
            if n.endswith("_b") and not has_bias:
                continue
            got = to_f64(gr[n], c.dtype)
            want = ref[n] if n in ("query", "key", "value") else ref[ORACLE[n]]
            if n == "k_b":
                # Adding one vector to every key shifts all scores into a
                # target equally, which the softmax ignores: the key bias
                # gradient is zero up to rounding, judged on the scale of
                # the key weight gradient (a sum over the same rows).
                assert np.abs(got).max() <= TOL[c.dtype] * np.abs(ref["wk"]).max(), n
                continue
            err = max_abs_rel(got.reshape(want.shape), want)
            assert err <= TOL[c.dtype], (n, err)
    finally:
        pma.pma_destroy(plan)


SHAPES = [("f32", 64, 4), ("f32", 16, 4), ("f32", 24, 2), ("f32", 128, 4), ("bf16", 64, 4),
          ("bf16", 128, 8)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}_E{s[1]}_H{s[2]}")
@pytest.mark.parametrize("shared", ["none", "kv", "qkv"])
def test_backward_random(shape, shared):
    dt, E, H = shape
    L = S = 70
    if shared == "none":
        S = 90
    c = synth.random_case(80, 3, L, S, E, H, 0.07, dtype=dt, same_kv=shared != "none",
                          same_qkv=shared == "qkv", name="bwd")
    _grad_check(c, shared)


# Weight gradients over many rows: with E = 128 one workgroup takes all of
# dW for its row range, here several 128-row slabs (bf16) or 16-row steps
# (fp32) per workgroup with a ragged last one.
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_weight_gradients_many_rows(dt):
    c = synth.random_case(84, 5, 2999, 3001, 128, 8, 0.002, dtype=dt, same_kv=True,
                          same_qkv=False, name="bwd_rows")
    _grad_check(c, "kv")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_mask_no_bias_self_loops(dt):
    c = synth.random_case(81, 4, 60, 60, 64, 4, 0.08, dtype=dt, bias="none", add_self_loops=True,
                          name="bwd_mask")
    kpm = np.random.default_rng(82).random((c.B, c.S)) < 0.35
    kpm[1] = True                                    # one sample entirely masked
    _grad_check(c, "qkv", kpm=kpm)


# Rows of 3 chunks per sample (3 heads of one 16-byte chunk): at B = 64 the
# target pass's wavefronts hold 21-22 samples that straddle multiples of 32
# (mask bits must then be looked up per lane), and the sample-group orders
# must map lanes to (sample, chunk) although 3 does not divide 64.
@pytest.mark.parametrize("shape", [("bf16", 24, 3), ("f32", 12, 3)],
                         ids=lambda s: f"{s[0]}_E{s[1]}_H{s[2]}")
@pytest.mark.parametrize("B", [64, 70])
@pytest.mark.parametrize("order", ["auto", "0", "1", "2"])
def test_backward_mask_rows_of_three_chunks(shape, B, order, monkeypatch):
    if order != "auto":
        monkeypatch.setenv("PMA_BWD_ORDER", order)
    dt, E, H = shape
    c = synth.random_case(92 + B, B, 40, 40, E, H, 0.12, dtype=dt, name="bwd_mask_cpr3")
    kpm = np.random.default_rng(93).random((c.B, c.S)) < 0.3
    kpm[40] = True
    _grad_check(c, "qkv", kpm=kpm)


def test_backward_hub_and_empty_targets():
    c = synth.random_case(83, 2, 150, 150, 32, 2, 0.02, name="bwd_hub")
    keep = c.tgt != 7
    c.src = np.concatenate([c.src[keep], np.arange(140)])
    c.tgt = np.concatenate([c.tgt[keep], np.full(140, 7)])
    _grad_check(c, "qkv")


def test_backward_rejects():
    c = synth.random_case(84, 2, 20, 30, 8, 2, 0.2, same_kv=True, name="bwd_bad")
    dev = synth.to_torch(c)
    plan = pma.pma_create(c.src, c.tgt, c.L, c.S, c.E, c.H)
    try:
        lib = pma._load()
        z = dev["xq"].data_ptr()
        st = lib.pma_backward(plan.handle, c.B, z, z, z, z, z, z, z, 0, None, z, None, 0, z, z, z,
                              z, None, z, None, z, None, z, None, None)
        assert pma.STATUS[st] == "PMA_E_NULL"
        st = lib.pma_backward(plan.handle, c.B, z, z, z, z, z, z, z, 2, z, z, None, 0, z, z, z,
                              z, None, z, None, z, None, z, None, None)
        assert pma.STATUS[st] == "PMA_E_ARG"
        # a key gradient shared with the query's needs L == S
        st = lib.pma_backward(plan.handle, c.B, z, z, z, z, z, z, z, 0, z, z, None, 0, z, z, z,
                              z, None, z, None, z, None, z, None, None)
        assert pma.STATUS[st] == "PMA_E_ARG"
        assert lib.pma_train_bytes(None, 4) == 0 and lib.pma_train_bytes(plan.handle, 0) == 0
    finally:
        pma.pma_destroy(plan)


# PMA_CHUNK=3 cuts every target and source with more than three edges into
# pieces, so the partial sums and their merge carry most of the result.
@pytest.mark.parametrize("shape", [("f32", 64, 4), ("bf16", 64, 4), ("f32", 128, 8),
                                   ("bf16", 128, 8), ("f32", 16, 4)],
                         ids=lambda s: f"{s[0]}_E{s[1]}_H{s[2]}")
@pytest.mark.parametrize("shared", ["none", "kv", "qkv"])
def test_backward_pieces(shape, shared, monkeypatch):
    monkeypatch.setenv("PMA_CHUNK", "3")
    dt, E, H = shape
    L = S = 64
    if shared == "none":
        S = 80
    c = synth.random_case(85, 3, L, S, E, H, 0.12, dtype=dt, same_kv=shared != "none",
                          same_qkv=shared == "qkv", name="bwd_pieces")
    _grad_check(c, shared)


@pytest.mark.parametrize("chunk", [None, "16"])
def test_backward_hub_source(chunk, monkeypatch):
    # source 7 feeds 140 of the 150 targets
    if chunk:
        monkeypatch.setenv("PMA_CHUNK", chunk)
    c = synth.random_case(86, 2, 150, 150, 64, 4, 0.02, name="bwd_hub_src")
    keep = c.src != 7
    c.src = np.concatenate([c.src[keep], np.full(140, 7)])
    c.tgt = np.concatenate([c.tgt[keep], np.arange(140)])
    _grad_check(c, "qkv")


# Hub sources (70-280 targets each) are cut at eight target bands, one per
# XCD; the band's pieces run with their sample groups interleaved (default)
# or one group after another (PMA_BWD_SORDER=2), with short pieces too.
@pytest.mark.parametrize("order", ["0", "2"])
@pytest.mark.parametrize("chunk", ["auto", "32"])
@pytest.mark.parametrize("shape", [("bf16", 128, 8, 8), ("f32", 128, 8, 8), ("bf16", 64, 4, 16)],
                         ids=lambda s: f"{s[0]}_E{s[1]}_B{s[3]}")
def test_backward_banded_source_order(order, chunk, shape, monkeypatch):
    monkeypatch.setenv("PMA_BWD_SORDER", order)
    if chunk != "auto":
        monkeypatch.setenv("PMA_BWD_CHUNK", chunk)
    dt, E, H, B = shape
    c = synth.random_case(89, B, 300, 200, E, H, 0.01, dtype=dt, same_kv=False,
                          name="bwd_bands")
    rng = np.random.default_rng(90)
    hubs = [3, 11, 50, 120]
    keep = ~np.isin(c.src, hubs)
    src, tgt = [c.src[keep]], [c.tgt[keep]]
    for h, n in zip(hubs, (70, 140, 210, 280)):
        src.append(np.full(n, h))
        tgt.append(rng.choice(c.L, size=n, replace=False))
    c.src, c.tgt = np.concatenate(src), np.concatenate(tgt)
    _grad_check(c, "none")


def test_backward_masked_pieces(monkeypatch):
    monkeypatch.setenv("PMA_CHUNK", "4")
    c = synth.random_case(87, 5, 50, 50, 64, 4, 0.15, dtype="bf16", name="bwd_mask_pieces")
    kpm = np.random.default_rng(88).random((c.B, c.S)) < 0.3
    _grad_check(c, "qkv", kpm=kpm)


@pytest.mark.parametrize("cfg", ["gene", "bipartite"])
def test_backward_full_graph_small_batch(cfg):
    # the full-size graphs (hub sources feeding thousands of targets, split
    # targets) at a batch the float64 gradient oracle finishes in seconds
    c = synth.gene(B=2) if cfg == "gene" else synth.bipartite(B=1)
    _grad_check(c, "qkv" if cfg == "gene" else "kv")


@pytest.mark.parametrize("compact", ["0", "1"])
@pytest.mark.parametrize("shared", ["none", "qkv"])
@pytest.mark.parametrize("mask", [False, True])
def test_backward_read_sources_only(compact, shared, mask, monkeypatch):
    # half of the sources are never read: with PMA_COMPACT=1 the training
    # forward saves keys and values for the read ones only (the mask still
    # refers to the original sources)
    monkeypatch.setenv("PMA_COMPACT", compact)
    c = synth.random_case(89, 3, 60, 60, 64, 4, 0.1, dtype="bf16", same_kv=shared != "none",
                          same_qkv=shared == "qkv", name="bwd_compact")
    keep = c.src % 2 == 0
    c.src, c.tgt = c.src[keep], c.tgt[keep]
    kpm = (np.random.default_rng(91).random((c.B, c.S)) < 0.3) if mask else None
    _grad_check(c, shared, kpm=kpm)


# The target pass over sample groups of 64 lanes: interleaved (0), groups
# pinned to XCDs (1) or groups in turn (2). bf16 E = 64 has 8 samples per
# group: B = 16, 32, 64 give 2, 4 and 8 groups; B = 128 gives 16, which do not
# divide the 8 XCDs (order 1 then falls back to 0); fp32 E = 128 with B = 6
# gives 3 groups.
@pytest.mark.parametrize("order", ["0", "1", "2"])
@pytest.mark.parametrize("shape", [("bf16", 64, 4, 16), ("bf16", 64, 4, 32), ("bf16", 64, 4, 64),
                                   ("bf16", 64, 4, 128), ("f32", 128, 8, 6)],
                         ids=lambda s: f"{s[0]}_E{s[1]}_B{s[3]}")
def test_backward_target_pass_order(order, shape, monkeypatch):
    monkeypatch.setenv("PMA_BWD_ORDER", order)
    monkeypatch.setenv("PMA_CHUNK", "5")   # split targets too
    dt, E, H, B = shape
    c = synth.random_case(97, B, 70, 70, E, H, 0.08, dtype=dt, same_kv=False, name="bwd_order")
    _grad_check(c, "none")


# The target pass with each step's rows loaded when they are used
# (PMA_BWD_PF=0) instead of one step ahead: unsplit and split targets
# (ragged last steps), masks with uniform words and per-lane bits.
@pytest.mark.parametrize("shape", [("bf16", 64, 4, 16), ("bf16", 128, 8, 8), ("f32", 128, 8, 6),
                                   ("f32", 64, 4, 4), ("bf16", 8, 1, 64)],
                         ids=lambda s: f"{s[0]}_E{s[1]}_B{s[3]}")
@pytest.mark.parametrize("chunk", ["auto", "5"])
@pytest.mark.parametrize("mask", [False, True])
def test_backward_target_pass_without_prefetch(shape, chunk, mask, monkeypatch):
    monkeypatch.setenv("PMA_BWD_PF", "0")
    if chunk != "auto":
        monkeypatch.setenv("PMA_CHUNK", chunk)
    dt, E, H, B = shape
    c = synth.random_case(96, B, 70, 70, E, H, 0.08, dtype=dt, same_kv=False, name="bwd_nopf")
    kpm = None
    if mask:
        kpm = np.random.default_rng(95).random((c.B, c.S)) < 0.3
        kpm[1] = True
    _grad_check(c, "none", kpm=kpm)


# Source pieces of the backward's source pass: short pieces (PMA_BWD_CHUNK)
# split most sources, and target bands cut into sub-bands per XCD
# (PMA_BWD_SUB) reorder the pieces; both only change which partial sums the
# merge adds.
@pytest.mark.parametrize("knobs", [{"PMA_BWD_CHUNK": "3"}, {"PMA_BWD_CHUNK": "16"},
                                   {"PMA_BWD_SUB": "2"}, {"PMA_BWD_SUB": "5", "PMA_BWD_CHUNK": "4"},
                                   {"PMA_BWD_PF": "1"}, {"PMA_BWD_NT": "0"},
                                   {"PMA_BWD_NT": "1", "PMA_BWD_PF": "0"}, {"PMA_BWD_NT": "6"}],
                         ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_source_piece_knobs(knobs, dt, monkeypatch):
    for k, v in knobs.items():
        monkeypatch.setenv(k, v)
    c = synth.random_case(94, 8, 90, 110, 128, 8, 0.08, dtype=dt, same_kv=False, name="bwd_knobs")
    _grad_check(c, "none")


# key_padding_mask in the fast target pass: whole wavefronts per piece read
# one mask word per edge (bf16 E = 64 at B = 16: 8 samples per wavefront;
# fp32 E = 128 at B = 8: 2), with split pieces; bf16 E = 8 puts 64 samples on
# a wavefront and looks the bits up per lane.
@pytest.mark.parametrize("shape", [("bf16", 64, 4, 16), ("f32", 128, 8, 8), ("bf16", 8, 1, 64)],
                         ids=lambda s: f"{s[0]}_E{s[1]}_B{s[3]}")
def test_backward_mask_whole_wavefronts(shape, monkeypatch):
    monkeypatch.setenv("PMA_CHUNK", "5")
    dt, E, H, B = shape
    c = synth.random_case(98, B, 60, 60, E, H, 0.1, dtype=dt, same_kv=False, name="bwd_mask_uni")
    kpm = np.random.default_rng(99).random((c.B, c.S)) < 0.3
    kpm[1] = True                                    # one sample entirely masked
    _grad_check(c, "none", kpm=kpm)


def _oracle_per_sample(c, shared, src, tgt, params, xq, xk, xv, G64, samples):
    """The gradient oracle one sample at a time (the loss is a sum over
    samples, each sample's token gradients depend on that sample alone, and
    the shared parameters' gradients are the sum over samples). Returns the
    token gradients of ``samples`` (len(samples), rows, E) and, when every
    sample is covered, the parameter gradients."""
    tok = {n: [] for n in ("query", "key", "value")}
    par = None
    for b in samples:
        r = ob.gradients(1, c.L, c.S, c.E, c.H, xq[b:b + 1], xk[b:b + 1], xv[b:b + 1], params,
                         src, tgt, G64[b:b + 1], shared=shared)
        for n in tok:
            tok[n].append(r[n][0])
        if len(samples) == c.B:
            p = {k: r[k] for k in ORACLE.values() if k in r}
            par = p if par is None else {k: par[k] + p[k] for k in par}
    return {n: np.stack(v) for n, v in tok.items()}, par


def _full_size_check(c, shared, samples=None):
    """The training forward's output over the whole tensor, and every
    gradient element of the given samples (all by default) against the
    oracle; with all samples also every parameter gradient. The out_proj
    gradients are checked over all samples in any case: the bias gradient as
    the column sums of the upstream gradient G, the weight gradient as G^T
    times the forward oracle's mixed rows."""
    g = np.random.default_rng(11)
    samples = list(range(c.B)) if samples is None else list(samples)
    print(f"[backward] full {c.name} B={c.B} nnz={len(c.src)} {c.dtype} samples={samples}",
          flush=True)
    dev = synth.to_torch(c)
    G = g.standard_normal((c.B, c.L, c.E)).astype(np.float32)
    if c.dtype == "bf16":
        G = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(G))
    tdt = torch.float32 if c.dtype == "f32" else torch.bfloat16
    plan = pma.pma_create(c.src, c.tgt, c.L, c.S, c.E, c.H, add_self_loops=c.add_self_loops,
                          dtype=c.dtype)
    try:
        args = (dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["bq"], dev["wk"], dev["bk"],
                dev["wv"], dev["bv"], dev["wo"], dev["bo"])
        out, _, save = pma.pma_forward_train(plan, *args)
        gr = pma.pma_backward(plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["wk"],
                              dev["wv"], dev["wo"], True, save, torch.from_numpy(G).to(tdt).cuda())
        torch.cuda.synchronize()
        out = to_f64(out, c.dtype).reshape(c.B, c.L, c.E)
        got = {n: to_f64(gr[n], c.dtype) for n in NAMES}
    finally:
        pma.pma_destroy(plan)
    del dev
    tol = TOL[c.dtype]
    fwd = oracle.case_forward(c, want_mixed=True)
    err = max_abs_rel(out, fwd["out"])
    record(f"training forward {c.name}", "out", err, tol)
    assert err <= tol, ("out", err)
    src, tgt = fwd["src"], fwd["tgt"]
    G64 = G.astype(np.float64)
    err = max_abs_rel(got["o_b"], G64.sum(axis=(0, 1)))
    record(f"backward {c.name}", "o_b", err, tol)
    assert err <= tol, ("o_b", err)
    dwo = G64.reshape(-1, c.E).T @ fwd["mixed"].reshape(-1, c.E)
    err = max_abs_rel(got["o_w"].reshape(c.E, c.E), dwo)
    record(f"backward {c.name}", "o_w", err, tol)
    assert err <= tol, ("o_w", err)
    del fwd
    params = {k: oracle.widen(v, c.dtype) for k, v in c.params.items()}
    xq = oracle.widen(c.xq, c.dtype)
    xk = xq if shared == "qkv" else oracle.widen(c.xk, c.dtype)
    xv = xk if shared in ("kv", "qkv") else oracle.widen(c.xv, c.dtype)
    tok, par = _oracle_per_sample(c, shared, src, tgt, params, xq, xk, xv, G64, samples)
    rows = {"query": c.L, "key": c.S, "value": c.S}
    for n in ("query", "key", "value"):
        want = tok[n]
        have = got[n].reshape(c.B, rows[n], c.E)[samples]
        err = max_abs_rel(have, want)
        tag = "" if len(samples) == c.B else f" (samples {samples})"
        record(f"backward {c.name}{tag}", n, err, tol)
        assert err <= tol, (n, err)
    if par is not None:
        for n in ("q_w", "k_w", "v_w", "o_w", "q_b", "v_b", "o_b"):
            want = par[ORACLE[n]]
            err = max_abs_rel(got[n].reshape(want.shape), want)
            record(f"backward {c.name}", n, err, tol)
            assert err <= tol, (n, err)
        # the key bias gradient is zero up to rounding (see _grad_check)
        assert np.abs(got["k_b"]).max() <= tol * np.abs(par["wk"]).max()


def test_backward_full_size_gene():
    # The gene workload at its full size and batch (B = 32: four sample
    # groups, split targets, hub sources in the backward's source bands; the
    # training benchmark's launch configuration), with separate key and value
    # tokens so that each gradient tensor has one origin.
    c = synth.gene()
    g = np.random.default_rng(12)
    c.xk = synth._tokens(g, c.xq.shape, c.dtype)
    c.xv = synth._tokens(g, c.xq.shape, c.dtype)
    _full_size_check(c, "none")


def test_backward_full_size_gene_shared_tokens():
    # the same graph and batch with one token tensor (as the bench's training
    # step runs it): each node's gradient sums its query, key and value uses
    _full_size_check(synth.gene(), "qkv")


def test_backward_full_size_bipartite():
    # The bipartite workload at its full size and batch (fp32, B = 16, key =
    # value tokens: the key and value gradients are one tensor's).
    _full_size_check(synth.bipartite(), "kv")


def test_backward_full_size_large():
    # The 100k-node workload at its full size and batch (bf16, B = 8, E =
    # 128, one token tensor, self loops, 5.1M edges). The gradient oracle
    # takes about half a minute per sample of this graph, so the token
    # gradients are compared on two of the eight samples (every element of
    # them); the out_proj gradients over all samples.
    c = synth.large()
    _full_size_check(c, "qkv", samples=[0, c.B - 1])
