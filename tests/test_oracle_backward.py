"""Pins for the gradient oracle (oracle/backward.py), CPU only.

The gradients come from torch autograd over a plain float64 forward. They are
tied to things other than that code: the C oracle's forward (same values),
central finite differences of the C oracle's forward, and torch's own
nn.MultiheadAttention autograd on graph-masked dense attention. A planted
mistake in a copy of the gradient oracle must fail a pin.
"""
import importlib.util
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob
from graph_sparse_head_amd import synth


def _case(seed, mask=False, loops=False, shared="none"):
    rng = np.random.default_rng(9000 + seed)
    H = int(rng.choice([1, 2, 4]))
    E = H * int(rng.choice([1, 2, 3]))
    L = int(rng.integers(2, 9))
    S = L if (shared != "none" or loops or rng.random() < 0.5) else int(rng.integers(2, 9))
    B = int(rng.integers(1, 3))
    src, tgt = synth.random_graph(rng, L, S, float(rng.uniform(0.2, 0.7)))
    if src.size == 0:
        src, tgt = np.array([0], np.int64), np.array([0], np.int64)
    src, tgt = oracle.prepare_edges(src, tgt, L, S, E, H, loops)
    params = {}
    bias = bool(rng.random() < 0.8)
    for n in "qkvo":
        params["w" + n] = rng.uniform(-0.6, 0.6, (E, E))
        params["b" + n] = rng.normal(0, 0.2, E) if bias else None
    xq = rng.standard_normal((B, L, E))
    xk = xq if shared == "qkv" else rng.standard_normal((B, S, E))
    xv = xk if shared in ("qkv", "kv") else rng.standard_normal((B, S, E))
    kpm = (rng.random((B, S)) < 0.3) if mask else None
    G = rng.standard_normal((B, L, E))
    return B, L, S, E, H, params, xq, xk, xv, src, tgt, kpm, G


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("mask", [False, True])
def test_torch_forward_equals_c_oracle(seed, mask):
    B, L, S, E, H, params, xq, xk, xv, src, tgt, kpm, G = _case(seed, mask)
    P = {k: None if v is None else torch.from_numpy(v) for k, v in params.items()}
    out, w = ob.forward_torch(E, H, torch.from_numpy(xq), torch.from_numpy(xk), torch.from_numpy(xv),
                              P, src, tgt, kpm, L)
    ref = oracle.forward(B, L, S, E, H, xq, xk, xv, params, src, tgt, want_weights=True,
                         key_padding_mask=kpm)
    np.testing.assert_allclose(out.numpy(), ref["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(w.numpy(), ref["weights"], rtol=0, atol=1e-12)


def _c_objective(B, L, S, E, H, params, xq, xk, xv, src, tgt, kpm, G):
    out = oracle.forward(B, L, S, E, H, xq, xk, xv, params, src, tgt, key_padding_mask=kpm)["out"]
    return float((out * G).sum())


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("mask", [False, True])
def test_gradients_match_finite_differences_of_c_oracle(seed, mask):
    B, L, S, E, H, params, xq, xk, xv, src, tgt, kpm, G = _case(seed, mask)
    g = ob.gradients(B, L, S, E, H, xq, xk, xv, params, src, tgt, G, kpm)
    rng = np.random.default_rng(seed)
    h = 1e-6
    arrays = {"query": xq, "key": xk, "value": xv}
    arrays.update({k: v for k, v in params.items() if v is not None})
    for name, arr in arrays.items():
        for _ in range(4):
            i = tuple(int(rng.integers(0, n)) for n in arr.shape)
            old = arr[i]
            arr[i] = old + h
            fp = _c_objective(B, L, S, E, H, params, xq, xk, xv, src, tgt, kpm, G)
            arr[i] = old - h
            fm = _c_objective(B, L, S, E, H, params, xq, xk, xv, src, tgt, kpm, G)
            arr[i] = old
            fd = (fp - fm) / (2 * h)
            assert abs(fd - g[name][i]) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, g[name][i])


@pytest.mark.parametrize("seed", range(12))
def test_gradients_match_torch_mha_autograd(seed):
    # self-loops give every target a source, so dense masked MHA has no NaN rows
    B, L, S, E, H, params, xq, xk, xv, src, tgt, kpm, G = _case(seed, loops=True)
    g = ob.gradients(B, L, S, E, H, xq, xk, xv, params, src, tgt, G)
    bias = params["bq"] is not None
    mha = torch.nn.MultiheadAttention(E, H, bias=bias, batch_first=True).double()
    with torch.no_grad():
        mha.in_proj_weight.copy_(torch.from_numpy(np.concatenate([params["wq"], params["wk"],
                                                                  params["wv"]])))
        mha.out_proj.weight.copy_(torch.from_numpy(params["wo"]))
        if bias:
            mha.in_proj_bias.copy_(torch.from_numpy(np.concatenate([params["bq"], params["bk"],
                                                                    params["bv"]])))
            mha.out_proj.bias.copy_(torch.from_numpy(params["bo"]))
    mha.train(False)
    allowed = np.zeros((L, S), bool)
    allowed[tgt, src] = True
    q = torch.from_numpy(xq).requires_grad_(True)
    k = torch.from_numpy(xk).requires_grad_(True)
    v = torch.from_numpy(xv).requires_grad_(True)
    out, _ = mha(q, k, v, attn_mask=torch.from_numpy(~allowed), need_weights=False)
    (out * torch.from_numpy(G)).sum().backward()
    tol = dict(rtol=0, atol=1e-10)
    np.testing.assert_allclose(g["query"], q.grad.numpy(), **tol)
    np.testing.assert_allclose(g["key"], k.grad.numpy(), **tol)
    np.testing.assert_allclose(g["value"], v.grad.numpy(), **tol)
    wg = mha.in_proj_weight.grad.numpy()
    np.testing.assert_allclose(g["wq"], wg[:E], **tol)
    np.testing.assert_allclose(g["wk"], wg[E:2 * E], **tol)
    np.testing.assert_allclose(g["wv"], wg[2 * E:], **tol)
    np.testing.assert_allclose(g["wo"], mha.out_proj.weight.grad.numpy(), **tol)
    if bias:
        bg = mha.in_proj_bias.grad.numpy()
        np.testing.assert_allclose(g["bq"], bg[:E], **tol)
        np.testing.assert_allclose(g["bk"], bg[E:2 * E], **tol)
        np.testing.assert_allclose(g["bv"], bg[2 * E:], **tol)
        np.testing.assert_allclose(g["bo"], mha.out_proj.bias.grad.numpy(), **tol)


@pytest.mark.parametrize("shared", ["kv", "qkv"])
def test_shared_tensor_gets_sum_of_uses(shared):
    B, L, S, E, H, params, xq, xk, xv, src, tgt, kpm, G = _case(4, shared=shared)
    g = ob.gradients(B, L, S, E, H, xq, xk, xv, params, src, tgt, G, shared=shared)
    sep = ob.gradients(B, L, S, E, H, xq.copy(), xk.copy(), xv.copy(), params, src, tgt, G)
    want = sep["key"] + sep["value"] + (sep["query"] if shared == "qkv" else 0)
    np.testing.assert_allclose(g["key"], want, rtol=0, atol=1e-12)
    assert np.array_equal(g["key"], g["value"])


def test_masked_keys_and_empty_targets_get_no_gradient():
    B, L, S, E, H, params, xq, xk, xv, src, tgt, kpm, G = _case(5, mask=True)
    g = ob.gradients(B, L, S, E, H, xq, xk, xv, params, src, tgt, G, kpm)
    # a key that no sample reads unmasked gets zero key / value gradient
    for b in range(B):
        read = np.zeros(S, bool)
        read[src[~kpm[b, src]]] = True
        assert (g["key"][b][~read] == 0).all() and (g["value"][b][~read] == 0).all()


def test_planted_mistake_fails_a_pin(tmp_path, monkeypatch):
    text = open(ob.__file__).read()
    old = "score = (q[:, tgt] * k[:, src]).sum(-1) / math.sqrt(d)"
    assert old in text
    path = tmp_path / "bad_backward.py"
    path.write_text(text.replace(old, "score = (q[:, tgt] * k[:, src]).sum(-1) / d"))
    spec = importlib.util.spec_from_file_location("bad_backward", path)
    bad = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bad)
    monkeypatch.setattr(ob, "gradients", bad.gradients)
    monkeypatch.setattr(ob, "forward_torch", bad.forward_torch)
    failures = 0
    for seed in range(6):
        try:
            test_gradients_match_torch_mha_autograd(seed)
        except AssertionError:
            failures += 1
    assert failures > 0
