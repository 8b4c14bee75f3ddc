"""Pins for the PackedLinear oracle (oracle/linear.py), CPU only.

The oracle's per-edge accumulation is tied to things other than itself: the
dense masked product (a library matmul with the weight scattered into an
(L, S) matrix, the page's MaskedLinear), a case worked by hand, the bias of a
target without edges, central finite differences and torch autograd of the
dense product. A planted mistake in a copy of the oracle must fail a pin.
"""
import importlib.util

import numpy as np
import pytest
import torch

from oracle import linear as ol
from graph_sparse_head_amd import synth


def _case(seed, C=1, bias=True):
    rng = np.random.default_rng(7000 + seed)
    L = int(rng.integers(1, 12))
    S = int(rng.integers(1, 12))
    B = int(rng.integers(1, 4))
    src, tgt = synth.random_graph(rng, L, S, float(rng.uniform(0.1, 0.8)))
    if src.size == 0:
        src, tgt = np.array([0], np.int64), np.array([0], np.int64)
    x = rng.standard_normal((B, S, C))
    w = rng.standard_normal(src.size)
    b = rng.standard_normal(L) if bias else None
    return B, L, S, C, x, w, b, src, tgt


def _dense(w, src, tgt, L, S):
    W = np.zeros((L, S))
    W[tgt, src] = w
    return W


@pytest.mark.parametrize("seed", range(25))
@pytest.mark.parametrize("C", [1, 3])
def test_equals_dense_masked_product(seed, C):
    B, L, S, C, x, w, b, src, tgt = _case(seed, C, bias=seed % 3 != 0)
    y = ol.forward(x, w, b, src, tgt, L)
    W = _dense(w, src, tgt, L, S)
    want = np.matmul(W[None], x) + (0 if b is None else b[None, :, None])
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-12)


def test_worked_example():
    # edges 0 -> 1 (w 2), 2 -> 1 (w -1), 1 -> 0 (w 0.5); node 2 has no source
    x = np.array([[[1.0], [2.0], [3.0]]])
    y = ol.forward(x, [2.0, -1.0, 0.5], [10.0, 20.0, 30.0], [0, 2, 1], [1, 1, 0], 3)
    assert y[0, :, 0].tolist() == [10.0 + 1.0, 20.0 + 2.0 - 3.0, 30.0]


def test_target_without_edges_gets_bias():
    x = np.ones((2, 4, 2))
    y = ol.forward(x, [1.0, 1.0], [5.0, 6.0, 7.0], [0, 3], [0, 0], 3)
    assert (y[:, 1:, :] == np.array([6.0, 7.0])[None, :, None]).all()


@pytest.mark.parametrize("seed", range(10))
def test_gradients_match_finite_differences(seed):
    B, L, S, C, x, w, b, src, tgt = _case(seed, 2)
    G = np.random.default_rng(seed).standard_normal((B, L, C))
    dx, dw, db = ol.gradients(x, w, src, tgt, L, G)

    def f(x_, w_, b_):
        return float((ol.forward(x_, w_, b_, src, tgt, L) * G).sum())
    h = 1e-6
    for arr, grad in ((x, dx), (w, dw), (b, db)):
        for i in np.ndindex(arr.shape):
            old = arr[i]
            arr[i] = old + h
            fp = f(x, w, b)
            arr[i] = old - h
            fm = f(x, w, b)
            arr[i] = old
            assert abs((fp - fm) / (2 * h) - grad[i]) <= 1e-6 * max(1.0, abs(grad[i]))


@pytest.mark.parametrize("seed", range(10))
def test_gradients_match_torch_dense_autograd(seed):
    B, L, S, C, x, w, b, src, tgt = _case(seed, 3)
    G = np.random.default_rng(seed + 50).standard_normal((B, L, C))
    dx, dw, db = ol.gradients(x, w, src, tgt, L, G)
    xt = torch.from_numpy(x).requires_grad_(True)
    Wt = torch.from_numpy(_dense(w, src, tgt, L, S)).requires_grad_(True)
    bt = torch.from_numpy(b).requires_grad_(True)
    y = torch.matmul(Wt, xt) + bt[None, :, None]
    (y * torch.from_numpy(G)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dw, Wt.grad.numpy()[tgt, src], rtol=0, atol=1e-12)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=0, atol=1e-12)


def test_planted_mistake_fails_a_pin(tmp_path, monkeypatch):
    text = open(ol.__file__).read()
    old = "y[:, tgt[e], :] += w[e] * x[:, src[e], :]"
    assert old in text
    path = tmp_path / "bad_linear.py"
    path.write_text(text.replace(old, "y[:, src[e] % L, :] += w[e] * x[:, tgt[e] % S, :]"))
    spec = importlib.util.spec_from_file_location("bad_linear", path)
    bad = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bad)
    monkeypatch.setattr(ol, "forward", bad.forward)
    failures = 0
    for seed in range(8):
        try:
            test_equals_dense_masked_product(seed, 1)
        except (AssertionError, IndexError, NameError):
            failures += 1
    assert failures > 0
