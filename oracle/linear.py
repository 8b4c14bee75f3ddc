"""PackedLinear on packed pairs, in float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): only the tests, the smoke
check and the bench's CPU-baseline leg use it. It shares no code with the GPU
library.

Reading of the kpnn2 PackedMultiheadAttention page, "See also" (PackedLinear:
the same packed pairs with one trained weight per edge, the same for every
sample) together with its opening paragraphs (information flows along an
edge from source to target, as in PackedLinear): a linear map from the S
source features to the L target features whose weight matrix is w_e at each
live pair (t_e, s_e) and zero elsewhere, applied to every sample b and
channel c:

    y[b, t, c] = bias[t] + sum over edges e with t_e = t of w_e x[b, s_e, c].

The page prints no formula or example for it; the pins in
tests/test_oracle_linear.py tie this code to the dense masked product (the
page's MaskedLinear: a dense (out, in) weight), to a hand-worked case, to
finite differences and to torch autograd.
"""
from __future__ import annotations

import numpy as np


def forward(x, w, bias, src, tgt, L: int):
    """x (B, S, C), w (nnz,), bias (L,) or None, src / tgt (nnz,) int;
    returns y (B, L, C) float64. Each edge adds its weighted source row to
    its target row, edges taken in the given order."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    B, S, C = x.shape
    y = np.zeros((B, L, C))
    if bias is not None:
        y += np.asarray(bias, np.float64)[None, :, None]
    for e in range(len(src)):
        y[:, tgt[e], :] += w[e] * x[:, src[e], :]
    return y


def gradients(x, w, src, tgt, L: int, grad_out):
    """Gradients of sum(y * grad_out): (dx (B, S, C), dw (nnz,), dbias (L,)).
    dx[b, s] gathers w_e dy[b, t_e] over the edges leaving s; dw_e is the
    sample-and-channel sum of dy[b, t_e] x[b, s_e]; dbias[t] sums dy[b, t]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    g = np.asarray(grad_out, np.float64)
    dx = np.zeros_like(x)
    dw = np.zeros(len(src))
    for e in range(len(src)):
        dx[:, src[e], :] += w[e] * g[:, tgt[e], :]
        dw[e] = np.sum(g[:, tgt[e], :] * x[:, src[e], :])
    db = g.sum(axis=(0, 2))
    return dx, dw, db
