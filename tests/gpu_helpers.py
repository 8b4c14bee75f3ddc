"""Shared pieces of the GPU parity tests: run a synthetic case through the
C-ABI and compare with the oracle."""
import numpy as np

import graph_sparse_head_amd as pma
import oracle
from graph_sparse_head_amd import synth

TOL = {"f32": 1e-5, "bf16": 2e-2}


def record(name, tensor, err, tol):
    """Keep a parity figure for the terminal summary (tests/conftest.py)."""
    from parity_log import PARITY
    PARITY.append((name, tensor, float(err), float(tol)))


def max_abs_rel(got, ref):
    """max |got - ref| / max |ref| over the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def to_f64(t, dtype):
    """A torch tensor of the case dtype, back on the host as float64."""
    import torch
    if t.dtype == torch.bfloat16:
        return oracle.widen(t.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    return t.detach().cpu().numpy().astype(np.float64)


def make_plan(case, stream=None):
    return pma.pma_create(case.src, case.tgt, case.L, case.S, case.E, case.H,
                          add_self_loops=case.add_self_loops, dtype=case.dtype, stream=stream)


def run(case, plan=None, need_weights=None, average=None, dev=None, lead=None, kpm=None):
    """One forward on the GPU. Returns (out float64 (B, L, E), weights float64
    or None, plan). ``lead`` reshapes the batch into several leading axes;
    ``kpm`` is a numpy boolean key_padding_mask, (S,) or (B, S)."""
    import torch
    own = plan is None
    if own:
        plan = make_plan(case)
    if dev is None:
        dev = synth.to_torch(case)
    nw = case.need_weights if need_weights is None else need_weights
    avg = case.average if average is None else average
    q, k, v = dev["xq"], dev["xk"], dev["xv"]
    if lead is not None:
        q = q.reshape(*lead, case.L, case.E)
        k = q if dev["xk"] is dev["xq"] else k.reshape(*lead, case.S, case.E)
        v = k if dev["xv"] is dev["xk"] else v.reshape(*lead, case.S, case.E)
    mask = None
    if kpm is not None:
        mask = torch.from_numpy(np.ascontiguousarray(kpm, np.bool_)).cuda()
        if mask.dim() == 2 and lead is not None:
            mask = mask.reshape(*lead, case.S)
    out, w = pma.pma_forward(plan, q, k, v, dev["wq"], dev["bq"], dev["wk"], dev["bk"],
                             dev["wv"], dev["bv"], dev["wo"], dev["bo"],
                             need_weights=nw, average_attn_weights=avg, key_padding_mask=mask)
    torch.cuda.synchronize()
    o = to_f64(out, case.dtype).reshape(case.B, case.L, case.E)
    wn = None
    if w is not None:
        wn = w.cpu().numpy().astype(np.float64).reshape(case.B, plan.nnz, *([] if avg else [case.H]))
    return o, wn, plan
