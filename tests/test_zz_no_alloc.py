"""The allocation-free forward (pma_forward_static, include/pma.h) against
pma_forward: the same kernels on a workspace carved from the library's
static scratch instead of the plan's, so the results must be identical bit
for bit, and within the oracle's tolerance. Each case makes two calls in a
row on one plan, the second with fewer samples, since every call reuses
(and leaves its data in) the same scratch."""
import numpy as np
import pytest
import torch

import graph_sparse_head_amd as pma
import oracle
from graph_sparse_head_amd import synth
from gpu_helpers import TOL, max_abs_rel, record, to_f64

pytestmark = pytest.mark.gpu


def _args(dev, b):
    """The case's tensors restricted to the first b samples (views of one
    token tensor stay one tensor)."""
    q = dev["xq"][:b]
    k = q if dev["xk"] is dev["xq"] else dev["xk"][:b]
    v = k if dev["xv"] is dev["xk"] else (q if dev["xv"] is dev["xq"] else dev["xv"][:b])
    return (q, k, v, dev["wq"], dev["bq"], dev["wk"], dev["bk"], dev["wv"], dev["bv"],
            dev["wo"], dev["bo"])


def _sub(case, b):
    """The case with its first b samples (for the oracle)."""
    c = synth.Case(case.name, b, case.L, case.S, case.E, case.H, case.dtype, case.src, case.tgt,
                   case.add_self_loops, case.need_weights, case.average, case.xq[:b],
                   case.xq[:b] if case.xk is case.xq else case.xk[:b],
                   case.xq[:b] if case.xv is case.xq else
                   (case.xk[:b] if case.xv is case.xk else case.xv[:b]), case.params)
    return c


def _static_vs_forward(case, batches, need_weights, average=True, oracle_check=True):
    dev = synth.to_torch(case)
    plan = pma.pma_create(case.src, case.tgt, case.L, case.S, case.E, case.H,
                          add_self_loops=case.add_self_loops, dtype=case.dtype)
    try:
        for b in batches:
            print(f"[static] {case.name} B={b} E={case.E} H={case.H} {case.dtype} "
                  f"w={need_weights}", flush=True)
            a = _args(dev, b)
            o1, w1 = pma.pma_forward_static(plan, *a, need_weights=need_weights,
                                            average_attn_weights=average)
            o2, w2 = pma.pma_forward(plan, *a, need_weights=need_weights,
                                     average_attn_weights=average)
            torch.cuda.synchronize()
            assert torch.equal(o1.view(torch.int16) if o1.dtype == torch.bfloat16 else o1,
                               o2.view(torch.int16) if o2.dtype == torch.bfloat16 else o2)
            if need_weights:
                assert torch.equal(w1, w2)
            if oracle_check:
                ref = oracle.case_forward(_sub(case, b), want_weights=need_weights)
                err = max_abs_rel(to_f64(o1, case.dtype).reshape(b, case.L, case.E), ref["out"])
                record(f"static forward {case.name} B={b}", "out", err, TOL[case.dtype])
                assert err <= TOL[case.dtype], err
                if need_weights:
                    rw = ref["weights"]
                    rw = oracle.average_heads(rw) if average else rw
                    werr = max_abs_rel(w1.cpu().numpy().astype(np.float64), rw)
                    assert werr <= TOL[case.dtype], werr
    finally:
        pma.pma_destroy(plan)


def test_static_forward_bf16_fused_split_targets(monkeypatch):
    # E = 64 bf16: q projection and out_proj inside the edge kernel; short
    # pieces (PMA_CHUNK) so that targets are split and merged
    monkeypatch.setenv("PMA_CHUNK", "7")
    c = synth.random_case(200, 9, 300, 300, 64, 4, 0.05, dtype="bf16", name="static_bf16")
    _static_vs_forward(c, [9, 5], need_weights=False)


def test_static_forward_f32_weights_per_head():
    # fp32, E = 128: separate projections and out_proj, scores and
    # statistics in the scratch for need_weights
    c = synth.random_case(201, 6, 120, 260, 128, 8, 0.04, dtype="f32", same_kv=True,
                          same_qkv=False, name="static_f32")
    _static_vs_forward(c, [6, 2], need_weights=True, average=False)


def test_static_forward_generic_head_size():
    c = synth.random_case(202, 4, 90, 90, 48, 4, 0.06, dtype="f32", name="static_generic")
    _static_vs_forward(c, [4, 3], need_weights=True)


def test_static_forward_gene_workload():
    # the 20,000-node gene workload at its full batch (about 67 MB of
    # workspace), then half the batch
    c = synth.gene()
    _static_vs_forward(c, [32, 16], need_weights=False, oracle_check=False)


def test_static_forward_refuses_a_workspace_beyond_the_scratch():
    c = synth.bipartite()                      # keys and values alone are 328 MB
    dev = synth.to_torch(c)
    plan = pma.pma_create(c.src, c.tgt, c.L, c.S, c.E, c.H, dtype=c.dtype)
    try:
        out = torch.full((c.B, c.L, c.E), 7.0, device="cuda")
        with pytest.raises(pma.PmaError) as e:
            pma.pma_forward_static(plan, *_args(dev, c.B), out=out)
        assert e.value.name == "PMA_E_SIZE" and "static scratch" in str(e.value)
        torch.cuda.synchronize()
        assert (out == 7.0).all()                 # nothing was launched
        # a smaller batch of the same graph fits and matches pma_forward
        o1, _ = pma.pma_forward_static(plan, *_args(dev, 1))
        o2, _ = pma.pma_forward(plan, *_args(dev, 1))
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
    finally:
        pma.pma_destroy(plan)


# The reason for the entry point: it can be captured in a HIP graph
# (torch.cuda.CUDAGraph) and replayed. Each replay follows eager work of the
# program (new tokens copied into the captured inputs, synchronisation), and
# its output must equal an eager pma_forward on the same inputs bit for bit.
@pytest.mark.parametrize("case", ["bf16_fused_split", "f32_weights", "complete"])
def test_static_forward_replayed_from_a_graph(case, monkeypatch):
    if case == "bf16_fused_split":
        monkeypatch.setenv("PMA_CHUNK", "7")
        c = synth.random_case(210, 8, 200, 200, 64, 4, 0.05, dtype="bf16", name=case)
        nw = False
    elif case == "f32_weights":
        c = synth.random_case(211, 4, 90, 150, 128, 8, 0.05, dtype="f32", same_kv=True,
                              same_qkv=False, name=case)
        nw = True
    else:
        c = synth.complete()
        nw = True
    print(f"[graph] {case}", flush=True)
    dev = synth.to_torch(c)
    plan = pma.pma_create(c.src, c.tgt, c.L, c.S, c.E, c.H, add_self_loops=c.add_self_loops,
                          dtype=c.dtype)
    try:
        args = [dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["bq"], dev["wk"], dev["bk"],
                dev["wv"], dev["bv"], dev["wo"], dev["bo"]]
        out = torch.empty(c.B, c.L, c.E, dtype=dev["xq"].dtype, device="cuda")
        w = torch.empty(c.B, plan.nnz, dtype=torch.float32, device="cuda") if nw else None
        pma.pma_forward_static(plan, *args, out=out, weights=w)      # first use on the device
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                pma.pma_forward_static(plan, *args, out=out, weights=w)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gen = torch.Generator(device="cpu").manual_seed(7)
        for r in range(4):
            # new tokens in the captured input tensors (eager work between replays)
            for t in {id(x): x for x in args[:3]}.values():
                t.copy_(torch.randn(t.shape, generator=gen).to(t.dtype))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ref_out, ref_w = pma.pma_forward(plan, *args, need_weights=nw)
            torch.cuda.synchronize()
            a = out.view(torch.int16) if out.dtype == torch.bfloat16 else out
            b = ref_out.view(torch.int16) if ref_out.dtype == torch.bfloat16 else ref_out
            assert torch.equal(a, b), (case, r)
            if nw:
                assert torch.equal(w, ref_w), (case, r)
        del g
    finally:
        pma.pma_destroy(plan)
