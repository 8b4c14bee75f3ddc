"""Forward throughput of packed multi-head attention over live edges on one GPU.

One step = one pma_forward over one batch: the key/value projection, the
fused edge kernel (q projection, scores, online softmax, mix and out_proj) and
the merge of split targets, on the gene-regulatory-prior workload (n = 20,000
nodes, Zipf 1.5 source hubs, log-normal in-degree of mean 10, B = 32, E = 64,
H = 4, bf16 tokens; softmax, mixing weights and sums in fp32). Inputs are seeded synthetic tensors
already resident in HBM when the timed region starts.

Prints one JSON line. ``value`` is edge-heads per second (nnz * H * B per
forward) over the cold-cache leg: before each step a 1 GiB buffer is
overwritten outside the step's events, so no input is still cached from the
step before; the warm leg (steps back to back) is reported beside it.
``roofline`` rates the edge kernel, timed with HIP events on the forward's own
stream inside the headline leg, against MI355X's 8 TB/s HBM, counting the
launch's compulsory bytes (each input and output byte once); the gather model
(every edge's key and value rows per sample, mostly served by the caches) is
reported under its own key. ``cpu_baseline`` times the plain CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "edge-heads/s fwd (nnz·H·B per sec) + % HBM roofline, 20k-node gene graph"
HBM_PEAK_GBS = 8000.0

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")


def _workload(name: str):
    from graph_sparse_head_amd import synth
    return synth.make_config(name)


def edge_kernel_bytes(B, L, n_kv, nnz, n_tasks, E, s, weights=False, H=1, masked=False):
    """Compulsory HBM bytes of one edge-kernel launch: what the launch must
    move at the least, each byte once. Per (target, sample): its query row in
    (query tokens when the kernel projects q itself, else the projected q)
    and its output row out (out when out_proj is fused, else the mixed row):
    2 E s. Per (read source, sample): its key row and value row, once: 2 E s.
    Per edge its gather index (4 B) and per piece its bounds, target and slot
    (16 B). need_weights adds the stored score of every (edge, sample, head)
    and the (max, sum) of every (target, sample, head), 4 B each. A
    key_padding_mask adds its bits by edge position: one 32-bit word per
    edge and 32 samples."""
    b = B * L * 2 * E * s + B * n_kv * 2 * E * s + 4 * nnz + 16 * n_tasks
    if weights:
        b += 4 * B * nnz * H + 8 * B * L * H
    if masked:
        b += 4 * nnz * ((B + 31) // 32)
    return b


def edge_gather_bytes(B, L, nnz, E, s):
    """The gather model: every edge reads its source's key and value rows for
    every sample (2 E s per edge and sample), plus each target's query row in
    and output row out. Most of these reads are served by the L2 and the
    last-level cache (hub sources repeat), so this counts the bytes the
    vector memory path delivers, not HBM bytes."""
    return B * (L * E * s + nnz * 2 * E * s + L * E * s) + 4 * (L + 1) + 4 * nnz


def _traffic(cfg_name: str):
    """HBM bytes per edge-kernel launch from committed rocprofv3 counters, if
    they were taken for this kernel build and workload."""
    try:
        with open(os.path.join(PROFILES, f"edge_{cfg_name}_traffic.json")) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != cfg_name or t.get("kernel_sha") != _kernel_sha():
        return None
    return t


def _kernel_sha():
    import hashlib
    p = os.path.join(ROOT, "graph_sparse_head_amd", "csrc", "edge.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(oracle, case, src, tgt, params, nthreads, budget_s):
    """Edge-heads/s of whole oracle forwards: as many of the batch's samples
    as fit the budget, repeated until the budget is spent (at least once)."""
    xq1 = oracle.widen(case.xq[:1], case.dtype)
    t0 = time.perf_counter()
    oracle.forward(1, case.L, case.S, case.E, case.H, xq1, xq1, xq1, params, src, tgt,
                   nthreads=nthreads)
    one = time.perf_counter() - t0
    nb = int(max(1, min(case.B, budget_s // max(one, 1e-3))))
    xq = oracle.widen(case.xq[:nb], case.dtype)
    reps, dt = 0, 0.0
    while reps == 0 or dt + dt / reps <= budget_s:
        t0 = time.perf_counter()
        oracle.forward(nb, case.L, case.S, case.E, case.H, xq, xq, xq, params, src, tgt,
                       nthreads=nthreads)
        dt += time.perf_counter() - t0
        reps += 1
    return src.shape[0] * case.H * nb * reps / dt, nb, reps, dt


def cpu_baseline(case, budget_s: float = 12.0):
    """The oracle (fp64) on a bounded sample of the workload, on all host
    threads, and again on one thread for context."""
    import oracle

    src, tgt = oracle.prepare_edges(case.src, case.tgt, case.L, case.S, case.E, case.H,
                                    case.add_self_loops)
    params = {k: oracle.widen(v, case.dtype) for k, v in case.params.items()}
    cores = oracle.num_threads(0)
    v, nb, reps, dt = _oracle_rate(oracle, case, src, tgt, params, 0, budget_s)
    v1, nb1, reps1, dt1 = _oracle_rate(oracle, case, src, tgt, params, 1, budget_s)
    return {"value": v, "unit": "edge-heads/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} whole forward(s) (fp64) of {nb} of {case.B} samples, every "
                      f"target, {dt:.1f} s on {cores} threads",
            "single_thread": {"value": v1, "sample": f"{reps1} x {nb1} samples, {dt1:.1f} s"},
            "cpu": _cpu_model()}


def linear_bytes(B, L, nnz, C, s):
    """Algorithmic bytes of one PackedLinear forward: per sample, gather one
    source row of C channels per edge and write each target row; plus the
    weight, source id and edge-order id of every edge and the row pointers."""
    return B * (nnz * C * s + L * C * s) + nnz * (s + 8) + 4 * (L + 1)


def bench_linear(args):
    """PackedLinear forward (or forward + backward with --train) on the
    workload's graph, batch and dtype, with ``--channels`` channels per node."""
    import torch
    import graph_sparse_head_amd as pma
    from graph_sparse_head_amd import synth
    import oracle
    from oracle import linear as ol

    case = _workload(args.config)
    C = args.channels
    rng = np.random.default_rng(5)
    src, tgt = oracle.prepare_edges(case.src, case.tgt, case.L, case.S, 1, 1, case.add_self_loops)
    nnz = len(src)
    tdt = torch.bfloat16 if case.dtype == "bf16" else torch.float32

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(tdt)
    x = dev(rng.standard_normal((case.B, case.S, C)))
    w = dev(rng.uniform(-1, 1, nnz) / np.sqrt(10.0))
    b = dev(rng.normal(0, 0.1, case.L))
    g = dev(rng.standard_normal((case.B, case.L, C)))
    plan = pma.pma_create_graph(case.src, case.tgt, case.L, case.S,
                                add_self_loops=case.add_self_loops, dtype=case.dtype)
    out = torch.empty(case.B, case.L, C, dtype=tdt, device="cuda")

    def step():
        pma.pma_linear_forward(plan, x, w, b, out=out)
        if args.train:
            pma.pma_linear_backward(plan, x, w, g, has_bias=True)

    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    es = 2 if case.dtype == "bf16" else 4
    nbytes = linear_bytes(case.B, case.L, nnz, C, es)
    res = {
        "metric": "edge-samples/s PackedLinear fwd (nnz·B·C per sec)", "value":
            nnz * case.B * C / (ms * 1e-3), "unit": "edge-samples/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": case.dtype, "data": "synthetic",
        "config": {"workload": f"PackedLinear on the {case.name} graph: L={case.L} S={case.S} "
                               f"nnz={nnz} B={case.B} C={C} {case.dtype}"
                               f"{' train step (forward + backward)' if args.train else ''}",
                   "batch": case.B, "channels": C, "nnz": nnz, "parallelism": "single GPU"},
    }
    if not args.train:
        achieved = nbytes / (ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                           "kernel": "lin_spmm (+ lin_merge), whole call",
                           "bytes_per_launch": nbytes, "avg_launch_us": ms * 1e3}
    pma.pma_destroy(plan)
    if not args.no_cpu_baseline:
        xs = x.float().cpu().numpy().astype(np.float64)
        ws = w.float().cpu().numpy().astype(np.float64)
        bs = b.float().cpu().numpy().astype(np.float64)
        nb = max(1, min(case.B, 4))
        t0, reps = time.perf_counter(), 0
        while reps == 0 or time.perf_counter() - t0 < 10.0:
            ol.forward(xs[:nb], ws, bs, src, tgt, case.L)
            reps += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": nnz * nb * C * reps / dt, "unit": "edge-samples/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{reps} forward(s) (fp64) of {nb} of {case.B} samples, "
                                         f"{dt:.1f} s, numpy on one thread"}
    print(json.dumps(res), flush=True)


# Table sizes of the gather-ceiling calibration: within one CU's 32 KB L1,
# within one XCD's 4 MB L2, within the 256 MB last-level cache, and far past it.
CEILING_TABLES = (("L1", 16 << 10), ("L2", 2 << 20), ("LLC", 128 << 20), ("HBM", 3 << 30))


def gather_ceiling(n_rows=1 << 24, per=64, launches=10, levels=None, verbose=True):
    """Rate of random 1 KB row gathers (16 bytes per lane, eight rows in
    flight per wavefront) from each level of the memory hierarchy: the
    ceiling for the edge kernel's key and value gathers."""
    import torch
    import graph_sparse_head_amd as pma
    g = torch.Generator(device="cuda").manual_seed(11)
    sink = torch.empty(((n_rows + per - 1) // per) * 1024, dtype=torch.uint8, device="cuda")
    res = {"rows_per_launch": n_rows, "row_bytes": 1024, "rows_per_wave": per, "levels": {}}
    for name, nbytes in CEILING_TABLES:
        if levels is not None and name not in levels:
            continue
        table = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
        rows = torch.randint(0, nbytes // 1024, (n_rows,), generator=g, device="cuda",
                             dtype=torch.int32)
        for _ in range(3):
            pma.pma_gather_ceiling(table, rows, per, sink)
        st = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(launches):
            pma.pma_gather_ceiling(table, rows, per, sink)
        b.record(st)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / launches
        rate = n_rows * 1024 / (us * 1e-6)
        res["levels"][name] = {"table_bytes": nbytes, "avg_launch_us": us,
                               "delivered_TBs": rate / 1e12,
                               "bytes_per_clk_per_cu": rate / (2.4e9 * 256)}
        del table, rows
        if verbose:
            print(f"gather ceiling {name:4s} table {nbytes:>11d} B: {us:9.1f} us per launch, "
                  f"{rate / 1e12:6.2f} TB/s, {rate / (2.4e9 * 256):5.1f} B/clk/CU",
                  file=sys.stderr, flush=True)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="gene",
                    choices=["tiny", "complete", "gene", "bipartite", "large"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--train", action="store_true",
                    help="time a training step: pma_forward_train + pma_backward")
    ap.add_argument("--key-padding-mask", type=float, default=0.0, metavar="FRAC",
                    help="mask this fraction of keys per sample (seeded); 0: no mask")
    ap.add_argument("--no-profile", action="store_true",
                    help="time without per-stage events (no roofline)")
    ap.add_argument("--linear", action="store_true",
                    help="time PackedLinear (pma_linear_forward) on the workload's graph instead")
    ap.add_argument("--channels", type=int, default=1,
                    help="channels per node for --linear (1: the nn.Linear-shaped layer)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph that captured one pma_forward_static "
                         "(needs a workspace within the static scratch)")
    ap.add_argument("--legs", default="cold,warm",
                    help="timed legs in order: cold (each step after a 1 GiB cache overwrite; "
                         "the first leg is the headline) and/or warm (steps back to back)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized device buffer 5 times (counter calibration)")
    ap.add_argument("--gather-ceiling", action="store_true",
                    help="only time pma_gather_ceiling (random 1 KB row gathers) from tables "
                         "sized for L1, L2, the last-level cache and HBM")
    args = ap.parse_args()
    if args.gather_ceiling:
        print(json.dumps(gather_ceiling()), flush=True)
        return
    if args.copy_probe:
        import torch
        n = args.copy_probe << 20
        a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": n, "launches": 5}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this path runs on a single GPU)", file=sys.stderr)
        sys.exit(2)

    if args.linear:
        bench_linear(args)
        return
    legs = [x for x in args.legs.split(",") if x]
    if not legs or any(x not in ("cold", "warm") for x in legs) or len(set(legs)) != len(legs):
        ap.error("--legs takes cold and/or warm")

    import torch
    import graph_sparse_head_amd as pma
    from graph_sparse_head_amd import synth

    case = _workload(args.config)
    dev = synth.to_torch(case)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    plan = pma.pma_create(case.src, case.tgt, case.L, case.S, case.E, case.H,
                          add_self_loops=case.add_self_loops, dtype=case.dtype)
    create_ms = (time.perf_counter() - t0) * 1e3
    nnz = plan.nnz
    info = pma.pma_plan_info(plan)
    tdt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    out = torch.empty(case.B, case.L, case.E, dtype=tdt, device="cuda")
    weights = None
    if case.need_weights:
        shape = (case.B, nnz) if case.average else (case.B, nnz, case.H)
        weights = torch.empty(shape, dtype=torch.float32, device="cuda")

    kpm = None
    if args.key_padding_mask > 0:
        kpm = torch.from_numpy(np.random.default_rng(3).random((case.B, case.S))
                               < args.key_padding_mask).cuda()

    if args.train:
        save = torch.empty(pma.pma_train_bytes(plan, case.B), dtype=torch.uint8, device="cuda")
        gout = torch.randn(out.shape, generator=torch.Generator().manual_seed(4)).to(out.dtype).cuda()

    graph = None
    if args.graph:
        if args.train or kpm is not None:
            ap.error("--graph times the inference forward without a mask")
        fargs = (dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["bq"], dev["wk"], dev["bk"],
                 dev["wv"], dev["bv"], dev["wo"], dev["bo"])
        pma.pma_forward_static(plan, *fargs, out=out, weights=weights,
                               need_weights=case.need_weights, average_attn_weights=case.average)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                pma.pma_forward_static(plan, *fargs, out=out, weights=weights,
                                       need_weights=case.need_weights,
                                       average_attn_weights=case.average)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        args.no_profile = True    # (a replay records no stage events)

    def step():
        if graph is not None:
            graph.replay()
            return
        if args.train:
            pma.pma_forward_train(plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["bq"],
                                  dev["wk"], dev["bk"], dev["wv"], dev["bv"], dev["wo"], dev["bo"],
                                  save=save, out=out, weights=weights,
                                  need_weights=case.need_weights,
                                  average_attn_weights=case.average, key_padding_mask=kpm)
            pma.pma_backward(plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["wk"],
                             dev["wv"], dev["wo"], dev["bq"] is not None, save, gout,
                             key_padding_mask=kpm)
            return
        pma.pma_forward(plan, dev["xq"], dev["xk"], dev["xv"], dev["wq"], dev["bq"], dev["wk"],
                        dev["bk"], dev["wv"], dev["bv"], dev["wo"], dev["bo"], out=out,
                        weights=weights, need_weights=case.need_weights,
                        average_attn_weights=case.average, key_padding_mask=kpm)

    stream = torch.cuda.current_stream()
    lib = pma._load()
    # Cold cache (the headline): before every step, overwrite a 1 GiB buffer
    # (four times the 256 MB last-level cache) outside the step's events, so
    # that no input, weight or workspace line is still cached from the step
    # before. Warm: steps back to back, for context.
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if "cold" in legs else None

    def timed_steps(n, cold, stage_mask_of=None):
        """Per-step event times (ms) of n steps; stage_mask_of(i) picks the
        stages timed with HIP events inside step i (None: none)."""
        evs = []
        for i in range(n):
            if cold:
                scratch.fill_(float(i))
            if stage_mask_of is not None:
                lib.pma_profile_stages(plan.handle, stage_mask_of(i))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        if stage_mask_of is not None:
            lib.pma_profile_stages(plan.handle, 0)
        return [a.elapsed_time(b) for a, b in evs]

    first = legs[0]
    for i in range(args.warmup):
        if first == "cold":
            scratch.fill_(float(i))
        step()
    torch.cuda.synchronize()
    if not args.no_profile:
        pma.pma_profile_read(plan)          # discard anything earlier
    # The edge kernel is timed with HIP events on the forward's own stream in
    # every EVERY-th step of the headline leg: each timed stage adds two event
    # records, which themselves cost a few microseconds of that step.
    EVERY = 5
    edge_bit = 1 << pma.STAGES.index("edge")
    times, stages = {}, None
    for leg in legs:
        prof = None if args.no_profile or leg != first else \
            (lambda i: edge_bit if i % EVERY == 0 else 0)
        torch.cuda.synchronize()
        times[leg] = timed_steps(args.steps, leg == "cold", prof)
        if prof is not None:
            stages = pma.pma_profile_read(plan)
    all_stages = None
    if not args.no_profile:
        # per-stage breakdown from a separate pass (outside the measured legs),
        # under the headline leg's cache state
        timed_steps(args.steps, first == "cold", lambda i: (1 << len(pma.STAGES)) - 1)
        all_stages = pma.pma_profile_read(plan)
    probe = None
    if not args.train and not args.no_profile:
        # Calibration: the edge kernel's loads alone (same pieces, order,
        # lanes and gather index; no arithmetic), under the same cache state:
        # what the memory path needs for this access pattern.
        step()
        pt = []
        for i in range(args.steps):
            if first == "cold":
                scratch.fill_(float(i))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            try:
                pma.pma_gather_probe(plan)
            except pma.PmaError:     # head sizes of the per-channel kernel
                break
            e1.record(stream)
            pt.append((e0, e1))
        torch.cuda.synchronize()
        if pt:
            probe = sum(a.elapsed_time(b) for a, b in pt) / len(pt) * 1e-3
    del scratch
    ceiling = None
    if not args.train and not args.no_profile:
        # Calibration: what the memory path delivers for random 1 KB row
        # gathers from L2 and from the last-level cache (a few ms)
        ceiling = gather_ceiling(n_rows=1 << 22, launches=5, levels=("L2", "LLC"), verbose=False)
    head = times[first]
    ms_per_step = sum(head) / len(head)
    edge_heads = nnz * case.H * case.B
    value = edge_heads / (ms_per_step * 1e-3)

    es = 2 if case.dtype == "bf16" else 4
    fused = case.E == 64                     # q projection and out_proj inside the edge kernel
    res = {
        "metric": METRIC, "value": value, "unit": "edge-heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": case.dtype, "data": "synthetic",
        "config": {"workload": (f"{case.name}: L={case.L} S={case.S} nnz={nnz} B={case.B} "
                                f"E={case.E} H={case.H} {case.dtype}"
                                f"{' (fp32 softmax, sums and mixing weights; q, k, v, mixed stored bf16)' if case.dtype == 'bf16' else ''}"
                                f"{' need_weights' if case.need_weights else ''}"
                                f"{f' key_padding_mask {args.key_padding_mask:g}' if kpm is not None else ''}"
                                f"{' train step (forward + backward)' if args.train else ''}"
                                f"{'; HIP graph replay of pma_forward_static' if graph is not None else ''}"
                                + ("; cold cache: each step after a 1 GiB overwrite"
                                   if first == "cold" else "; warm cache: steps back to back")),
                   "batch": case.B, "nodes": case.L, "nnz": nnz, "embed_dim": case.E,
                   "num_heads": case.H, "parallelism": "single GPU"},
    }
    for leg in legs:
        t = sorted(times[leg])
        res[f"{leg}_ms_per_step"] = {"mean": sum(t) / len(t), "median": t[len(t) // 2],
                                     "min": t[0]}
    if stages is not None and not args.train:
        edge_ms, edge_calls = stages["edge"]
        edge_avg_s = edge_ms / max(edge_calls, 1) * 1e-3
        nbytes = edge_kernel_bytes(case.B, case.L, info["kv_rows"], nnz, info["n_tasks"],
                                   case.E, es, case.need_weights, case.H, kpm is not None)
        gbytes = edge_gather_bytes(case.B, case.L, nnz, case.E, es)
        achieved = nbytes / edge_avg_s / 1e9
        # (the committed counters are of the unmasked forward)
        traffic = _traffic(args.config) if kpm is None else None
        res["roofline"] = {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic["bytes_per_launch"] if traffic else None,
            "kernel": "edge_fast" + (" (q projection and out_proj fused)" if fused else ""),
            "bytes_per_launch": nbytes, "bytes": "compulsory: each input and output byte once",
            "avg_launch_us": edge_avg_s * 1e6, "timed_launches": edge_calls,
            "gather_model": {"bytes_per_launch": gbytes,
                             "delivered_GBs": gbytes / edge_avg_s / 1e9,
                             "note": "every edge's key and value rows per sample; mostly "
                                     "served by L2 and the last-level cache, not an HBM rate"},
        }
        if ceiling is not None:
            lv = ceiling["levels"]
            l2, llc = lv["L2"]["delivered_TBs"], lv["LLC"]["delivered_TBs"]
            gc = {"L2_TBs": l2, "LLC_TBs": llc,
                  "gather_vs_L2": gbytes / edge_avg_s / 1e12 / l2,
                  "note": "pma_gather_ceiling: random 1 KB row gathers (the edge kernel's lane "
                          "layout) from a 2 MiB table (L2) and a 128 MiB one (last-level cache); "
                          "gather_vs_L2 = the gather model's rate over the L2 ceiling"}
            if traffic:
                rd = traffic["read_bytes"] / edge_avg_s / 1e12
                gc["beyond_L2_read_TBs"] = rd
                gc["beyond_L2_vs_LLC"] = rd / llc
            res["roofline"]["gather_ceiling"] = gc
        if probe is not None:
            res["roofline"]["gather_probe"] = {
                "avg_launch_us": probe * 1e6, "delivered_GBs": gbytes / probe / 1e9,
                "edge_frac_of_probe": probe / edge_avg_s,
                "note": "the edge kernel's loads and stores alone (pma_gather_probe): the "
                        "memory path's time for this access pattern"}
    if all_stages is not None:
        res["stages_us"] = {k: (v[0] / max(v[1], 1)) * 1e3 for k, v in all_stages.items() if v[1]}
    res["create_ms"] = create_ms
    res["plan"] = {k: info[k] for k in ("n_tasks", "n_split", "chunk", "max_degree", "kv_rows")}
    pma.pma_destroy(plan)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
