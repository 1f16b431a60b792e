"""Throughput of the hashed n-gram embedding hot path on one MI355X.

One step = one pass of the whole path over one token batch:
    engram_lookup (forward: the row ids hashed from the tokens and their
       table rows gathered, in one kernel)
    -> engram_scatter_plan_tokens + engram_scatter_apply (backward: per-row
       fp32 sums; the same work as hashing, then the one-call scatter-add)
The plan (sorting the row ids) needs only the tokens, so the next batch's
plan runs on a second stream while the current step's forward and backward
run (a training loop knows its next batch), into the other of two
workspaces; the apply waits for the forward and for its batch's plan.  The
timed region holds exactly one plan, forward and apply per step (it ends
when the plan made during the last step is done too); untimed steps run
before it for --settle seconds (0.25 by default), then the W warm-up steps.
Every step is timed twice: each step's calls and events enqueued by one
native call (engram_run_ops, the binding's Schedule, built once per token
batch), which is the line's time, and the same calls made one by one
through the binding (eager_ms_per_step).  The last timed step's backward is
checked bit for bit against the same batch planned and applied one call
after another, in both.  With --graphs the step
is also captured once per token batch as a HIP graph and replayed (one host
launch per step, the same kernels and the same plan beside the forward and
apply; checked the same way) and reported as graph_ms_per_step: on MI355X
the replays measured slower than the calls launched one by one (e2e 0.721
against 0.692 ms, the backward workload 89 against 83 us), since a replay
ends only when all its branches have, and the next cannot start before.  A
serial pass of the same calls gives the per-phase times, and the same step
with separate calls (engram_hash, then engram_scatter_plan of the ids beside
engram_gather, then the apply) is timed beside it.

The default run measures the end-to-end workload -- tokens [8, 8192]
(Zipf(1.1) ids, EOS w.p. 1/4096), ngram_size 4, 8 heads per order (24
heads), a 200M x 256 bf16 table (102.4 GB, resident in HBM), upstream
gradients [8, 8192, 24, 256] bf16, row-sparse fp32 gradients -- and prints
it as the JSON line, with the other configurations of the benchmark nested
under "other_configs", each with its own roofline and CPU baseline:
    medium    forward only: tokens [4, 4096] uniform, 16 heads, 16.8M x 64 table
    full      forward only: tokens [1, 32768] packed documents, Zipf(1.1),
              32 heads, the 200M x 256 table (the e2e run's, reused)
    backward  forward + dense fp32 backward: tokens [4, 4096] Zipf(1.2), 16
              heads, 16.8M x 64 table; also the one-call scatter-add, sorted
              against fp32 atomics, on the same ids and gradients
    e2e_padtail  the e2e step on packs of whole documents whose row tails are
              pad tokens in a segment of their own (hot rows of thousands of
              terms per head), on the same table
Eight distinct token batches are cycled so one step does not warm the next.
All inputs are resident in HBM before timing starts.

`value` is row lookups per second over the whole step.  The roofline entry
is for the step's dominant call, timed with HIP events on the stream it
runs on: the forward as the step itself, the apply (its two launches) as
back-to-back calls on two batches' plans in turn ("apply_back_to_back_ms";
the fused SignSGD apply as a single call).
The CPU baseline is the oracle on the host: one core, and the same source
built with OpenMP on every thread the process may use.

    python bench.py [--steps K] [--warmup W] [--no-other-configs]
                    [--workload e2e|e2e_signsgd|full|medium|backward|cp_slice|ple_conv]

--workload ple_conv times the PLE causal dilated depthwise convolution
(engram_ple_conv) on bf16 [8, 8192, 8192] with packed-document segment ids,
kernel 4, dilation 4 (the metric is then positions x channels per second).

--workload e2e_signsgd is the e2e step with the optimizer: the apply is
engram_scatter_apply_signsgd, which sums each distinct row's gradients and
applies one SignSGD step to that row of the bf16 table in the same pass
(the fp32 sums are never written).  The line also reports the same step
done in two calls (row-sparse apply, then engram_signsgd_rowsparse).

--workload cp_slice times one context-parallel rank's forward on the
full-scale workload (tokens [1, 32768], 32 heads, the 200M x 256 table):
engram_lookup_slice over the last of 8 equal slices of the replicated
sequence (with its packed-segment ids), hashing and gathering the slice in
one kernel; the two-call form (engram_hash_slice, then engram_gather) is
timed beside it.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("row lookups/s and achieved HBM GB/s (% of peak), "
          "fwd hash+gather and bwd scatter")
PEAK_HBM_GBS = 8000.0
N_BATCHES = 8
# Bytes of the host copy of a table the CPU baseline gathers from: a table
# larger than this (the 102.4 GB ones) is copied in part, its first rows, and
# the baseline's row ids are folded modulo their count.
HOST_TABLE_BYTES = 8 << 30
CPU_BUDGET_S = 6.0  # per CPU leg: repeat within this, at most 5 runs, median


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(wl, unique_rows, separate=False):
    """Bytes the method must move per call (reads + writes), per phase.  The
    fused forward (engram_lookup) reads the tokens and the table rows and
    writes the output; the row ids never reach memory.  With separate calls
    (engram_hash, engram_gather, engram_scatter_plan) the ids are written
    once and read twice."""
    N, R, D = wl.tokens_per_batch, wl.lookups, wl.dim
    if separate:
        out = {"hash": 8 * N + 8 * R, "gather": 8 * R + 2 * D * R + 2 * D * R}
    else:
        out = {"lookup": 8 * N + 2 * D * R + 2 * D * R}
    # the backward's plan (sorting the ids) is overhead: its algorithmic
    # bytes are what it reads (the ids, or the tokens it hashes again); the
    # apply moves the gradients
    if wl.grads != "none":
        out["scatter_plan"] = 8 * R if separate else 8 * N
    if wl.grads == "rowsparse":
        out["scatter_apply"] = 2 * D * R + (4 * D + 8) * unique_rows
    elif wl.grads == "dense":
        out["scatter_apply"] = 2 * D * R + 8 * D * unique_rows
    return out


def code_digest(paths):
    """sha256 of the code in `paths` (repository-relative) with comments and
    whitespace removed, so that edits to comments alone keep it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in paths:
        text = open(os.path.join(ROOT, rel)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(call, wl):
    """HBM bytes per launch of `call` on workload wl from the committed
    rocprofv3 counter summary (profiles/hbm_traffic.json), or None when no
    counters were taken on that workload or the kernel's code has changed
    since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("workloads", {}).get(wl.name)
    key = {"lookup": "lookup", "gather": "gather", "scatter_apply": "apply"}.get(call)
    if rec is None or key not in rec["kernels"]:
        return None
    k = rec["kernels"][key]
    if code_digest(k["code_files"]) != k.get("code_sha256"):
        return None
    return k["fetch_bytes"] + k["write_bytes"]


# ------------------------------------------------------------ CPU baseline --
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def timed_runs(fn, budget_s=CPU_BUDGET_S):
    """Seconds per run of fn: repeated until the budget is spent (at least
    once, at most 5 times); the median."""
    times, start = [], time.perf_counter()
    while len(times) < 5 and (not times or time.perf_counter() - start < budget_s):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times)


def cpu_baseline(work, units, unit, sample):
    """The oracle on this host: `work(oracle)` run by the serial build on one
    core, and by the OpenMP build of the same source on every thread it may
    use.  The all-core rate is `value`; the one-core rate is reported beside."""
    from oracle import default_oracle, openmp_oracle

    serial, par = default_oracle(), openmp_oracle()
    t1, n1 = timed_runs(lambda: work(serial))
    tn, nn = timed_runs(lambda: work(par))
    return {"value": units / tn, "unit": unit, "cores": par.threads, "kind": "oracle",
            "sample": f"{sample}; median of {nn} runs (one core: {n1})",
            "single_core": {"value": units / t1, "cores": 1},
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "threads_allowed": len(os.sched_getaffinity(0))}


def host_bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_table(table):
    """(uint16 bits of the table, or of as many of its first rows as fit in
    HOST_TABLE_BYTES, and whether ids must be folded into those rows)."""
    rows, dim = table.shape
    fit = HOST_TABLE_BYTES // (2 * dim)
    if rows <= fit:
        return host_bits(table), False
    return host_bits(table[:fit]), True


def step_cpu_baseline(wl, tokens_host, segs_host, mult, table, grads):
    """The oracle's step on this workload's first token batch: the hash, the
    gather and (when the workload has a backward) the scatter-add of the
    upstream gradients into the workload's gradient form."""
    import torch
    tab_bits, folded = host_table(table)
    hargs = (wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult, wl.primes, wl.offsets)
    tok, seg = tokens_host[0], segs_host[0]
    from oracle import default_oracle
    rows = default_oracle().hash(tok, *hargs, seg).reshape(-1)
    gather_rows = rows % tab_bits.shape[0] if folded else rows
    grad_bits = host_bits(grads) if grads is not None else None
    dense = None
    if wl.grads == "dense":
        dense = np.zeros((wl.table_rows, wl.dim), dtype=np.float32)
        dense.fill(0.0)  # touch every page before timing

    def work(o):
        o.hash(tok, *hargs, seg)
        o.gather(gather_rows, tab_bits)
        if wl.grads == "rowsparse":
            o.scatter_add_rowsparse(rows, grad_bits, wl.dim, wl.table_rows)
        elif wl.grads == "dense":
            o.scatter_add_dense(rows, grad_bits, dense, inplace=True)

    what = {"rowsparse": "hash, gather and row-sparse scatter-add",
            "dense": "hash, gather and dense fp32 scatter-add (into a host table of the "
                     "workload's shape)",
            "none": "hash and gather"}[wl.grads]
    where = (f"gathering from a host copy of the table's first {tab_bits.shape[0]} rows "
             f"({tab_bits.nbytes / 1e9:.1f} GB) with row ids folded modulo that count"
             if folded else "gathering from a host copy of the whole table")
    del torch
    return cpu_baseline(work, wl.lookups, "lookups/s",
                        f"the {wl.name} step on one token batch ({wl.lookups} lookups): {what}; "
                        f"{where}")


# --------------------------------------------------------------- HBM probe --
def copy_probe_gbps(torch, dev, stream):
    """The hand-written streaming copy (gram_hashed_embedding_amd/probe) over
    2 GiB each way: what this GPU's HBM gives a plain 16-byte copy."""
    path = os.path.join(ROOT, "gram_hashed_embedding_amd", "probe", "libengram_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.engram_probe_stream_copy.restype = ctypes.c_int
    lib.engram_probe_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_void_p]
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    s = ctypes.c_void_p(stream.cuda_stream)

    def run():
        rc = lib.engram_probe_stream_copy(ctypes.c_void_p(src.data_ptr()),
                                          ctypes.c_void_p(dst.data_ptr()), nbytes // 16, s)
        if rc != 0:
            raise RuntimeError("copy probe launch failed")
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(10):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    gbps = 2 * nbytes * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    return gbps


# ------------------------------------------------------- the step benchmark --
def bench_step(args, torch, E, workloads, name, table=None, cpu=True):
    """One workload's step (see the module docstring): the result dict.
    `table` is an existing bf16 table of the workload's shape to reuse."""
    signsgd = name == "e2e_signsgd"
    lr = 1e-6  # the learning rate of the pages' SignSGD runs
    wl = workloads.get("e2e" if signsgd else name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    mult = wl.multipliers()
    log(f"[bench] workload {wl.describe()}")

    # packed workloads carry their segment ids (the pad-tail one needs them:
    # its tail is a segment of its own)
    with_seg = wl.token_kind == "packed_pad"
    drawn = [wl.tokens(k, with_segments=True) for k in range(N_BATCHES)]
    tokens_host = [t for t, _ in drawn]
    tokens = [torch.from_numpy(t).to(dev) for t in tokens_host]
    segs_host = [sg if with_seg else None for _, sg in drawn]
    segs = [None if sg is None else torch.from_numpy(sg).to(dev) for sg in segs_host]
    t0 = time.perf_counter()
    shared_table = table is not None and tuple(table.shape) == (wl.table_rows, wl.dim)
    if not shared_table:
        table = workloads.make_table(wl.table_rows, wl.dim, wl.seed, dev)
    torch.cuda.synchronize()
    log(f"[bench] table {tuple(table.shape)} bf16 ready in {time.perf_counter() - t0:.1f}s")

    R, D = wl.lookups, wl.dim
    rows = torch.empty((wl.batch, wl.seq, wl.heads), dtype=torch.int64, device=dev)
    out = torch.empty((R, D), dtype=torch.bfloat16, device=dev)
    backward = wl.grads != "none"
    grads = None
    if backward:
        grads = workloads.make_grads(R, D, wl.seed + 2, dev)
    if wl.grads == "rowsparse":  # (the SignSGD step's comparison uses these too)
        uid = torch.empty(R, dtype=torch.int64, device=dev)
        uval = torch.empty((R, D), dtype=torch.float32, device=dev)
        count = torch.zeros(1, dtype=torch.int64, device=dev)
        mode = E.SCATTER_ROWSPARSE
    elif wl.grads == "dense":
        gtab = workloads.make_grad_table(wl.table_rows, D, None, dev)
        mode = E.SCATTER_SORTED
    if backward:
        # two workspaces: the plan of the next batch is made while this
        # batch's step runs, so consecutive steps use alternate workspaces
        wss = [torch.empty(max(E.engram_scatter_add_workspace(R, wl.table_rows, D, mode), 1),
                           dtype=torch.uint8, device=dev) for _ in range(2)]
        ws = wss[0]

    side = torch.cuda.Stream(dev)  # default priority
    # every plan and apply reports into one device counter, checked after the
    # run: an expired wait or an apply without its plan would show there
    err = torch.zeros(1, dtype=torch.int64, device=dev)
    hargs = (wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult, wl.primes, wl.offsets)
    ev_plan = [torch.cuda.Event() for _ in range(2)]
    ev_apply = [torch.cuda.Event() for _ in range(2)]
    ev_rows = [torch.cuda.Event() for _ in range(2)]

    planned = {"next": None}

    def plan_ahead(k):
        """The plan of batch k (engram_scatter_plan_tokens: it needs only the
        tokens) on the side stream, into workspace k % 2, once the apply that
        last read that workspace (batch k - 2) is done."""
        side.wait_event(ev_apply[k % 2])
        E.engram_scatter_plan_tokens(tokens[k % N_BATCHES], wl.table_rows, D, *hargs,
                                     seq_ids=segs[k % N_BATCHES], workspace=wss[k % 2],
                                     err_count=err, stream=side)
        ev_plan[k % 2].record(side)
        planned["next"] = k

    def step(k):
        """One step.  The forward is one pass (engram_lookup: hash and gather
        fused).  The backward's plan needs only the tokens, so the next
        batch's plan is made on a side stream while this step's forward and
        backward run (a training loop knows its next batch); the apply
        follows the forward and waits for its own batch's plan, made during
        the step before.  Every step makes one plan, one forward and one
        apply."""
        tok, sg = tokens[k % N_BATCHES], segs[k % N_BATCHES]
        if not backward:
            E.engram_lookup(tok, table, *hargs, seq_ids=sg, out=out)
            return
        if planned["next"] != k:  # the first step: nothing planned yet
            plan_ahead(k)
        plan_ahead(k + 1)
        E.engram_lookup(tok, table, *hargs, seq_ids=sg, out=out)
        stream.wait_event(ev_plan[k % 2])
        apply_backward(wss[k % 2])
        ev_apply[k % 2].record(stream)

    scheds = None

    def build_schedules():
        """The step of each token batch as one engram_run_ops schedule: the
        same calls and events as step() (the next batch's plan on the side
        stream after the apply that last read its workspace; the fused
        forward; the apply after this batch's plan), enqueued by one native
        call instead of one binding call and one torch event call each."""
        out_ = []
        for k in range(N_BATCHES):
            nk = (k + 1) % N_BATCHES
            sc = E.Schedule()
            sc.wait(ev_apply[nk % 2], stream=side)
            sc.plan_tokens(tokens[nk], wl.table_rows, D, *hargs, seq_ids=segs[nk],
                           workspace=wss[nk % 2], err_count=err, stream=side)
            sc.record(ev_plan[nk % 2], stream=side)
            sc.lookup(tokens[k], table, *hargs, seq_ids=segs[k], out=out, stream=stream)
            sc.wait(ev_plan[k % 2], stream=stream)
            if signsgd:
                sc.apply_signsgd(grads, wss[k % 2], table, lr, err_count=err, stream=stream)
            elif wl.grads == "rowsparse":
                sc.apply(grads, wss[k % 2], wl.table_rows, unique_ids=uid, unique_grads=uval,
                         num_unique=count, err_count=err, stream=stream)
            else:
                sc.apply(grads, wss[k % 2], wl.table_rows, grad_table=gtab, err_count=err,
                         stream=stream)
            sc.record(ev_apply[k % 2], stream=stream)
            out_.append(sc)
        return out_

    def step_scheduled(k):
        """step(k), enqueued as the prebuilt schedule of its token batch."""
        if not backward:  # the forward alone: one operation
            scheds[k % N_BATCHES].run()
            return
        if planned["next"] != k:  # the first step: nothing planned yet
            plan_ahead(k)
        scheds[k % N_BATCHES].run()
        planned["next"] = k + 1

    def step_separate(k):
        """The same step with separate calls (hash, then the plan of the ids
        beside the gather), for comparison."""
        E.engram_hash(tokens[k % N_BATCHES], *hargs, wl.table_rows, seq_ids=segs[k % N_BATCHES],
                      out=rows)
        if not backward:
            E.engram_gather(rows, table, out=out)
            return
        ev_rows[k % 2].record(stream)
        side.wait_event(ev_rows[k % 2])
        E.engram_scatter_plan(rows.view(-1), wl.table_rows, D, workspace=ws, err_count=err,
                              stream=side)
        ev_plan[k % 2].record(side)
        E.engram_gather(rows, table, out=out)
        stream.wait_event(ev_plan[k % 2])
        apply_backward(ws)

    def apply_backward(ws):
        if signsgd:
            E.engram_scatter_apply_signsgd(grads, ws, table, lr, err_count=err)
        elif wl.grads == "rowsparse":
            E.engram_scatter_apply(grads, ws, wl.table_rows, unique_ids=uid, unique_grads=uval,
                                   num_unique=count, err_count=err)
        else:
            E.engram_scatter_apply(grads, ws, wl.table_rows, grad_table=gtab, err_count=err)

    def serial_step(k, ev, separate=False):
        """The calls of a step one after another on one stream, with events
        between them (per-phase times)."""
        tok, sg = tokens[k % N_BATCHES], segs[k % N_BATCHES]
        ev[0].record(stream)
        if separate:
            E.engram_hash(tok, *hargs, wl.table_rows, seq_ids=sg, out=rows)
            ev[1].record(stream)
            E.engram_gather(rows, table, out=out)
        else:
            E.engram_lookup(tok, table, *hargs, seq_ids=sg, out=out)
            ev[1].record(stream)
        ev[2].record(stream)
        if backward:
            if separate:
                E.engram_scatter_plan(rows.view(-1), wl.table_rows, D, workspace=ws,
                                      err_count=err)
            else:
                E.engram_scatter_plan_tokens(tok, wl.table_rows, D, *hargs, seq_ids=sg,
                                             workspace=ws, err_count=err)
            ev[3].record(stream)
            apply_backward(ws)
            ev[4].record(stream)

    last_step = {"k": None}  # the last timed step's index (its token batch)

    def timed_steps(fn):
        # untimed settle steps for args.settle seconds, then the W warm-up
        # steps: a few warm-up steps alone leave the fused SignSGD step about
        # 6% slower than its steady state (790 against 744 us on one box; the
        # row-sparse step is the same either way)
        k = 0
        t_end = time.perf_counter() + args.settle
        while time.perf_counter() < t_end:
            fn(k)
            k += 1
            if k % 32 == 0:
                torch.cuda.synchronize()
        for _ in range(args.warmup):
            fn(k)
            k += 1
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for k in range(k, k + args.steps):
            fn(k)
        last_step["k"] = k
        if fn in (step, step_scheduled) and backward:
            # the plan made during the last step (the next batch's) is part
            # of the timed work: the stop mark waits for it too
            stream.wait_event(ev_plan[planned["next"] % 2])
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps

    def serial_phases(separate):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
               for _ in range(args.steps)]
        for k in range(args.steps):
            serial_step(k, evs[k], separate)
        torch.cuda.synchronize()
        mean = lambda i, j: float(np.mean([e[i].elapsed_time(e[j]) for e in evs]))
        ph = ({"hash": mean(0, 1), "gather": mean(1, 2)} if separate
              else {"lookup": mean(0, 2)})
        if backward:
            ph["scatter_plan"] = mean(2, 3)
            ph["scatter_apply"] = mean(3, 4)
        return ph, mean(0, 4 if backward else 2)

    def capture_steps():
        """The step as HIP graphs, one per token batch: graph k makes batch
        k + 1's plan (into workspace (k + 1) % 2) on a branch beside batch k's
        forward and apply (which reads workspace k % 2), joined at its end.
        Replays on one stream run one after another, so a graph's plan never
        overlaps the apply that last read its workspace (N_BATCHES is even:
        the batches and the workspaces cycle together).  The launches of a
        step then cost one graph launch on the host."""
        assert N_BATCHES % 2 == 0
        torch.cuda.synchronize()
        graphs = []
        cap = torch.cuda.Stream(dev)  # default priority
        for k in range(N_BATCHES):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                cur = torch.cuda.current_stream(dev)
                side.wait_stream(cur)
                with torch.cuda.stream(side):
                    E.engram_scatter_plan_tokens(
                        tokens[(k + 1) % N_BATCHES], wl.table_rows, D, *hargs,
                        seq_ids=segs[(k + 1) % N_BATCHES], workspace=wss[(k + 1) % 2],
                        err_count=err, stream=side)
                E.engram_lookup(tokens[k], table, *hargs, seq_ids=segs[k], out=out)
                apply_backward(wss[k % 2])
                cur.wait_stream(side)
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs

    def check_last():
        """The timed schedule's last apply against the same batch planned and
        applied one call after another on one stream, bit for bit."""
        last = last_step["k"]
        ws_ref = torch.empty_like(ws)
        uid_ref, uval_ref = torch.empty_like(uid), torch.empty_like(uval)
        cnt_ref = torch.zeros_like(count)
        E.engram_scatter_plan_tokens(tokens[last % N_BATCHES], wl.table_rows, D, *hargs,
                                     seq_ids=segs[last % N_BATCHES], workspace=ws_ref,
                                     err_count=err)
        E.engram_scatter_apply(grads, ws_ref, wl.table_rows, unique_ids=uid_ref,
                               unique_grads=uval_ref, num_unique=cnt_ref, err_count=err)
        torch.cuda.synchronize()
        u_ref = int(cnt_ref.item())
        if not (int(count.item()) == u_ref and torch.equal(uid[:u_ref], uid_ref[:u_ref])
                and torch.equal(uval[:u_ref].view(torch.int32),
                                uval_ref[:u_ref].view(torch.int32))):
            raise RuntimeError("the timed schedule's backward differs from the serial calls")
        del ws_ref, uid_ref, uval_ref, cnt_ref

    # whole-step timing (the driver's step): nothing between the calls,
    # launched call by call through the binding ...
    eager_ms = timed_steps(step)
    checkable = wl.grads == "rowsparse" and not signsgd
    if checkable:
        check_last()
    # ... and each step enqueued by one native call (engram_run_ops)
    if backward:
        scheds = build_schedules()
    else:
        scheds = [E.Schedule().lookup(tokens[k], table, *hargs, seq_ids=segs[k], out=out,
                                      stream=stream) for k in range(N_BATCHES)]
    planned["next"] = None
    torch.cuda.synchronize()
    sched_ms = timed_steps(step_scheduled)
    if checkable:
        check_last()
    # ... and, on request, as one graph replay per step
    graph_ms = None
    if backward and args.graphs:
        graphs = capture_steps()
        # batch 0's plan, before graph 0 (which plans batch 1)
        E.engram_scatter_plan_tokens(tokens[0], wl.table_rows, D, *hargs, seq_ids=segs[0],
                                     workspace=wss[0], err_count=err)
        torch.cuda.synchronize()
        graph_ms = timed_steps(lambda k: graphs[k % N_BATCHES].replay())
        if checkable:
            check_last()
        del graphs
    ms_per_step = sched_ms
    schedule = ("each step's calls and events enqueued by one engram_run_ops call"
                if backward else "each step's lookup enqueued by one engram_run_ops call")
    schedule_check = ("last step bit-exact against serial calls, in the scheduled and the "
                      "call-by-call runs" + (", and replayed as graphs" if graph_ms is not None
                                             else "") if checkable else None)
    phase_ms, serial_ms = serial_phases(False)
    # the same work with separate calls, timed in the same process
    sep_ms = timed_steps(step_separate)
    sep_phase_ms, _ = serial_phases(True)
    if backward and int(err.item()) != 0:
        raise RuntimeError(f"the step's plans or applies reported errors: {int(err.item())}")

    # distinct rows of each cycled batch (the backward's U), read after timing;
    # the step's bytes use their mean, as the timed steps cycle the batches
    unique_per_batch = []
    if backward:
        for k in range(N_BATCHES):
            E.engram_hash(tokens[k], *hargs, wl.table_rows, seq_ids=segs[k], out=rows)
            unique_per_batch.append(int(torch.unique(rows).numel()))
    unique_rows = float(np.mean(unique_per_batch)) if unique_per_batch else 0
    nbytes = algorithmic_bytes(wl, unique_rows)
    sep_bytes = algorithmic_bytes(wl, unique_rows, separate=True)
    scatter_modes = None
    if wl.grads == "dense":
        # the one-call scatter-add, sorted (plan + apply) and fp32-atomic, side
        # by side on the same ids and gradients (the dense table accumulates)
        E.engram_hash(tokens[0], *hargs, wl.table_rows, seq_ids=segs[0], out=rows)

        def timed_call(fn, reps=max(args.steps, 3)):
            fn()
            torch.cuda.synchronize()
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            for _ in range(reps):
                fn()
            b_.record(stream)
            torch.cuda.synchronize()
            return a_.elapsed_time(b_) / reps
        flat = rows.view(-1)
        dense_bytes = 8 * R + 2 * D * R + 8 * D * unique_per_batch[0]
        scatter_modes = {"algorithmic_bytes": dense_bytes, "unique_rows": unique_per_batch[0]}
        for name_, mode_ in (("sorted", E.SCATTER_SORTED), ("atomic", E.SCATTER_ATOMIC)):
            ms_ = timed_call(lambda: E.engram_scatter_add(
                flat, grads, gtab, mode=mode_,
                workspace=ws if mode_ == E.SCATTER_SORTED else None))
            gbps_ = dense_bytes / (ms_ * 1e-3) / 1e9
            scatter_modes[name_] = {"ms": ms_, "gbps": gbps_, "frac_of_peak": gbps_ / PEAK_HBM_GBS}
    unfused = None
    if signsgd:
        # the fused apply reads the gradient rows and reads + writes each
        # distinct row of the bf16 table once
        nbytes["scatter_apply"] = 2 * D * R + 4 * D * unique_rows
        sep_bytes["scatter_apply"] = nbytes["scatter_apply"]
        # the same step in two calls, for comparison (same plan, same stream)
        u0, u1, u2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        E.engram_hash(tokens[0], *hargs, wl.table_rows, out=rows)
        E.engram_scatter_plan(rows.view(-1), wl.table_rows, D, workspace=ws)
        tw = []
        for k in range(max(args.steps // 2, 3)):
            u0.record(stream)
            E.engram_scatter_apply(grads, ws, wl.table_rows, unique_ids=uid, unique_grads=uval,
                                   num_unique=count)
            u1.record(stream)
            E.engram_signsgd_rowsparse(uid, uval, count, table, lr)
            u2.record(stream)
            torch.cuda.synchronize()
            tw.append((u0.elapsed_time(u1), u1.elapsed_time(u2)))
        a_ms, s_ms = (float(np.median([t[i] for t in tw])) for i in range(2))
        u0_ = unique_per_batch[0]
        unfused = {"scatter_apply_ms": a_ms, "engram_signsgd_rowsparse_ms": s_ms,
                   "total_ms": a_ms + s_ms,
                   "algorithmic_bytes": 2 * D * R + (4 * D + 8) * u0_
                   + (8 + 4 * D + 4 * D) * u0_}

    def phase_table(pm, nb):
        out_ = {}
        for p_, ms in pm.items():
            b_ = nb.get(p_, 0)
            out_[p_] = {"ms": ms, "algorithmic_bytes": b_, "gbps": b_ / (ms * 1e-3) / 1e9,
                        "frac_of_peak": b_ / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
        return out_

    phases = phase_table(phase_ms, nbytes)
    step_bytes = sum(nbytes.values())
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    separate_calls = {"ms_per_step": sep_ms, "value": R / (sep_ms * 1e-3),
                      "step_algorithmic_bytes": sum(sep_bytes.values()),
                      "phases": phase_table(sep_phase_ms, sep_bytes)}

    # the apply's own duration: back-to-back calls between two events on its
    # stream (an event pair around a single call also counts
    # the host's submission of it whenever the GPU is ahead of the host, as on
    # the small backward workload)
    # (The fused SignSGD apply runs slower back to back than in the step, 473
    # against 421 us on one box, whose rocprofv3 average was 403 + 7 us: its
    # roofline keeps the single call's time.)
    apply_b2b_ms = None
    if backward:
        # two batches' plans, applied in turn: consecutive applies touch
        # different rows, as consecutive steps do
        for k in range(2):
            E.engram_scatter_plan_tokens(tokens[k], wl.table_rows, D, *hargs, seq_ids=segs[k],
                                         workspace=wss[k], err_count=err)
        apply_backward(wss[0])
        torch.cuda.synchronize()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(args.steps, 10)
        a_.record(stream)
        for k in range(reps):
            apply_backward(wss[k % 2])
        b_.record(stream)
        torch.cuda.synchronize()
        apply_b2b_ms = a_.elapsed_time(b_) / reps

    # roofline of the dominant call: the fused forward is one kernel launch,
    # and the apply two (the second adds up the rare runs split across chunks)
    dominant = "lookup"
    kernel = f"lookup_kernel<{wl.ngram_size}> (engram_lookup)"
    if backward and phase_ms["scatter_apply"] > phase_ms["lookup"]:
        dominant = "scatter_apply"
        kernel = ("segment_reduce_kernel, SignSGD output (engram_scatter_apply_signsgd)"
                  if signsgd else f"segment_reduce_kernel, {wl.grads} output "
                  "(engram_scatter_apply)")
    # a forward-only step is the one lookup launch, back to back: its time
    # per step is the kernel's own (an event pair around a single small
    # launch also counts the launch)
    if dominant == "scatter_apply" and not signsgd:
        achieved = nbytes["scatter_apply"] / (apply_b2b_ms * 1e-3) / 1e9
    else:
        achieved = phases[dominant]["gbps"] if backward else step_gbps
    roofline = {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "traffic": None if signsgd else measured_traffic(dominant, wl)}

    cpu_result = None
    if cpu and not args.no_cpu_baseline and not signsgd:
        try:
            cpu_result = step_cpu_baseline(wl, tokens_host, segs_host, mult, table, grads)
        except Exception as exc:  # the baseline must not hide the GPU number
            log(f"[bench] cpu baseline failed: {exc!r}")

    result = {
        "metric": METRIC,
        "value": R / (ms_per_step * 1e-3),
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {**wl.describe(),
                   **({"workload": "e2e_signsgd", "optimizer": "signsgd", "lr": lr}
                      if signsgd else {}),
                   "step": "lookup(hash+gather fused)"
                   + ("+scatter(plan from tokens, made for the next batch beside this step;"
                      " apply)" if backward else "")
                   + ("+signsgd(fused into the apply)" if signsgd else ""),
                   "backward": wl.grads, "accumulate": "f64" if backward else None,
                   "unique_rows": unique_rows, "unique_rows_per_batch": unique_per_batch,
                   "token_batches_cycled": N_BATCHES,
                   **({"table": "the e2e run's 200M x 256 bf16 table, reused"}
                      if shared_table else {}),
                   **({"segments": "packed documents; each row's tail after its last whole "
                       "document is pad tokens in a segment of their own"} if with_seg else {})},
        "schedule": schedule,
        "eager_ms_per_step": eager_ms,
        "scheduled_ms_per_step": sched_ms,
        "graph_ms_per_step": graph_ms,
        "serial_ms_per_step": serial_ms,
        "schedule_check": schedule_check,
        "step_algorithmic_bytes": step_bytes,
        "step_gbps": step_gbps,
        "step_frac_of_peak": step_gbps / PEAK_HBM_GBS,
        "phases": phases,
        **({"apply_back_to_back_ms": apply_b2b_ms} if backward else {}),
        "separate_calls": separate_calls,
        **({"two_call_apply_and_signsgd": unfused} if unfused else {}),
        **({"scatter_add_sorted_vs_atomic": scatter_modes} if scatter_modes else {}),
        "roofline": roofline,
        "cpu_baseline": cpu_result,
    }
    return result, table


def sub_config(res):
    """The fields of a nested configuration's result."""
    keep = ("metric", "value", "unit", "ms_per_step", "config", "schedule",
            "eager_ms_per_step", "scheduled_ms_per_step", "graph_ms_per_step", "schedule_check",
            "step_algorithmic_bytes",
            "step_gbps", "step_frac_of_peak", "phases", "apply_back_to_back_ms",
            "separate_calls", "scatter_add_sorted_vs_atomic", "roofline", "cpu_baseline")
    return {k: res[k] for k in keep if k in res}


def bench_cp_slice(args, torch, E, workloads, ranks=8):
    """One context-parallel rank's forward: its slice of the replicated
    sequence hashed (history read across the slice boundary) and looked up in
    one pass (engram_lookup_slice); the two-call form (engram_hash_slice,
    then engram_gather) is timed beside it."""
    wl = workloads.full()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    mult = wl.multipliers()
    S = wl.seq
    a, b = (ranks - 1) * S // ranks, S
    local = b - a
    log(f"[bench] cp_slice: workload {wl.describe()}, slice [{a}, {b}) of {ranks}")
    host = [wl.tokens(k, with_segments=True) for k in range(N_BATCHES)]
    tokens = [torch.from_numpy(t).to(dev) for t, _ in host]
    segs = [torch.from_numpy(s_).to(dev) for _, s_ in host]
    table = workloads.make_table(wl.table_rows, wl.dim, wl.seed, dev)
    R, D = wl.batch * local * wl.heads, wl.dim
    rows = torch.empty((wl.batch, local, wl.heads), dtype=torch.int64, device=dev)
    out = torch.empty((R, D), dtype=torch.bfloat16, device=dev)
    hargs = (wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult, wl.primes, wl.offsets)

    def step(k):
        E.engram_lookup_slice(tokens[k % N_BATCHES], a, b, table, *hargs,
                              seq_ids=segs[k % N_BATCHES], out=out)

    def step_separate(k, ev=None):
        if ev is not None:
            ev[0].record(stream)
        E.engram_hash_slice(tokens[k % N_BATCHES], a, b, *hargs, wl.table_rows,
                            seq_ids=segs[k % N_BATCHES], out=rows)
        if ev is not None:
            ev[1].record(stream)
        E.engram_gather(rows, table, out=out)
        if ev is not None:
            ev[2].record(stream)

    def timed(fn):
        for k in range(args.warmup):
            fn(k)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for k in range(args.steps):
            fn(k)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    ms = timed(step)
    sep_ms = timed(step_separate)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        step_separate(k, evs[k])
    torch.cuda.synchronize()
    E.engram_hash_slice(tokens[0], a, b, *hargs, wl.table_rows, seq_ids=segs[0], out=rows)
    hist = wl.ngram_size - 1
    tok_bytes = 8 * wl.batch * (local + hist) * 2  # tokens + seg ids of the slice and its history
    look_bytes = tok_bytes + 4 * D * R
    look_gbps = look_bytes / (ms * 1e-3) / 1e9
    phases = {"lookup": {"ms": ms, "algorithmic_bytes": look_bytes, "gbps": look_gbps,
                         "frac_of_peak": look_gbps / PEAK_HBM_GBS}}
    nbytes = {"hash": tok_bytes + 8 * R, "gather": 8 * R + 4 * D * R}
    sep_phases = {}
    for i, p_ in enumerate(("hash", "gather")):
        pm = float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
        g = nbytes[p_] / (pm * 1e-3) / 1e9
        sep_phases[p_] = {"ms": pm, "algorithmic_bytes": nbytes[p_], "gbps": g,
                          "frac_of_peak": g / PEAK_HBM_GBS}
    cpu = None
    if not args.no_cpu_baseline:
        t_host, s_host = host[0]
        ids = rows.cpu().numpy().reshape(-1)
        tab_bits, folded = host_table(table)
        gather_rows = ids % tab_bits.shape[0] if folded else ids

        def work(o):
            o.hash_global_slice(t_host, a, b, wl.ngram_size, wl.heads_per_ngram, wl.eos_id,
                                mult, wl.primes, wl.offsets, s_host)
            o.gather(gather_rows, tab_bits)
        cpu = cpu_baseline(work, R, "lookups/s",
                           f"one rank's slice ({R} lookups): the oracle hashes the whole "
                           "replicated sequence and keeps the slice, then gathers from a host "
                           f"copy of the table's first {tab_bits.shape[0]} rows with row ids "
                           "folded modulo that count")
    result = {
        "metric": METRIC, "value": R / (ms * 1e-3), "unit": "lookups/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {**wl.describe(), "workload": "cp_slice", "cp_ranks": ranks,
                   "slice": [a, b], "lookups": R, "segments": True,
                   "step": "lookup_slice (hash and gather of the slice in one pass)"},
        "phases": phases,
        "separate_calls": {"ms_per_step": sep_ms, "value": R / (sep_ms * 1e-3),
                           "step": "hash_slice+gather", "phases": sep_phases},
        "roofline": {"bound": "hbm", "kernel": f"lookup_kernel<{wl.ngram_size}> "
                     "(engram_lookup_slice)", "achieved": look_gbps, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": look_gbps / PEAK_HBM_GBS, "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def bench_ple_conv(args, torch, E, workloads):
    """The PLE convolution over one batch of hidden states; a second pass
    with the context-parallel halo (the preceding (K-1) * dilation rows)."""
    wl = workloads.ple_conv()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    B, S, C, K, d = wl.batch, wl.seq, wl.channels, wl.kernel_size, wl.dilation
    log(f"[bench] ple_conv: {wl.describe()}")
    x = workloads.make_bf16((B, S, C), wl.seed, dev)
    w = workloads.make_bf16((C, K), wl.seed + 1, dev, std=0.5)
    bias = workloads.make_bf16((C,), wl.seed + 2, dev, std=0.5)
    seg = torch.from_numpy(wl.segments()).to(dev)
    H = wl.history
    halo = workloads.make_bf16((B, H, C), wl.seed + 3, dev)
    seg_h = torch.from_numpy(wl.segments(halo=H)).to(dev)
    out = torch.empty_like(x)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / max(steps, 1)

    plain = lambda: E.engram_ple_conv(x, w, d, bias=bias, seq_ids=seg, out=out)
    with_halo = lambda: E.engram_ple_conv(x, w, d, bias=bias, seq_ids=seg_h, halo=halo, out=out)
    timed(plain, 0, 20)       # bring the clocks up before either timing
    timed(with_halo, 0, 20)
    ms = timed(plain, args.steps, args.warmup)
    ms_h = timed(with_halo, args.steps, args.warmup)
    nbytes = 2 * B * S * C * 2 + 8 * B * S + 2 * C * (K + 1)
    nbytes_h = nbytes + 2 * B * H * C + 8 * B * H
    gbps, gbps_h = nbytes / (ms * 1e-3) / 1e9, nbytes_h / (ms_h * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        xs = x[0:1, :, :256].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        ws_ = w[:256].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        bs = bias[:256].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        sg = seg[0:1].cpu().numpy()
        cpu = cpu_baseline(lambda o: o.ple_conv(xs, ws_, d, bs, sg), S * 256,
                           "position-channels/s",
                           f"one row x 256 channels ({S * 256} outputs)")
    result = {
        "metric": "PLE conv position-channels/s and achieved HBM GB/s (% of peak)",
        "value": B * S * C / (ms * 1e-3), "unit": "position-channels/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {**wl.describe(), "segments": "packed documents", "bias": True},
        "algorithmic_bytes": nbytes, "gbps": gbps,
        "with_cp_halo": {"halo_rows": H, "ms": ms_h, "algorithmic_bytes": nbytes_h,
                         "gbps": gbps_h},
        "roofline": {"bound": "hbm", "kernel": f"ple_conv_k4_kernel<{d}>", "achieved": gbps,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBS,
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="e2e",
                    choices=["e2e", "e2e_signsgd", "e2e_padtail", "full", "medium", "backward",
                             "cp_slice", "ple_conv"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="the e2e line alone, without the nested configurations")
    ap.add_argument("--settle", type=float, default=0.25,
                    help="seconds of untimed steps before the warm-up steps")
    ap.add_argument("--graphs", action="store_true",
                    help="also time the backward steps captured as HIP graphs and replayed")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X with the whole table in HBM)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from gram_hashed_embedding_amd import engram as E
    from gram_hashed_embedding_amd import workloads

    if args.workload == "cp_slice":
        return bench_cp_slice(args, torch, E, workloads)
    if args.workload == "ple_conv":
        return bench_ple_conv(args, torch, E, workloads)
    result, table = bench_step(args, torch, E, workloads, args.workload)
    dev = torch.device("cuda:0")
    result["copy_probe_gbps"] = copy_probe_gbps(torch, dev, torch.cuda.current_stream(dev))
    if args.workload == "e2e" and not args.no_other_configs:
        others = {}
        for name in ("medium", "full", "backward", "e2e_padtail"):
            res, _ = bench_step(args, torch, E, workloads, name,
                                table=table if name in ("full", "e2e_padtail") else None)
            others[name] = sub_config(res)
            torch.cuda.empty_cache()
        result["other_configs"] = others
    del table
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
