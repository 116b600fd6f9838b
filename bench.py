"""Benchmark of the balanced expert-parallel hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic router output:
moonep_plan -> moonep_dispatch -> moonep_combine (-> moonep_reduce_grad when the workload
carries replica gradients).  The expert between dispatch and combine is the identity
(y = recv), so combine reads exactly what dispatch wrote.

Default workload: DeepSeek-V3-shaped, R=8 simulated ranks, E=256, K=8, S=4096 tokens per
rank, H=7168 bf16, 32 prefetch slots per rank, router imbalance swept over maxvio
0.2 / 1 / 5 / 20; the timed steps cycle through the four batches.

value = algorithmic dispatch+combine bytes of the timed steps / wall time of the timed
steps (plan included).  Algorithmic bytes per token: dispatch (K+1)*2H + 4K (read x and
K row indices, write K rows), combine (K+1)*2H + 8K (read K rows, K indices and K
weights, write one row); padding rows are not counted.

Prints one JSON line on stdout; progress goes to stderr.
"""

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0   # MI355X HBM3E, vendor figure


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dispatch_bytes(T, K, H):
    return T * (K + 1) * 2 * H + T * 4 * K


def combine_bytes(T, K, H):
    return T * (K + 1) * 2 * H + T * 8 * K


def reduce_bytes(plan_pieces, G_el):
    # per expert with n slot replicas: read home + n replicas, write home
    per = {}
    for (e, r, slot) in plan_pieces:
        if slot >= 0:
            per[e] = per.get(e, 0) + 1
    return sum((n + 2) * 4 * G_el for n in per.values())


def pctl(vals, q):
    """q-th percentile of a list (linear interpolation between order statistics)."""
    v = sorted(vals)
    x = (len(v) - 1) * q / 100.0
    lo = int(x)
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (x - lo)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_traffic(kernel_prefix, workload):
    """HBM bytes per launch of one kernel, from the committed rocprofv3 counter record
    (FETCH_SIZE and WRITE_SIZE, each scaled by a 4 GiB copy's reading).  None when there
    is no record for this workload or the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_pmc_traffic.txt")
    src = os.path.join(ROOT, "combine_top_id_amd", "csrc", "moonep_move.hip")
    if not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    rec = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        key, val = line.split(":", 1)
        rec.setdefault(key.strip(), []).append(val.strip())
    if rec.get("source_sha256", [""])[0] != sha:
        return None
    for val in rec.get("kernel", []):
        name, _fetch, _write, calibrated, _alg = [v.strip() for v in val.split("|")]
        if name.startswith(kernel_prefix):
            return int(calibrated)
    return None


def cpu_baseline(wl, ids_np, w_np, x_np, home=None, rep=None, budget_s=20.0):
    """The oracle, as it stands, on a bounded sample of the same workload: each stage timed
    on its own (time.perf_counter, median of 3).  Plan and slot map run on the whole batch;
    dispatch and combine on its first n tokens, n sized to fit the time budget; the
    replica-gradient reduce (workloads that carry gradients) on the leading columns of the
    gradient slabs."""
    import numpy as np
    from oracle import moonep_oracle as O

    def med3(fn):
        ts = []
        for _ in range(3):
            t = time.perf_counter()
            r = fn()
            ts.append(time.perf_counter() - t)
        return statistics.median(ts), r

    t_plan, p = med3(lambda: O.plan(ids_np, wl.R, wl.E, wl.K, wl.S, wl.slots))
    t_map, dst = med3(lambda: O.slot_map(p, ids_np))
    rows_total = wl.R * p.sz.NvS

    # size the dispatch+combine sample: one probe on 2048 tokens (smaller probes carry
    # more fixed cost per token), then n tokens so that three repetitions of both stages
    # take about budget_s
    probe = min(2048, wl.T)
    t = time.perf_counter()
    r = O.dispatch(dst[:probe], x_np[:probe], rows_total)
    O.combine(dst[:probe], w_np[:probe], r)
    per_tok = (time.perf_counter() - t) / probe
    del r
    n = int(min(wl.T, max(probe, budget_s / 3 / max(per_tok, 1e-9))))
    d, xs, ws = dst[:n], x_np[:n], w_np[:n]
    t_disp, recv = med3(lambda: O.dispatch(d, xs, rows_total))
    t_comb, _ = med3(lambda: O.combine(d, ws, recv))
    del recv
    db, cb = dispatch_bytes(n, wl.K, wl.H), combine_bytes(n, wl.K, wl.H)
    stages = {
        "plan_ms": round(t_plan * 1e3, 3),
        "slot_map_ms": round(t_map * 1e3, 3),
        "dispatch_ms": round(t_disp * 1e3, 3), "dispatch_gbps": round(db / t_disp / 1e9, 4),
        "combine_ms": round(t_comb * 1e3, 3), "combine_gbps": round(cb / t_comb / 1e9, 4),
    }
    sample = (f"plan and slot map of the whole maxvio={wl.maxvio[0]} batch ({wl.T} tokens); "
              f"dispatch and combine of its first {n} tokens")
    if home is not None and p.n_replicas:
        cols = min(home.shape[1], 1 << 18)
        h_np = home[:, :cols].cpu().numpy()
        r_np = rep[:, :, :cols].cpu().numpy()
        t_red, _ = med3(lambda: O.reduce_grad(p, h_np, r_np))
        per = {}
        for q in p.pieces:
            if q[2] >= 0:
                per[int(q[0])] = per.get(int(q[0]), 0) + 1
        rb = sum((c + 2) * 4 * cols for c in per.values())
        stages.update(reduce_ms=round(t_red * 1e3, 3), reduce_gbps=round(rb / t_red / 1e9, 4))
        sample += f"; replica-gradient reduce over the first {cols} columns of each slab"
    return {
        "value": round((db + cb) / (t_disp + t_comb) / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": sample + "; each stage median of 3; numpy, 1 thread",
        "stages": stages,
        "host_cpus": len(os.sched_getaffinity(0)),
        "host_cpu_model": cpu_model(),
    }


def ceilings(wl, x, recv, out, dev, reps=10):
    """Plain 16-byte streams on the same GPU (libmoonep_streams.so): a linear read, write
    and copy of 4 GiB, and the row mixes of dispatch (one row read, K rows written) and
    combine (K rows read, one row written) on this workload's rows, to contiguous rows and
    to a seeded random permutation of the rows, and the combine backward's (one row and K
    permuted rows read, those K rows written to a second buffer); GB/s, median of `reps`
    launches."""
    import numpy as np
    import torch
    from combine_top_id_amd import streams as ST

    def med(fn):
        for _ in range(2):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(); fn(); b.record()
        torch.cuda.synchronize()
        return statistics.median([a.elapsed_time(b) * 1e3 for a, b in ev])   # us

    res = {}
    n4 = 4 << 30
    a = torch.empty(n4, dtype=torch.uint8, device=dev)
    b = torch.empty(n4, dtype=torch.uint8, device=dev)
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    res["read_linear"] = round(n4 / med(lambda: ST.read(a, sink)) / 1e3, 1)
    res["write_linear"] = round(n4 / med(lambda: ST.write(a)) / 1e3, 1)
    res["copy_linear"] = round(n4 / med(lambda: ST.copy(a[:n4 // 2], b[:n4 // 2])) / 1e3, 1)
    del a, b
    T, K, H = wl.T, wl.K, wl.H
    A = T * K
    rb = 2 * H
    ident = torch.arange(A, dtype=torch.int32, device=dev)
    perm = torch.from_numpy(np.random.default_rng(20260001).permutation(A).astype(np.int32)).to(dev)
    fan_rw, fan_w = T * (K + 1) * rb, T * K * rb
    res["fanout_contiguous"] = round(fan_rw / med(lambda: ST.fanout(ident, K, x, recv)) / 1e3, 1)
    res["fanout_scattered"] = round(fan_rw / med(lambda: ST.fanout(perm, K, x, recv)) / 1e3, 1)
    res["write_scattered_rows"] = round(
        fan_w / med(lambda: ST.fanout(perm, K, None, recv, read_src=False)) / 1e3, 1)
    res["gather_contiguous"] = round(fan_rw / med(lambda: ST.gather(ident, K, recv, out)) / 1e3, 1)
    res["gather_scattered"] = round(fan_rw / med(lambda: ST.gather(perm, K, recv, out)) / 1e3, 1)
    res["read_scattered_rows"] = round(
        fan_w / med(lambda: ST.gather(perm, K, recv, out, write_dst=False)) / 1e3, 1)
    # the combine backward's mix: a source row and K rows of recv read, the K rows written
    # to a second receive-shaped buffer
    upd = torch.empty_like(recv)
    res["update_scattered"] = round(
        T * (2 * K + 1) * rb / med(lambda: ST.update(perm, K, x, recv, upd)) / 1e3, 1)
    del upd
    res["unit"] = "GB/s"
    res["rows"] = (f"{T} source rows x K={K} of {rb} B; random destination rows are a seeded "
                   f"permutation of {A} rows; fan-out and gather one 64-lane workgroup per row "
                   f"chunk (2 KB fan-out, 1 KB gather), update one workgroup per source row, "
                   f"linear streams 256 lanes per 4 KB")
    return res


def device_facts(dev):
    """What the figures depend on beyond the code: the GPU and its HBM (read-only queries).
    Boxes of the same model differ; scattered-row writes in particular ran about 20%
    faster on one box than on the others measured."""
    import re
    import shutil
    import subprocess
    import torch
    p = torch.cuda.get_device_properties(dev)
    facts = {"arch": p.gcnArchName, "compute_units": p.multi_processor_count,
             "memory_gb": round(p.total_memory / 1e9, 1), "memory_vendor": None, "mclk_mhz": None}
    smi = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    try:
        out = subprocess.run([smi, "--showmemvendor", "--showclocks"], capture_output=True,
                             text=True, timeout=30).stdout
        v = re.search(r"memory vendor:\s*(\S+)", out)
        m = re.search(r"mclk clock level:.*\((\d+)\s*Mhz\)", out)
        facts["memory_vendor"] = v.group(1) if v else None
        facts["mclk_mhz"] = int(m.group(1)) if m else None
    except (OSError, subprocess.SubprocessError):
        pass
    return facts


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-prefetch", action="store_true")
    ap.add_argument("--no-staged", action="store_true")
    ap.add_argument("--flush", choices=("auto", "on", "off"), default="auto",
                    help="read a 1 GiB buffer before every step so no input is served from "
                         "the 256 MB last-level cache (auto: when a step moves < 2 GB)")
    ap.add_argument("--no-ceilings", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: R expert-parallel ranks are simulated as HBM "
              "partitions of a single MI355X, and nothing here uses a second GPU "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import combine_top_id_amd as M
    from gen import BY_NAME, make_routing, make_hidden, make_grads, bf16_bits

    wl = BY_NAME[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"workload {wl.name}: R={wl.R} E={wl.E} K={wl.K} S={wl.S} H={wl.H} slots={wl.slots} "
        f"maxvio={wl.maxvio}")

    batches = []
    for mi, mv in enumerate(wl.maxvio):
        ids, w, alpha, got = make_routing(wl.R, wl.E, wl.K, wl.S, mv, wl.seed(mi), device=dev)
        x = make_hidden(wl.T, wl.H, wl.seed(mi) + 1, device=dev)
        batches.append(dict(maxvio=mv, achieved=got, ids=ids, w=w, x=x))
        log(f"  batch maxvio={mv}: achieved {got:.3f}")

    sz = M.moonep_query(wl.R, wl.E, wl.K, wl.S, wl.slots)
    recv = torch.empty(sz.recv_rows, wl.H, dtype=torch.bfloat16, device=dev)
    out = torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device=dev)
    home = rep = None
    if wl.G_el:
        home, rep = make_grads(wl.E, wl.R, wl.slots, wl.G_el, wl.seed(0) + 3, device=dev)
    plan = None
    stream = torch.cuda.current_stream()

    def step(b, ev=None):
        nonlocal plan
        if ev: ev[0].record(stream)
        plan = M.moonep_plan(b["ids"], b["w"], wl.R, wl.E, wl.K, wl.S, wl.slots, plan=plan)
        if ev: ev[1].record(stream)
        M.moonep_dispatch(plan, b["x"], recv)
        if ev: ev[2].record(stream)
        M.moonep_combine(plan, recv, out)
        if ev: ev[3].record(stream)
        if home is not None:
            M.moonep_reduce_grad(plan, home, rep)
            if ev: ev[4].record(stream)

    nb = len(batches)
    stats = []
    for b in batches:
        step(b)
        stats.append(M.moonep_plan_status(plan))
        b["pieces"] = [tuple(int(v) for v in q[:3])
                       for q in plan.array("pieces", plan.sz.P_max * 8).view(-1, 8)
                       [:stats[-1]["n_pieces"]].cpu().tolist()]
    for s in range(args.warmup):
        step(batches[s % nb])
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    nev = 5 if home is not None else 4
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    step_bytes = dispatch_bytes(wl.T, wl.K, wl.H) + combine_bytes(wl.T, wl.K, wl.H)
    flush = args.flush == "on" or (args.flush == "auto" and step_bytes < 2e9)
    scrub = torch.ones(1 << 30, dtype=torch.uint8, device=dev) if flush else None
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    if flush:
        from combine_top_id_amd import streams as ST
    # the timed pass: exactly `steps` steps, no instrumentation between the kernels (with
    # flushing, one event pair brackets each step so the flush itself is not counted)
    spans = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if flush:
            # a plain-load read of 1 GiB (4x the last-level cache) displaces the step's
            # inputs and leaves no dirty lines behind; not inside a step
            ST.read(scrub, sink, policy=0)
            spans[s][0].record(stream)
        step(batches[s % nb])
        if flush:
            spans[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # with flushing, the timed work is the sum of the steps' own event spans
    timed = (sum(a.elapsed_time(b) for a, b in spans) * 1e-3) if flush else wall
    log(f"timed {args.steps} steps in {wall * 1e3:.2f} ms (steps themselves {timed * 1e3:.2f} ms)")

    # the instrumented pass, after the timed one: the same steps again with HIP events
    # between the kernels, for the per-stage figures (not part of `value`)
    for s in range(args.steps):
        if flush:
            ST.read(scrub, sink, policy=0)
        step(batches[s % nb], events[s])
    torch.cuda.synchronize()

    per = [dict(plan=[], disp=[], comb=[], red=[]) for _ in range(nb)]
    for s in range(args.steps):
        ev = events[s]
        d = per[s % nb]
        d["plan"].append(ev[0].elapsed_time(ev[1]) * 1e3)
        d["disp"].append(ev[1].elapsed_time(ev[2]) * 1e3)
        d["comb"].append(ev[2].elapsed_time(ev[3]) * 1e3)
        if home is not None:
            d["red"].append(ev[3].elapsed_time(ev[4]) * 1e3)

    db = dispatch_bytes(wl.T, wl.K, wl.H)
    cb = combine_bytes(wl.T, wl.K, wl.H)
    rows = []
    for b, d, st in zip(batches, per, stats):
        if not d["disp"]:
            continue      # fewer timed steps than batches
        td, tc = statistics.median(d["disp"]), statistics.median(d["comb"])
        row = dict(maxvio=b["maxvio"], achieved_maxvio=round(b["achieved"], 3),
                   plan_us=round(statistics.median(d["plan"]), 2),
                   dispatch_us=round(td, 2), combine_us=round(tc, 2),
                   p10_p90_us={k: [round(pctl(d[v], 10), 2), round(pctl(d[v], 90), 2)]
                               for k, v in (("plan", "plan"), ("dispatch", "disp"),
                                            ("combine", "comb"))},
                   dispatch_gbps=round(db / td / 1e3, 1), combine_gbps=round(cb / tc / 1e3, 1),
                   dc_gbps=round((db + cb) / (td + tc) / 1e3, 1),
                   plan_plus_combine_us=round(statistics.median(
                       [a + b for a, b in zip(d["plan"], d["comb"])]), 2),
                   n_replicas=st["n_replicas"], n_fallback=st["n_fallback"],
                   max_pieces_per_rank=st["max_pieces_per_rank"])
        if home is not None:
            tr = statistics.median(d["red"])
            rb = reduce_bytes(b["pieces"], wl.G_el)
            row.update(reduce_us=round(tr, 2), reduce_gbps=round(rb / tr / 1e3, 1))
        rows.append(row)

    # plan latency back to back: 20 plans of the first batch between one event pair (the
    # event-bracketed figures above include the launch latency after each event)
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    b0 = batches[0]
    for _ in range(3):
        plan = M.moonep_plan(b0["ids"], b0["w"], wl.R, wl.E, wl.K, wl.S, wl.slots, plan=plan)
    pe[0].record(stream)
    for _ in range(20):
        plan = M.moonep_plan(b0["ids"], b0["w"], wl.R, wl.E, wl.K, wl.S, wl.slots, plan=plan)
    pe[1].record(stream)
    torch.cuda.synchronize()
    plan_b2b_us = pe[0].elapsed_time(pe[1]) * 1e3 / 20

    all_d = [v for d in per for v in d["disp"]]
    all_c = [v for d in per for v in d["comb"]]
    mean_d, mean_c = statistics.mean(all_d), statistics.mean(all_c)
    if mean_c >= mean_d:
        dom, dom_bytes, dom_us = "combine", cb, mean_c
    else:
        dom, dom_bytes, dom_us = "dispatch", db, mean_d
    achieved = dom_bytes / dom_us / 1e3
    dc_times = [r["dispatch_us"] + r["combine_us"] for r in rows]

    # backward pair on the first batch, reusing its plan: dispatch-bwd of a gradient laid
    # out like recv, combine-bwd of a gradient laid out like out (y = recv)
    backward = None
    if not args.no_backward:
        b0 = batches[0]
        plan = M.moonep_plan(b0["ids"], b0["w"], wl.R, wl.E, wl.K, wl.S, wl.slots, plan=plan)
        M.moonep_dispatch(plan, b0["x"], recv)
        g_y = torch.empty_like(recv)
        dw = torch.empty(wl.T, wl.K, dtype=torch.float32, device=dev)
        gx = torch.empty_like(out)
        dout = b0["x"]                       # any bf16 [T, H] gradient
        reps = 10
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        M.moonep_combine_bwd(plan, dout, recv, g_y, dw)
        M.moonep_dispatch_bwd(plan, g_y, gx)
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(reps):
            M.moonep_combine_bwd(plan, dout, recv, g_y, dw)
        ev[1].record(stream)
        for _ in range(reps):
            M.moonep_dispatch_bwd(plan, g_y, gx)
        ev[2].record(stream)
        torch.cuda.synchronize()
        tcb = ev[0].elapsed_time(ev[1]) * 1e3 / reps
        tdb = ev[1].elapsed_time(ev[2]) * 1e3 / reps
        cbb = wl.T * (2 * wl.K + 1) * 2 * wl.H + wl.T * 12 * wl.K
        dbb = dispatch_bytes(wl.T, wl.K, wl.H)
        backward = dict(combine_bwd_us=round(tcb, 2), combine_bwd_gbps=round(cbb / tcb / 1e3, 1),
                        dispatch_bwd_us=round(tdb, 2), dispatch_bwd_gbps=round(dbb / tdb / 1e3, 1),
                        bytes_per_token="combine_bwd (2K+1)*2H + 12K; dispatch_bwd (K+1)*2H + 4K")
        del g_y, dw, gx

    # zero-copy vs staged (non-zero-copy) A/B on the first batch: the staged path adds an
    # epilogue row copy to dispatch and a prologue row copy to combine
    staged = None
    if not args.no_staged:
        b0 = batches[0]
        plan = M.moonep_plan(b0["ids"], b0["w"], wl.R, wl.E, wl.K, wl.S, wl.slots, plan=plan)
        stage = torch.empty(wl.A, wl.H, dtype=torch.bfloat16, device=dev)
        M.moonep_dispatch_staged(plan, b0["x"], recv, stage)
        M.moonep_combine_staged(plan, recv, out, stage)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        reps = 10
        ev[0].record(stream)
        for _ in range(reps):
            M.moonep_dispatch(plan, b0["x"], recv)
        ev[1].record(stream)
        for _ in range(reps):
            M.moonep_dispatch_staged(plan, b0["x"], recv, stage)
        ev[2].record(stream)
        for _ in range(reps):
            M.moonep_combine(plan, recv, out)
        ev[3].record(stream)
        for _ in range(reps):
            M.moonep_combine_staged(plan, recv, out, stage)
        ev[4].record(stream)
        torch.cuda.synchronize()
        t = [ev[i].elapsed_time(ev[i + 1]) * 1e3 / reps for i in range(4)]
        staged = dict(dispatch_zero_copy_us=round(t[0], 2), dispatch_staged_us=round(t[1], 2),
                      combine_zero_copy_us=round(t[2], 2), combine_staged_us=round(t[3], 2),
                      staged_over_zero_copy=round((t[1] + t[3]) / (t[0] + t[2]), 3))
        del stage

    # replica weight prefetch on the first batch's plan, DeepSeek-V3-shaped experts:
    # three 7168 x 2048 bf16 matrices (88 MB) per expert
    prefetch = None
    if not args.no_prefetch:
        W_el = 3 * 7168 * 2048
        b0 = batches[0]
        plan = M.moonep_plan(b0["ids"], b0["w"], wl.R, wl.E, wl.K, wl.S, wl.slots, plan=plan)
        st0 = M.moonep_plan_status(plan)
        home_w = torch.empty(wl.E, W_el, dtype=torch.bfloat16, device=dev)
        slot_w = torch.empty(wl.R, wl.slots, W_el, dtype=torch.bfloat16, device=dev)
        M.moonep_prefetch_weight(plan, home_w, slot_w)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        reps = 10
        ev[0].record(stream)
        for _ in range(reps):
            M.moonep_prefetch_weight(plan, home_w, slot_w)
        ev[1].record(stream)
        torch.cuda.synchronize()
        tp = ev[0].elapsed_time(ev[1]) * 1e3 / reps
        pb = st0["n_replicas"] * 2 * W_el * 2
        prefetch = dict(replicas=st0["n_replicas"], expert_bytes=2 * W_el, prefetch_us=round(tp, 2),
                        gbps=round(pb / tp / 1e3, 1) if st0["n_replicas"] else None)
        del home_w, slot_w

    # plain memory streams on the same GPU: the ceilings the kernels are set against
    ceil = None
    if not args.no_ceilings:
        log("ceilings ...")
        ceil = ceilings(wl, batches[0]["x"], recv, out, dev)
        ceil["dispatch_over_fanout_scattered"] = round(
            db / statistics.median(all_d) / 1e3 / ceil["fanout_scattered"], 4)
        ceil["combine_over_gather_scattered"] = round(
            cb / statistics.median(all_c) / 1e3 / ceil["gather_scattered"], 4)
        if backward is not None:
            ceil["combine_bwd_over_update_scattered"] = round(
                backward["combine_bwd_gbps"] / ceil["update_scattered"], 4)

    value = args.steps * (db + cb) / timed / 1e9
    res = {
        "metric": "dispatch+combine GB/s & % HBM peak; plan µs, across maxvio 0.2–20",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(timed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: R={wl.R} simulated ranks, E={wl.E}, K={wl.K}, "
                        f"S={wl.S} tokens/rank, H={wl.H} bf16, slots={wl.slots}, maxvio "
                        f"sweep {'/'.join(str(m) for m in wl.maxvio)} (steps cycle through "
                        f"the batches); identity expert",
            "R": wl.R, "E": wl.E, "K": wl.K, "S": wl.S, "H": wl.H, "slots": wl.slots,
            "tokens": wl.T, "accumulate": "fp32",
            "cache": "flushed before every step by a plain-load read of 1 GiB (no dirty lines); "
                     "value from the steps' own event spans"
                     if flush else "not flushed (working set far above the 256 MB cache)",
        },
        "pct_hbm_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": measured_traffic(dom + "_kernel", wl.name),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, calibrated)",
            "algorithmic_bytes": dom_bytes,
        },
        "per_maxvio": rows,
        "flatness_max_over_min": round(max(dc_times) / min(dc_times), 4),
        "plan_us_median": round(statistics.median([r["plan_us"] for r in rows]), 2),
        "plan_us_back_to_back": round(plan_b2b_us, 2),
        "ceilings": ceil,
        "device": device_facts(dev),
        "backward": backward,
        "prefetch": prefetch,
        "zero_copy_ab": staged,
    }
    if not args.no_cpu_baseline:
        b0 = batches[0]
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(wl, b0["ids"].cpu().numpy(), b0["w"].cpu().numpy(),
                                           bf16_bits(b0["x"]), home, rep)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
