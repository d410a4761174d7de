#!/usr/bin/env python3
"""Benchmark of the HiSparse swap-in path on one MI355X.

A step is one hs_resolve over every request of the workload (one decode step): hit test, LRU victims, page
table update and the copy of every missed row from pinned host memory into HBM. Inputs (the per-step top-k
ids) are staged in HBM before the timed region. The JSON line reports resolved top-k entries/s (the value),
the miss-copy rate against the host link, HBM figures, the roofline of the resolve kernel and the CPU oracle
timed on a bounded sample of the same workload. Further legs, each from a reset on the same stream: the split
step (hs_plan + hs_copy) and the plans alone back to back (the hit path, priced against HBM), the split step
pipelined over two streams, the copy beside independent HBM-bound work, a captured graph, the unfused gather,
the retryable step, and the residency transitions (offload, tail advance). Measured traffic, where given, comes
from a committed rocprofv3 summary of the same sources and workload, beside the algorithmic bytes it is
compared with.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PCIE5_X16_GBPS = 64.0      # MI355X host link, PCIe 5.0 x16, per direction (published)
HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E (published)


def kernel_source_digest() -> str:
    """Digest of the kernel sources' code: comments and blank lines are left out, so a comment edit keeps a
    traffic record taken on the same code valid, and any change to the code itself does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("hs_kernels.hip", "hs_internal.h"):
        with open(os.path.join(ROOT, "hierarchical_memory_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments (no string literal holds one)
        lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
        h.update("\n".join(ln for ln in lines if ln.strip()).encode())
    return h.hexdigest()[:16]


TRAFFIC_SOURCE = "profiles/pmc_traffic.json (rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE of an earlier run on these sources)"


def measured_traffic(workload_name: str, kernel: str):
    """Bytes per launch (reads + writes, HBM and host link together) from the committed rocprofv3 --pmc summary
    (FETCH_SIZE, WRITE_SIZE, each scaled by what the same counter reads for a 1 GiB device copy), or None when
    that summary was taken on other kernel sources or another workload. Not measured in this run."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_digest") != kernel_source_digest() or rec.get("workload") != workload_name:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k["fetch_bytes"] + k["write_bytes"]


def traffic_fields(workload_name: str, kernel: str, algorithmic_total: float) -> dict:
    """The measured traffic beside the algorithmic bytes it is to be compared with: both count reads and writes,
    HBM and host link together."""
    t = measured_traffic(workload_name, kernel)
    return {"traffic": t, "algorithmic_total_bytes": algorithmic_total,
            "traffic_ratio": (t / algorithmic_total) if t and algorithmic_total else None,
            "traffic_source": TRAFFIC_SOURCE if t else None}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=960)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="concurrency_256req_L32768_B4096_k2048")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="buffer-size sweep instead: B in {2048,4096,6144} x keep in {0.6,0.8,0.95}, 64 requests, "
                         "512 steps each; reports the 100-step rolling mean of misses per step and the resolve rate")
    ap.add_argument("--policy", choices=["lru", "fifo", "both"], default="lru",
                    help="eviction policy (--sweep: 'both' runs every (B, keep) under LRU and FIFO)")
    ap.add_argument("--gather-launches", type=int, default=64,
                    help="timed launches of hs_gather on the last step's selection (0: skip)")
    ap.add_argument("--offload-launches", type=int, default=32,
                    help="timed launches of hs_offload (and hs_advance_tail on workloads with a device tail); 0: skip")
    ap.add_argument("--graph-steps", type=int, default=256,
                    help="steps captured in one HIP graph and replayed (0: skip)")
    ap.add_argument("--trial-steps", type=int, default=256,
                    help="steps of the hs_trial + hs_commit leg after a reset (0: skip)")
    ap.add_argument("--split-steps", type=int, default=-1,
                    help="steps of the plan+copy leg after a reset (default: the same warmup+steps)")
    return ap.parse_args()


def link_and_hbm_probes(torch):
    """Measured host-to-device link peak (pinned 1 GiB, hipMemcpyAsync via torch, median of 10), HBM copy rate
    (read + write) and device-to-host link rate (the same copy the other way)."""
    n = 1 << 30
    h = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(n, dtype=torch.uint8, device="cuda")
    d2 = torch.empty(n, dtype=torch.uint8, device="cuda")

    def med(fn, reps=10):
        ts = []
        fn()
        torch.cuda.synchronize()
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        ts.sort()
        return ts[len(ts) // 2]

    link_ms = med(lambda: d.copy_(h, non_blocking=True))
    d2h_ms = med(lambda: h.copy_(d, non_blocking=True))
    hbm_ms = med(lambda: d2.copy_(d))
    del h, d, d2
    torch.cuda.empty_cache()
    return n / link_ms / 1e6, 2 * n / hbm_ms / 1e6, n / d2h_ms / 1e6


def copy_probes(hm, torch, np, sw, w, reps: int = 7):
    """Zero-copy reads of the host pool by the library's own copy kernel, driven by synthetic plans that move
    k rows per request: consecutive host rows into consecutive slots (sequential), and random distinct rows
    into random distinct slots (the pattern of real misses). Median of reps launches each, in GB/s. Run before
    the first step: the slots it fills hold no token yet, and every later use of a slot first copies into it."""
    R, k, B, H, rb = w.num_requests, w.top_k, w.buffer_slots, w.host_rows, w.row_bytes
    m = min(k, H)
    rng = np.random.default_rng(7)
    seq = np.full((R, 4, k), -1, np.int32)  # the plan layout of hs_plan: tokens, slots, evicted tokens, sources
    seq[:, 0, :m] = np.arange(m, dtype=np.int32)
    seq[:, 1, :m] = np.arange(m, dtype=np.int32)
    rnd = np.full((R, 4, k), -1, np.int32)
    for r in range(R):
        rnd[r, 0, :m] = rng.choice(H, size=m, replace=False)
        rnd[r, 1, :m] = rng.choice(B, size=m, replace=False)
    miss = torch.full((R,), m, dtype=torch.int32, device="cuda")
    out = {}
    for name, plan in (("sequential", seq), ("random_rows", rnd)):
        pd = torch.from_numpy(plan).cuda()
        hm.hs_copy(sw.ctx, pd, miss)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            hm.hs_copy(sw.ctx, pd, miss)
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        out[name] = R * m * rb / (sorted(ts)[reps // 2] / 1e3) / 1e9
    return out


def cpu_baseline(w, ids, seconds: float, policy: int = 0):
    """The oracle, as it is, on the first requests of the same streams (its own rows from the generator), on one
    host core: the process is pinned to its first allowed core for this leg (and unpinned after). Timed with
    perf_counter around the oracle's C calls; the sample's rows are drawn before the clock starts."""
    import numpy as np
    import oracle
    import workload
    allowed = sorted(os.sched_getaffinity(0))
    pinned = allowed[0]
    os.sched_setaffinity(0, {pinned})
    try:
        rep = _cpu_baseline_pinned(w, ids, seconds, policy, np, oracle, workload)
    finally:
        os.sched_setaffinity(0, set(allowed))
    rep["pinned_core"] = pinned
    rep["available_cores"] = len(allowed)
    rep["all_cores"] = _oracle_all_cores(w, rep.pop("_sample"), rep.pop("_host"), rep.pop("_tail"), rep.pop("_tail0"),
                                         policy, ids.shape[1])
    return rep


def _cpu_baseline_pinned(w, ids, seconds, policy, np, oracle, workload):
    n_steps = ids.shape[1]
    # size the sample from a short calibration on one request
    cal = oracle.Oracle(1, w.buffer_slots, w.top_k, w.host_rows, w.row_bytes,
                        host=np.zeros((1, w.host_rows, w.row_bytes), np.uint8))
    t0 = time.perf_counter()
    cal_steps = min(n_steps, 64)
    for t in range(cal_steps):
        cal.step(ids[:1, t])
    per_req_step = (time.perf_counter() - t0) / cal_steps
    n_req = max(1, min(w.num_requests, int(seconds / (per_req_step * n_steps))))
    host = np.empty((n_req, w.host_rows, w.row_bytes), np.uint8)
    for j in range(n_req):
        workload.fill_rows(host[j].view(np.uint16).reshape(w.host_rows, w.row_elems), j * w.host_rows, w.host_rows,
                           w.row_elems, w.row_seed)
    tail = tail0 = None
    if w.tail_tokens:
        tail = np.zeros((n_req, w.tail_tokens, w.row_bytes), np.uint8)
        for x in range(w.tail0, w.tail0 + w.tail_tokens):  # the device tail is a ring: token x in row x mod T
            tail[:, x % w.tail_tokens] = host[:, x]
        tail0 = np.full(n_req, w.tail0, np.int32)
    o = oracle.Oracle(n_req, w.buffer_slots, w.top_k, w.host_rows, w.row_bytes, T=w.tail_tokens, host=host, tail=tail,
                      policy=policy)
    sub = np.ascontiguousarray(ids[:n_req])
    misses = 0
    t0 = time.perf_counter()
    for t in range(n_steps):
        _, miss, _, _ = o.step(sub[:, t], tail0, gather=w.fused_gather)
        misses += int(miss.sum())
    dt = time.perf_counter() - t0
    entries = n_req * n_steps * w.top_k
    rep = {"value": entries / dt, "unit": "entries/s", "cores": 1, "kind": "oracle",
           "sample": f"{n_req} of {w.num_requests} requests x all {n_steps} steps ({dt:.1f} s, single thread "
                     f"pinned to one core)",
           "miss_copy_GBps": misses * w.row_bytes / dt / 1e9,
           "_sample": sub, "_host": host, "_tail": tail, "_tail0": tail0}
    return rep


def _oracle_all_cores(w, sub, host, tail, tail0, policy, n_steps):
    """The same oracle on the same sample, its requests split over one thread per available core (at most 16,
    the host share of one GPU); each thread steps its own requests (the C calls release the GIL)."""
    import threading
    import numpy as np
    import oracle
    n_req = sub.shape[0]
    cores = max(1, min(16, len(os.sched_getaffinity(0)), n_req))
    bounds = np.linspace(0, n_req, cores + 1).astype(int)
    parts = []
    for c in range(cores):
        a, b = int(bounds[c]), int(bounds[c + 1])
        o = oracle.Oracle(b - a, w.buffer_slots, w.top_k, w.host_rows, w.row_bytes, T=w.tail_tokens, host=host[a:b],
                          tail=None if tail is None else tail[a:b], policy=policy)
        parts.append((o, np.ascontiguousarray(sub[a:b]), None if tail0 is None else tail0[a:b]))

    def run(o, ids, t0):
        for t in range(n_steps):
            o.step(ids[:, t], t0, gather=w.fused_gather)

    threads = [threading.Thread(target=run, args=part) for part in parts]
    t_start = time.perf_counter()
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    dt = time.perf_counter() - t_start
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": n_req * n_steps * w.top_k / dt, "unit": "entries/s", "cores": cores, "kind": "oracle",
            "sample": f"the same {n_req} requests x {n_steps} steps on {cores} threads ({dt:.1f} s)", "cpu_model": model}


def resolve_kernel_name(sw, mode: str, gather: bool) -> str:
    """The resolve kernel a launch of this shape runs: the direct layout (token -> slot table in LDS) where it
    fits, else the rank layout; the library decides per shape, separately for launches with a gather output."""
    direct = sw.sizes.token_slot_table & (2 if gather else 1)
    return f"{'resolve_direct_kernel' if direct else 'resolve_kernel'}<{mode}>"


def split_leg(hm, torch, np, sw, topk, tail0, W, K, w, mean_miss_per_step, hbm_copy=None):
    """The same stream again from a reset, as hs_plan + hs_copy on one stream. The plan kernel carries all the
    metadata work of a step (hit test, ranks, victims, page/slot tables, stamps, outputs) and no rows, so its
    duration prices the hit path against HBM."""
    R, k, B, rb = w.num_requests, w.top_k, w.buffer_slots, w.row_bytes
    stream = torch.cuda.current_stream()
    sw.reset()
    plan = sw.plan_buffer()
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    miss = torch.zeros((W + K, R), dtype=torch.int32, device="cuda")
    status = torch.zeros((W + K, R), dtype=torch.int32, device="cuda")
    for t in range(W):
        hm.hs_plan(sw.ctx, topk[t], tail0, out, miss[t], status[t], plan, stream)
        hm.hs_copy(sw.ctx, plan, miss[t], stream=stream)
    torch.cuda.synchronize()
    ea = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    eb = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        ea[i].record(stream)
        hm.hs_plan(sw.ctx, topk[W + i], tail0, out, miss[W + i], status[W + i], plan, stream)
        eb[i].record(stream)
        hm.hs_copy(sw.ctx, plan, miss[W + i], stream=stream)
    ea[K].record(stream)
    torch.cuda.synchronize()
    plan_ms = np.array([ea[i].elapsed_time(eb[i]) for i in range(K)])
    copy_ms = np.array([eb[i].elapsed_time(ea[i + 1]) for i in range(K)])
    total_ms = ea[0].elapsed_time(ea[K])
    m = miss[W:].cpu().numpy().astype(np.int64)
    if status[W:].cpu().numpy().any():
        raise SystemExit("device status bits set during the split leg")
    mean_m = m.sum() / K
    # what a plan must move, per request: ids 4k, slot table 4B and order list 2B read; outputs 4k, order list 2B,
    # stamps of the used slots (at most 4k) and the victims' slot-table entries 4m written; the miss list for
    # the copy (token, slot, evicted token) 12m written
    meta = R * (12 * k + 8 * B) + 16 * mean_m
    event_avg = float(plan_ms.mean())
    # The plans alone, back to back from a reset: a plan needs only the metadata the previous plan left (the
    # copies move bytes), so K plans in a row are the hit path run on its own. Two events around the chain
    # leave out the per-launch event overhead that dominates a ~15 us kernel.
    sw.reset()
    for t in range(W):
        hm.hs_plan(sw.ctx, topk[t], tail0, out, miss[t], status[t], plan, stream)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for i in range(K):
        hm.hs_plan(sw.ctx, topk[W + i], tail0, out, miss[W + i], status[W + i], plan, stream)
    c1.record(stream)
    torch.cuda.synchronize()
    if status[W:].cpu().numpy().any():
        raise SystemExit("device status bits set during the plan chain")
    same_chain = bool((miss[W:].cpu().numpy().astype(np.int64) == m).all())
    eager_avg = c0.elapsed_time(c1) / K
    # The same chain captured as one HIP graph and replayed once: the device runs the plans back to back with no
    # host launch in between, so the figure is the GPU's and not the Python launch rate (the launch path checks
    # every tensor argument, a few microseconds per call, close to a plan's own duration).
    sw.reset()
    for t in range(W):
        hm.hs_plan(sw.ctx, topk[t], tail0, out, miss[t], status[t], plan, stream)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(K):
            hm.hs_plan(sw.ctx, topk[W + i], tail0, out, miss[W + i], status[W + i], plan, side)
    torch.cuda.synchronize()
    miss[W:].zero_()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    del graph
    if status[W:].cpu().numpy().any():
        raise SystemExit("device status bits set during the captured plan chain")
    same_chain = same_chain and bool((miss[W:].cpu().numpy().astype(np.int64) == m).all())
    plan_avg = g0.elapsed_time(g1) / K
    hit_gbps = meta / (plan_avg / 1e3) / 1e9
    copy_gbps = mean_m * rb / (float(copy_ms.mean()) / 1e3) / 1e9
    log(f"[bench] split: plan {event_avg * 1e3:.1f} us/step between copies, {plan_avg * 1e3:.2f} us back to back in "
        f"a graph ({eager_avg * 1e3:.2f} us launched one by one; {hit_gbps:.0f} GB/s of metadata), copy "
        f"{copy_ms.mean() * 1e3:.0f} us/step ({copy_gbps:.1f} GB/s), whole step {total_ms / K:.3f} ms")
    return {"kernel": resolve_kernel_name(sw, "plan", False) + " (hs_plan)", "bound": "hbm", "achieved": hit_gbps,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": hit_gbps / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": meta,
            "bytes_model": "per request 12k + 8B + 16m (ids, slot table, order list, outputs, stamps, slot-table "
                           "entries, miss list); the page-table updates ride with hs_copy",
            "frac_of_measured_hbm_copy": (hit_gbps / hbm_copy) if hbm_copy else None,
            "avg_launch_us": plan_avg * 1e3,
            "timing": "K plans back to back, captured as one HIP graph and replayed once between two events",
            "avg_launch_us_eager_chain": eager_avg * 1e3,
            "avg_launch_us_between_copies": event_avg * 1e3, "p50_launch_us_between_copies": float(np.median(plan_ms)) * 1e3,
            "chain_same_misses": same_chain,
            **traffic_fields(w.name, "resolve_plan", meta),
            "copy_kernel_avg_us": float(copy_ms.mean()) * 1e3, "copy_kernel_GBps": copy_gbps,
            "split_step_ms": total_ms / K, "same_misses_as_fused": bool(abs(mean_m - mean_miss_per_step) < 1e-6)}


def overlap_leg(hm, torch, np, sw, topk, tail0, W, K, w):
    """The split path pipelined over two streams from a reset: the plan of step t+1 runs on the launch stream
    while the copy of step t is still in flight on a second stream (plans double-buffered; a plan depends only
    on the previous plan, whose metadata is final when it ends; copies stay in order on their stream). On a
    fused-gather workload the copy also gathers every selected row."""
    R, k = w.num_requests, w.top_k
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    sw.reset()
    plans = [sw.plan_buffer() for _ in range(2)]
    outs = [torch.empty((R, k), dtype=torch.int32, device="cuda") for _ in range(2)]
    miss = torch.zeros((W + K, R), dtype=torch.int32, device="cuda")
    status = torch.zeros((W + K, R), dtype=torch.int32, device="cuda")
    # a fused-gather workload gathers every selected row in the copy (one output: in a decode loop the step's
    # consumer would read it before the next copy)
    g = torch.empty((R, k, w.row_bytes), dtype=torch.uint8, device="cuda") if w.fused_gather else None
    copied = [None, None]

    def step(t):
        b = t % 2
        if copied[b] is not None:
            main.wait_event(copied[b])  # the copy that read this plan buffer is done
        hm.hs_plan(sw.ctx, topk[t], tail0, outs[b], miss[t], status[t], plans[b], main, row_sources=g is not None)
        planned = torch.cuda.Event()
        planned.record(main)
        side.wait_event(planned)
        hm.hs_copy(sw.ctx, plans[b], miss[t], g, stream=side)
        copied[b] = torch.cuda.Event()
        copied[b].record(side)

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(main)
    for t in range(W, W + K):
        step(t)
    main.wait_event(copied[(W + K - 1) % 2])
    end.record(main)
    torch.cuda.synchronize()
    if status[W:].cpu().numpy().any():
        raise SystemExit("device status bits set during the overlap leg")
    ms = start.elapsed_time(end) / K
    m = miss[W:].cpu().numpy().astype(np.int64)
    log(f"[bench] overlapped split: {ms:.3f} ms/step ({K * R * k / (ms * K / 1e3) / 1e6:.1f} M entries/s)")
    return {"step_ms": ms, "entries_per_s": R * k / (ms / 1e3), "miss_copy_GBps": m.sum() * w.row_bytes / K / (ms / 1e3) / 1e9,
            "steps": K, "warmup": W, "gather": w.fused_gather}


def overlap_compute_leg(hm, torch, np, sw, topk, tail0, W, K, w):
    """The copy of a step on a second stream beside independent HBM-bound work on the launch stream, standing in
    for the compute a decode step overlaps the swap-in I/O with: device-to-device copies of a 600 MB buffer,
    repeated to last about as long as the row copy. (A gather of the resident rows would race with the copy's
    writes into the victim slots, so the stand-in touches none of the library's buffers.) Each step is timed
    three ways: the copy alone, the HBM work alone, and both launched together."""
    R, k, rb = w.num_requests, w.top_k, w.row_bytes
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    sw.reset()
    plan = sw.plan_buffer()
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    miss = torch.zeros((R,), dtype=torch.int32, device="cuda")
    status = torch.zeros((R,), dtype=torch.int32, device="cuda")
    src = torch.empty(600 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(main)
        fn()
        b.record(main)
        b.synchronize()
        return a.elapsed_time(b)

    for t in range(W):
        hm.hs_plan(sw.ctx, topk[t], tail0, out, miss, status, plan, main)
        hm.hs_copy(sw.ctx, plan, miss, stream=main)
    torch.cuda.synchronize()
    one = timed(lambda: dst.copy_(src))
    copies = []
    for t in range(W, W + 3):  # the copy's duration at this point of the stream sizes the HBM work
        hm.hs_plan(sw.ctx, topk[t], tail0, out, miss, status, plan, main)
        copies.append(timed(lambda: hm.hs_copy(sw.ctx, plan, miss, stream=main)))
    reps = max(1, int(round(float(np.median(copies)) / one)))

    def hbm_work():
        for _ in range(reps):
            dst.copy_(src)

    def both():
        start = torch.cuda.Event()
        start.record(main)
        side.wait_event(start)
        hm.hs_copy(sw.ctx, plan, miss, stream=side)
        done = torch.cuda.Event()
        done.record(side)
        hbm_work()
        main.wait_event(done)

    alone, work, together = [], [], []
    n = min(K, 3 * 16)
    for i in range(n):
        t = W + 3 + i
        hm.hs_plan(sw.ctx, topk[t], tail0, out, miss, status, plan, main)
        if i % 3 == 0:
            alone.append(timed(lambda: hm.hs_copy(sw.ctx, plan, miss, stream=main)))
        elif i % 3 == 1:
            work.append(timed(hbm_work))
            hm.hs_copy(sw.ctx, plan, miss, stream=main)
        else:
            together.append(timed(both))
    del src, dst
    ca, wa, tg = float(np.median(alone)), float(np.median(work)), float(np.median(together))
    log(f"[bench] copy beside HBM work: copy {ca:.3f} ms, HBM work {wa:.3f} ms ({reps} x 1.2 GB moved), "
        f"together {tg:.3f} ms = {tg / max(ca, wa):.3f} x the longer")
    return {"copy_ms": ca, "hbm_work_ms": wa, "together_ms": tg, "together_over_longer": tg / max(ca, wa),
            "together_over_sum": tg / (ca + wa), "hbm_work": f"{reps} device-to-device copies of 600 MB",
            "hbm_work_GBps": reps * 2 * src_bytes(600) / (wa / 1e3) / 1e9, "copy_workgroups": 128, "copy_threads_per_workgroup": 64,
            "steps": n, "timing": "medians of steps timed one way each, in rotation"}


def src_bytes(mib: int) -> int:
    return mib << 20


def graph_leg(hm, torch, np, sw, topk, tail0, W, K, w, eager_miss):
    """The same stream from a reset, its K timed steps captured as one HIP graph (one hs_resolve node per step,
    each on its own staged ids) and replayed once between two events: the per-launch host overhead is gone,
    which is what decides small workloads. The miss counts must equal the eager run's."""
    R, k = w.num_requests, w.top_k
    sw.reset()
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    miss = torch.zeros((W + K, R), dtype=torch.int32, device="cuda")
    status = torch.zeros((W + K, R), dtype=torch.int32, device="cuda")
    g = torch.empty((R, k, w.row_bytes), dtype=torch.uint8, device="cuda") if w.fused_gather else None
    stream = torch.cuda.current_stream()
    for t in range(W):
        hm.hs_resolve(sw.ctx, topk[t], tail0, out, miss[t], status[t], g, stream)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(K):
            hm.hs_resolve(sw.ctx, topk[W + i], tail0, out, miss[W + i], status[W + i], g, side)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    if status[W:].cpu().numpy().any():
        raise SystemExit("device status bits set during the graph leg")
    same = bool((miss[W:W + K].cpu().numpy() == eager_miss[:K]).all())
    ms = start.elapsed_time(end) / K
    del graph
    log(f"[bench] graph: {ms * 1e3:.1f} us/step ({R * k / (ms / 1e3) / 1e6:.1f} M entries/s) over {K} captured steps")
    return {"step_ms": ms, "entries_per_s": R * k / (ms / 1e3), "steps": K, "warmup": W, "same_misses_as_eager": same}


def gather_leg(hm, torch, np, sw, out, w, n, hbm_copy):
    """hs_gather (the unfused gather) of the last step's selection, n launches timed one by one: every selected
    row is read from its hot slot (or tail row) and written to one [R, k, row] output, so it runs against HBM."""
    R, k, rb = w.num_requests, w.top_k, w.row_bytes
    stream = torch.cuda.current_stream()
    g = torch.empty((R, k, rb), dtype=torch.uint8, device="cuda")
    for _ in range(4):
        hm.hs_gather(sw.ctx, out, g, stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    for i in range(n):
        ev[2 * i].record(stream)
        hm.hs_gather(sw.ctx, out, g, stream)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)])
    valid = int((out >= 0).sum().item())
    # a selected row is read once and written once; an entry with no row writes a zero row
    algo = valid * 2 * rb + (R * k - valid) * rb
    avg = float(ms.mean())
    gbps = algo / (avg / 1e3) / 1e9
    del g
    log(f"[bench] gather: {avg * 1e3:.1f} us/launch, {gbps:.0f} GB/s of rows read + written")
    return {"kernel": "gather_kernel (hs_gather)", "bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS, "algorithmic_bytes_per_launch": algo,
            "avg_launch_us": avg * 1e3, "p50_launch_us": float(np.median(ms)) * 1e3, "launches": n,
            "frac_of_measured_hbm_copy": (gbps / hbm_copy) if hbm_copy else None,
            **traffic_fields(w.name, "gather", algo)}


def _timed_launches(torch, np, n, warm, launch):
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        launch(stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    for i in range(n):
        ev[2 * i].record(stream)
        launch(stream)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)])


OFFLOAD_ROWS = 64  # rows per request per offload / tail advance


def offload_leg(hm, torch, np, sw, w, n, d2h_peak):
    """hs_offload of OFFLOAD_ROWS device rows per request into the host pool (the residency transition from
    device to host), n launches timed one by one. It runs last: it rewrites host rows the other legs read."""
    R, H, rb = w.num_requests, w.host_rows, w.row_bytes
    rows = torch.full((R, OFFLOAD_ROWS, rb), 7, dtype=torch.uint8, device="cuda")
    pos = torch.full((R,), H - OFFLOAD_ROWS, dtype=torch.int32, device="cuda")
    status = torch.zeros(R, dtype=torch.int32, device="cuda")
    ms = _timed_launches(torch, np, n, 4, lambda st: hm.hs_offload(sw.ctx, rows, pos, status, st))
    if status.cpu().numpy().any():
        raise SystemExit("device status bits set during the offload leg")
    link_bytes = R * OFFLOAD_ROWS * rb
    avg = float(ms.mean())
    gbps = link_bytes / (avg / 1e3) / 1e9
    log(f"[bench] offload: {avg * 1e3:.1f} us/launch, {gbps:.1f} GB/s device to host")
    return {"kernel": "offload_kernel (hs_offload)", "bound": "host_link", "rows_per_request": OFFLOAD_ROWS,
            "achieved": gbps, "peak": PCIE5_X16_GBPS, "unit": "GB/s", "frac": gbps / PCIE5_X16_GBPS,
            "frac_of_measured_d2h": (gbps / d2h_peak) if d2h_peak else None, "link_bytes_per_launch": link_bytes,
            "avg_launch_us": avg * 1e3, "p50_launch_us": float(np.median(ms)) * 1e3, "launches": n}


def advance_tail_leg(hm, torch, np, sw, w, tail0, n, d2h_peak):
    """hs_advance_tail by OFFLOAD_ROWS tokens per request per launch on a copy of the tail window starts:
    the leaving tail rows go to the host pool over the link."""
    R, H, rb = w.num_requests, w.host_rows, w.row_bytes
    t0 = tail0.clone()
    if int(t0.max().item()) + (n + 4) * OFFLOAD_ROWS > H:
        return None
    step = torch.full((R,), OFFLOAD_ROWS, dtype=torch.int32, device="cuda")
    status = torch.zeros(R, dtype=torch.int32, device="cuda")
    ms = _timed_launches(torch, np, n, 4, lambda st: hm.hs_advance_tail(sw.ctx, t0, step, status, st))
    if status.cpu().numpy().any():
        raise SystemExit("device status bits set during the tail leg")
    link_bytes = R * OFFLOAD_ROWS * rb
    avg = float(ms.mean())
    gbps = link_bytes / (avg / 1e3) / 1e9
    log(f"[bench] advance tail: {avg * 1e3:.1f} us/launch, {gbps:.1f} GB/s device to host")
    return {"kernel": "advance_tail_kernel (hs_advance_tail)", "bound": "host_link", "rows_per_request": OFFLOAD_ROWS,
            "achieved": gbps, "peak": PCIE5_X16_GBPS, "unit": "GB/s", "frac": gbps / PCIE5_X16_GBPS,
            "frac_of_measured_d2h": (gbps / d2h_peak) if d2h_peak else None, "link_bytes_per_launch": link_bytes,
            "avg_launch_us": avg * 1e3, "p50_launch_us": float(np.median(ms)) * 1e3, "launches": n}


def sweep(args) -> int:
    """Misses per step (mean over requests, 100-step rolling mean) and resolve rate for each (B, keep) of the
    buffer sweep; one JSON line with one entry per run."""
    import numpy as np
    import torch

    import hierarchical_memory_amd as hm
    import workload
    torch.cuda.set_device(0)
    runs = []
    policies = {"lru": [hm.HS_EVICT_LRU], "fifo": [hm.HS_EVICT_FIFO], "both": [hm.HS_EVICT_LRU, hm.HS_EVICT_FIFO]}
    cases = [(w, pol) for w in workload.sweep_workloads() for pol in policies[args.policy]]
    for w, pol in cases:
        R, k, B, H, rb = w.num_requests, w.top_k, w.buffer_slots, w.host_rows, w.row_bytes
        sw = hm.SwapIn(hm.config(R, k, B, 0.0, rb, H, 0, pol))
        workload.fill_rows_ptr(sw.host_pool_address(), 0, R * H, w.row_elems, w.row_seed)
        ids = workload.streams(w)
        topk = torch.from_numpy(np.ascontiguousarray(ids.transpose(1, 0, 2))).cuda()
        out = torch.empty((R, k), dtype=torch.int32, device="cuda")
        miss = torch.zeros((w.steps, R), dtype=torch.int32, device="cuda")
        status = torch.zeros((w.steps, R), dtype=torch.int32, device="cuda")
        stream = torch.cuda.current_stream()
        W = min(args.warmup, w.steps // 4)
        for t in range(W):
            hm.hs_resolve(sw.ctx, topk[t], None, out, miss[t], status[t], None, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for t in range(W, w.steps):
            hm.hs_resolve(sw.ctx, topk[t], None, out, miss[t], status[t], None, stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        if status.cpu().numpy().any():
            raise SystemExit(f"{w.name}: device status bits set")
        m = miss.cpu().numpy().astype(np.float64).mean(axis=1)          # misses per request, per step
        roll = np.convolve(m, np.ones(100) / 100, mode="valid")          # step 99 onwards
        n = w.steps - W
        timed_miss = miss[W:].cpu().numpy().astype(np.int64).sum()
        run = {"policy": "fifo" if pol == hm.HS_EVICT_FIFO else "lru", "buffer_slots": B,
               "keep": w.keep_permille / 1000, "steps": w.steps,
               "miss_per_request_step_rolling100_at": {str(t): round(float(roll[t - 99]), 2)
                                                      for t in (99, 199, 299, 399, w.steps - 1)},
               "miss_per_request_step_mean_after_step_99": round(float(m[99:].mean()), 2),
               "entries_per_s": n * R * k / (ms / 1e3), "ms_per_step": ms / n,
               "miss_copy_GBps": timed_miss * rb / (ms / 1e3) / 1e9}
        log(f"[sweep] {run['policy']} B={B} keep={w.keep_permille / 1000}: misses/request-step {run['miss_per_request_step_mean_after_step_99']}"
            f", {run['ms_per_step']:.3f} ms/step, {run['entries_per_s'] / 1e6:.0f} M entries/s")
        runs.append(run)
        sw.close()
        del topk
    print(json.dumps({"metric": "buffer sweep: misses per request-step (100-step rolling mean) and resolve rate",
                      "workload": "sweep_64req_L65536_k2048", "n_gpus": 1, "data": "synthetic", "runs": runs}),
          flush=True)
    return 0


def trial_leg(hm, torch, np, sw, topk, tail0, W, K, w):
    """The same stream from a reset as hs_trial + hs_commit (every request accepted): the retryable step.
    Its state after the leg equals the resolve leg's; the extra cost is the gather of every selected row
    and the HBM-to-HBM move of the missed rows at commit."""
    R, k, rb = w.num_requests, w.top_k, w.row_bytes
    stream = torch.cuda.current_stream()
    sw.reset()
    trial = sw.trial_buffer()
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    miss = torch.zeros((W + K, R), dtype=torch.int32, device="cuda")
    status = torch.zeros((W + K, R), dtype=torch.int32, device="cuda")
    cstat = torch.zeros((W + K, R), dtype=torch.int32, device="cuda")
    g = torch.empty((R, k, rb), dtype=torch.uint8, device="cuda")
    for t in range(W):
        hm.hs_trial(sw.ctx, topk[t], tail0, out, miss[t], status[t], g, trial, stream)
        hm.hs_commit(sw.ctx, trial, g, None, cstat[t], stream)
    torch.cuda.synchronize()
    ea = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    eb = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        ea[i].record(stream)
        hm.hs_trial(sw.ctx, topk[W + i], tail0, out, miss[W + i], status[W + i], g, trial, stream)
        eb[i].record(stream)
        hm.hs_commit(sw.ctx, trial, g, None, cstat[W + i], stream)
    ea[K].record(stream)
    torch.cuda.synchronize()
    if status[W:].cpu().numpy().any() or cstat[W:].cpu().numpy().any():
        raise SystemExit("device status bits set during the trial leg")
    trial_ms = np.array([ea[i].elapsed_time(eb[i]) for i in range(K)])
    commit_ms = np.array([eb[i].elapsed_time(ea[i + 1]) for i in range(K)])
    total = ea[0].elapsed_time(ea[K])
    mean_m = miss[W:].cpu().numpy().astype(np.int64).sum() / K
    # the commit's bytes per launch: each missed row read from the gather output and written to its slot, the
    # record's four lists and the table entries of each miss (page table twice, slot table), the order list
    # read from the record and written, the record header, and the stamps of the slots used this step (hits
    # and misses, counted on the last step's outputs)
    used = int(((out >= 0) & (out < w.buffer_slots)).sum().item())
    commit_bytes = mean_m * (2 * rb + 16 + 12) + R * (4 * w.buffer_slots + 16) + 4 * used
    commit_avg = float(commit_ms.mean())
    commit_gbps = commit_bytes / (commit_avg / 1e3) / 1e9
    del g
    log(f"[bench] trial+commit: {total / K:.3f} ms/step (trial {trial_ms.mean() * 1e3:.0f} us, commit "
        f"{commit_avg * 1e3:.0f} us, {commit_gbps:.0f} GB/s)")
    return {"steps": K, "warmup": W, "step_ms": total / K, "trial_avg_us": float(trial_ms.mean()) * 1e3,
            "commit_avg_us": commit_avg * 1e3,
            "entries_per_s": K * R * k / (total / 1e3), "miss_rows_per_request_step": mean_m / R,
            "commit": {"kernel": "commit_kernel (hs_commit)", "bound": "hbm", "achieved": commit_gbps,
                       "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": commit_gbps / HBM_PEAK_GBPS,
                       "algorithmic_bytes_per_launch": commit_bytes,
                       "bytes_model": "per request 2 row + 28 bytes per miss, 4B + 16 of order list and header, "
                                      "4 per used slot (the last step's count)"}}


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the swap-in path shards by request with no exchange between GPUs, "
              f"so --gpus {args.gpus} is not run here", file=sys.stderr)
        return 2
    if args.sweep:
        return sweep(args)
    import numpy as np
    import torch

    import hierarchical_memory_amd as hm
    import workload

    by_name = {w.name: w for w in workload.ALL}
    w = by_name[args.workload]
    K, W = args.steps, args.warmup
    # the per-step percentiles come from a pass of their own after the timed steps, so that no event sits
    # between two timed launches; a growing context without room for it times the steps one by one instead
    P = min(128, K)
    if w.grow and w.L0 + W + K + P > w.host_rows:
        P = 0
    n_steps = W + K + P
    R, k, B, H, T, rb = w.num_requests, w.top_k, w.buffer_slots, w.host_rows, w.tail_tokens, w.row_bytes
    if w.grow and w.L0 + n_steps > H:
        raise SystemExit(f"{n_steps} steps outgrow the {H}-row host pool of {w.name}")
    torch.cuda.set_device(0)

    link_peak = hbm_copy = d2h_peak = memcpy_peak = None
    if not args.no_probes:
        link_peak, hbm_copy, d2h_peak = link_and_hbm_probes(torch)
        memcpy_peak = link_peak
        log(f"[bench] measured H2D link {link_peak:.1f} GB/s, D2H link {d2h_peak:.1f} GB/s, "
            f"HBM copy {hbm_copy:.0f} GB/s (read+write)")

    log(f"[bench] {w.name}: R={R} k={k} B={B} host_rows={H} T={T}, warmup {W} + timed {K} steps")
    t0 = time.perf_counter()
    policy = hm.HS_EVICT_FIFO if args.policy == "fifo" else hm.HS_EVICT_LRU
    sw = hm.SwapIn(hm.config(R, k, B, 0.0, rb, H, T, policy))
    workload.fill_rows_ptr(sw.host_pool_address(), 0, R * H, w.row_elems, w.row_seed)
    tail0 = None
    if T:
        pool = sw.host_pool()
        # the device tail is a ring of T rows: token x of the window [tail0, tail0 + T) in row x mod T
        ring = (np.arange(w.tail0, w.tail0 + T) % T)
        tail_rows = np.empty((R, T, rb), np.uint8)
        tail_rows[:, ring] = pool[:, w.tail0:w.tail0 + T]
        sw.tail.copy_(torch.from_numpy(tail_rows))
        tail0 = torch.full((R,), w.tail0, dtype=torch.int32, device="cuda")
    copy_link = None
    if not args.no_probes:
        copy_link = copy_probes(hm, torch, np, sw, w)
        log(f"[bench] zero-copy reads by the copy kernel: sequential rows {copy_link['sequential']:.1f} GB/s, "
            f"random rows {copy_link['random_rows']:.1f} GB/s")
        # the link peak is the faster of the runtime's copy and the sequential zero-copy read
        link_peak = max(link_peak, copy_link["sequential"])
    ids = workload.streams(w, n_steps=n_steps)                      # [R, steps, k]
    topk = torch.from_numpy(np.ascontiguousarray(ids.transpose(1, 0, 2))).cuda()  # [steps, R, k] in HBM
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    miss = torch.zeros((n_steps, R), dtype=torch.int32, device="cuda")
    status = torch.zeros((n_steps, R), dtype=torch.int32, device="cuda")
    g = torch.empty((R, k, rb), dtype=torch.uint8, device="cuda") if w.fused_gather else None
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t0:.1f} s (pool {R * H * rb / 1e9:.2f} GB pinned)")

    stream = torch.cuda.current_stream()
    cold = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for t in range(W):
        if t == 0:
            cold[0].record(stream)
        hm.hs_resolve(sw.ctx, topk[t], tail0, out, miss[t], status[t], g, stream)
        if t == 0:
            cold[1].record(stream)
    torch.cuda.synchronize()
    cold_ms = cold[0].elapsed_time(cold[1]) if W else None
    log(f"[bench] warmup done")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()   # one process, one GPU: the barrier is this synchronize
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(K):
        if P == 0 and i:
            evs[i].record(stream)
        hm.hs_resolve(sw.ctx, topk[W + i], tail0, out, miss[W + i], status[W + i], g, stream)
    evs[K].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    elapsed_ms = evs[0].elapsed_time(evs[K])
    if P:
        pev = [torch.cuda.Event(enable_timing=True) for _ in range(P + 1)]
        for i in range(P):
            pev[i].record(stream)
            hm.hs_resolve(sw.ctx, topk[W + K + i], tail0, out, miss[W + K + i], status[W + K + i], g, stream)
        pev[P].record(stream)
        torch.cuda.synchronize()
        per = np.array([pev[i].elapsed_time(pev[i + 1]) for i in range(P)])
    else:
        per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(K)])
    st = status[W:].cpu().numpy()
    if st.any():
        raise SystemExit(f"device status bits set during the timed steps: {np.unique(st)}")
    m = miss[W:W + K].cpu().numpy().astype(np.int64)
    total_miss = int(m.sum())
    secs = elapsed_ms / 1e3
    entries = K * R * k
    value = entries / secs
    miss_bytes = total_miss * rb
    miss_gbps = miss_bytes / secs / 1e9
    launch_ms = elapsed_ms / K
    # algorithmic HBM bytes of one resolve: per request 4k ids read + 4B slot table read + 4B LRU state read and
    # write (2B order list each way) + 4k outputs + stamps of hits and misses + 12 per miss (slot table, page
    # entry, evicted page entry) + the fetched rows written; fused gather adds k rows written and hit/tail rows read
    meta = R * (12 * k + 8 * B) + 12 * total_miss / K
    hbm_bytes = meta + miss_bytes / K
    if w.fused_gather:
        hbm_bytes += R * k * rb + (R * k - total_miss / K) * rb
    hbm_gbps = hbm_bytes / (launch_ms / 1e3) / 1e9
    log(f"[bench] {K} steps in {elapsed_ms:.1f} ms ({launch_ms:.3f} ms/step, wall {wall:.2f} s): "
        f"{value / 1e6:.1f} M entries/s, misses/request-step {total_miss / (K * R):.1f}, miss copy {miss_gbps:.1f} GB/s")
    rep = {
        "metric": "resolved top-k entries/s + miss-copy GB/s vs host-link & HBM peak, 1 GPU",
        "value": value,
        "unit": "entries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": launch_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": w.name, "requests": R, "top_k": k, "buffer_slots": B, "host_rows": H,
                   "tail_tokens": T, "row_bytes": rb, "fused_gather": w.fused_gather,
                   "eviction_policy": "fifo" if policy == hm.HS_EVICT_FIFO else "lru",
                   "timed_steps": [W, W + K]},
        "miss_copy_GBps": miss_gbps,
        "miss_rows_per_request_step": total_miss / (K * R),
        "measured_link_peak_GBps": link_peak,
        "measured_link_probes_GBps": None if copy_link is None else
        dict(copy_link, hipMemcpyAsync=memcpy_peak),
        "miss_copy_frac_of_measured_link": (miss_gbps / link_peak) if link_peak else None,
        "miss_copy_frac_of_random_row_probe": (miss_gbps / copy_link["random_rows"]) if copy_link else None,
        "measured_hbm_copy_GBps": hbm_copy,
        "step_ms_p10_p50_p90": [float(np.percentile(per, q)) for q in (10, 50, 90)],
        "step_percentiles_from": (f"{P} further steps, one event each" if P else "the timed steps, one event each"),
        "cold_step0_ms": cold_ms,
        "cold_step0_misses_per_request": float(miss[0].float().mean().item()) if W else None,
        "measured_d2h_link_GBps": d2h_peak,
        "roofline": {"bound": "host_link", "achieved": miss_gbps, "peak": PCIE5_X16_GBPS, "unit": "GB/s",
                     "frac": miss_gbps / PCIE5_X16_GBPS,
                     "kernel": resolve_kernel_name(sw, "fused", w.fused_gather) + " (hs_resolve)",
                     "algorithmic_bytes_per_launch": miss_bytes / K,
                     **traffic_fields(w.name, "resolve_fused", miss_bytes / K + hbm_bytes)},
        "hbm": {"achieved": hbm_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": hbm_gbps / HBM_PEAK_GBPS,
                "algorithmic_bytes_per_launch": hbm_bytes},
    }
    if args.graph_steps > 0:
        kg = min(args.graph_steps, K)
        rep["graph"] = graph_leg(hm, torch, np, sw, topk, tail0, W, kg, w, m)
    if args.gather_launches > 0:
        rep["gather"] = gather_leg(hm, torch, np, sw, out, w, args.gather_launches, hbm_copy)
    if args.split_steps != 0:
        rep["hit_path"] = split_leg(hm, torch, np, sw, topk, tail0, W, K if args.split_steps < 0 else args.split_steps,
                                    w, total_miss / K, hbm_copy)
    if args.split_steps != 0:
        rep["overlap"] = overlap_leg(hm, torch, np, sw, topk, tail0, W, K if args.split_steps < 0 else args.split_steps, w)
        if not w.fused_gather:
            rep["overlap_with_compute"] = overlap_compute_leg(hm, torch, np, sw, topk, tail0, W,
                                                              K if args.split_steps < 0 else args.split_steps, w)
    if args.trial_steps > 0:
        kt = min(args.trial_steps, K)
        rep["trial_commit"] = trial_leg(hm, torch, np, sw, topk, tail0, W, kt, w)
    if args.offload_launches > 0:
        rep["offload"] = offload_leg(hm, torch, np, sw, w, args.offload_launches, d2h_peak)
        if T:
            rep["advance_tail"] = advance_tail_leg(hm, torch, np, sw, w, tail0, args.offload_launches, d2h_peak)
    sw.close()
    del topk
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        rep["cpu_baseline"] = cpu_baseline(w, ids, args.cpu_seconds, policy)
        log(f"[bench] CPU oracle: {rep['cpu_baseline']['value'] / 1e6:.2f} M entries/s ({rep['cpu_baseline']['sample']})")
    print(json.dumps(rep), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
