"""Benchmark of the batched on-device sampler on one MI355X.

One step = one call of the hot path over one batch of synthetic logits that
are already resident in HBM.  The headline is sampling: arcs_sample on the
B=256, V=129,280 bf16 batch of Zipf-shaped logits with T=0.7, top_k=50,
top_p=0.9, min_p=0.05 on every row (66.2 MB of logits per step).  The other
named workloads are timed after it, each as a sub-record with its own
entry point, kernel, time per step, rows/s and roofline:
  normal_b4_bf16                   B=4 rows, temperature only (small batch)
  zipf_b256_bf16_greedy            argmax only (arcs_argmax)
  zipf_b512_bf16_mixed_penalties   penalties over 1,024-token histories
  flat_b1024_f32_t1_p0.95          fp32 logits, a 93,700-token nucleus
  zipf_b256_bf16_top_logprobs20    arcs_top_logprobs, n=20
Launches rotate over enough copies of the logits (>= 512 MiB, twice the
256 MiB Infinity Cache) that every step reads its logits from HBM.

Timing: the launches of the timed region are enqueued behind a device-side
sleep, so the queue is full when the first timed launch starts (no start-up
bubble from the host's enqueue rate); HIP events on the launch stream
bracket exactly K steps.  The headline is also timed as one HIP graph of
the K launches.

After them, `nucleus_ab` times nucleus (top-p 0.95) sampling on rows whose
mass sits on 1 .. 12,928 tokens, arcs_sample against the baseline hybrid
selector of arcs_sample_hybrid_nucleus (enumeration up to 32 ids, then
threshold bisection), at B = 1.

Prints ONE JSON line: rows/s (= tokens/s), ms per step, the roofline object
of the sampling kernel (algorithmic bytes per launch over its average launch
duration, against MI355X's 8 TB/s HBM peak; counted HBM traffic from the
committed rocprofv3 summary when it was taken on the current kernel sources),
the CPU oracle timed on a bounded sample of the same workload on this host's
cores (before the GPU is touched), and the sub-records.

Other modes: --only times one workload alone (the profiled command);
--calibrate-copy runs a plain device copy of known size (for scaling
rocprofv3's FETCH_SIZE / WRITE_SIZE counters).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sampled rows/s and achieved HBM GB/s (% of peak) at B=256, V=129,280"
HBM_PEAK_GBPS = 8000.0
HEADLINE = "zipf_b256_bf16_t0.7_k50_p0.9_minp0.05"
SUB_CONFIGS = ("normal_b4_bf16", "zipf_b256_bf16_greedy", "zipf_b512_bf16_mixed_penalties",
               "flat_b1024_f32_t1_p0.95", "zipf_b256_bf16_top_logprobs20")
ROTATE_BYTES = 512 * 2**20
# the sources each kernel is built from (with the launcher): a committed
# counter summary holds only while these are unchanged
KERNEL_SOURCES = {
    "argmax": ["device_common.hpp", "launch.hpp", "api.hip", "argmax_kernel.hip"],
    "sample": ["device_common.hpp", "launch.hpp", "api.hip", "sample_common.hpp", "summary_path.hpp",
               "sample_kernel.hip"],
    "logprobs": ["device_common.hpp", "launch.hpp", "api.hip", "logprobs_kernel.hip"],
}


def kernel_kind(w) -> str:
    return "logprobs" if w.top_n else ("argmax" if w.greedy_only else "sample")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "decode_step_token_row_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "include", "arcs.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w) -> int:
    """Bytes the step must move at least once: logits, per-row params,
    history ids and offsets (if any), output ids."""
    es = 2 if w.dtype == "bf16" else 4
    if w.top_n:  # logits, per-row temperature, ids and logprobs
        return int(w.B * w.V * es + w.B * 4 + w.B * w.top_n * 8)
    b = w.B * w.V * es + w.B * 4
    if not w.greedy_only:
        b += w.B * 32
    if w.hist_ids is not None:
        b += w.hist_ids.nbytes + w.hist_offsets.nbytes
    return int(b)


def kernel_name(w) -> str:
    """The kernel one step launches for this workload (as the launcher picks it)."""
    fits = w.dtype == "bf16" and w.V % 8 == 0 and w.V <= 131072
    if w.top_n:
        return "top_logprobs_kernel"
    if w.greedy_only:
        return "argmax_fast_kernel" if fits else "argmax_kernel"
    if fits:
        # small batches without history arrays read their greedy and
        # unfiltered rows split over many workgroups first
        split = w.B <= 64 and 8192 <= w.V and w.hist_ids is None
        return "split_partial_kernel + sample_summary_kernel" if split else "sample_summary_kernel"
    if w.dtype == "f32" and w.V % 4 == 0 and w.V <= 131072 and w.hist_ids is None:
        return "sample_f32_kernel (+ sample_kernel for deferred rows)"
    return "sample_kernel"


def entry_point(w) -> str:
    return "arcs_top_logprobs" if w.top_n else ("arcs_argmax" if w.greedy_only else "arcs_sample")


def read_traffic(workload: str, kind: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    or None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash(kind):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------------------
# the CPU oracle baseline (before the GPU is touched)
# --------------------------------------------------------------------------
def _oracle_rows(name: str, rows, seconds: float):
    """Oracle rows of workload `name` (cycling over `rows`) for about
    `seconds`; returns (rows done, elapsed)."""
    from oracle import sampler as oracle
    from workloads import make_workload
    w = make_workload(name, rows=np.asarray(rows))
    done = 0
    t0 = time.perf_counter()
    while True:
        i = done % w.logits.shape[0]
        if w.top_n:
            oracle.top_logprobs_row(w.logits[i], w.dtype, float(w.params[i]["temperature"]), w.top_n)
        elif w.greedy_only:
            oracle.argmax(w.logits[i:i + 1], w.dtype)
        else:
            hist = None
            if w.hist_ids is not None:
                hist = w.hist_ids[int(w.hist_offsets[i]):int(w.hist_offsets[i + 1])]
            oracle.sample_row(w.logits[i], w.dtype, w.params[i], hist, w.seed, int(w.rows[i]), 0)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds and done >= 4:
            return done, el


def _oracle_worker(a):
    return _oracle_rows(*a)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name: str, B: int, seconds1: float, seconds_mc: float, cores: int):
    """The oracle as it stands: one thread on the first 64 rows, then `cores`
    processes on disjoint row blocks; both in rows/s."""
    rows = list(range(min(B, 64)))
    n1, el1 = _oracle_rows(name, rows, seconds1)
    single = n1 / el1
    mc = None
    if cores > 1:
        blocks = [list(range(B))[c::cores][:16] or rows for c in range(cores)]
        ctx = mp.get_context("spawn")
        t0 = time.perf_counter()
        with ctx.Pool(cores) as pool:
            res = pool.map(_oracle_worker, [(name, b, seconds_mc) for b in blocks])
        wall = time.perf_counter() - t0
        done = sum(r[0] for r in res)
        # rows over the longest worker's time (start-up of the processes excluded)
        mc = done / max(r[1] for r in res)
        mc_desc = (f"{cores} processes x about {seconds_mc:.0f} s on disjoint row blocks of {name} "
                   f"({done} rows, {wall:.1f} s wall with start-up)")
    return single, n1, el1, mc, (mc_desc if mc is not None else None)


# --------------------------------------------------------------------------
# GPU timing
# --------------------------------------------------------------------------
def calibrate_copy(nbytes: int, reps: int):
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(json.dumps({"mode": "calibrate_copy", "bytes_per_copy": nbytes, "copies": reps,
                      "read_bytes": nbytes, "write_bytes": nbytes,
                      "GBps": 2 * nbytes * reps / el / 1e9}), flush=True)


class Gate:
    """A device-side sleep on the launch stream: the timed launches are
    enqueued while it runs, so none of them waits for the host."""

    def __init__(self, torch):
        self.torch = torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)  # load the kernel
        a.record()
        torch.cuda._sleep(2_000_000)
        b.record()
        torch.cuda.synchronize()
        self.cycles_per_us = 2_000_000 / max(a.elapsed_time(b) * 1e3, 1.0)

    def sleep(self, us: float):
        self.torch.cuda._sleep(int(us * self.cycles_per_us))


class Runner:
    """One workload's buffers and its step function."""

    def __init__(self, arcs, torch, w):
        self.w = w
        dev = torch.device("cuda:0")
        if w.dtype == "bf16":
            base = torch.from_numpy(w.logits.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            base = torch.from_numpy(w.logits).to(dev)
        self.nbuf = max(1, min(16, math.ceil(ROTATE_BYTES / base.numel() / base.element_size())))
        self.bufs = [base] + [base.clone() for _ in range(self.nbuf - 1)]
        self.buf_mb = base.numel() * base.element_size() / 1e6
        self.params = arcs.params_to_device(w.params, dev)
        self.hist_ids = self.hist_offs = None
        if w.hist_ids is not None:
            self.hist_ids = torch.from_numpy(w.hist_ids).to(dev)
            self.hist_offs = torch.from_numpy(w.hist_offsets).to(dev)
        self.out = torch.empty(w.B, dtype=torch.int32, device=dev)
        ws = (arcs.workspace_bytes(w.B, w.V, arcs.DTYPE_BF16 if w.dtype == "bf16" else arcs.DTYPE_F32)
              if not (w.top_n or w.greedy_only) else 0)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None
        if w.top_n:
            self.temps = torch.from_numpy(np.ascontiguousarray(w.params["temperature"], dtype=np.float32)).to(dev)
            self.lp_ids = torch.empty((w.B, w.top_n), dtype=torch.int32, device=dev)
            self.lp_vals = torch.empty((w.B, w.top_n), dtype=torch.float32, device=dev)
        self.arcs = arcs

    def step(self, i):
        w, arcs = self.w, self.arcs
        x = self.bufs[i % self.nbuf]
        if w.top_n:
            arcs.top_logprobs(x, w.top_n, temperature=self.temps, out_ids=self.lp_ids, out_logprobs=self.lp_vals)
        elif w.greedy_only:
            arcs.argmax(x, out=self.out)
        else:
            arcs.sample(x, self.params, self.hist_ids, self.hist_offs, seed=w.seed, step=i, out=self.out,
                        workspace=self.ws)


def time_steps(torch, gate, run, first: int, steps: int):
    """Exactly `steps` launches between two events, enqueued behind the gate.
    Returns (ms per step, host enqueue us per step, whether the whole region
    was enqueued before the gate ended)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gate.sleep(2000.0 + 40.0 * steps)
    e0.record()
    t0 = time.perf_counter()
    for i in range(steps):
        run.step(first + i)
    e1.record()
    issue = time.perf_counter() - t0
    full = not e0.query()  # the gate was still running when the last launch was enqueued
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, issue / steps * 1e6, full


def time_graph(torch, gate, run, first: int, steps: int):
    """The same `steps` launches captured as one HIP graph, replayed once
    between two events; None if the capture fails."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                run.step(first + i)
    except Exception as exc:  # pragma: no cover - reported, not fatal
        log(f"[bench] graph capture failed: {exc}")
        return None
    torch.cuda.synchronize()
    g.replay()  # first replay uploads the graph
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gate.sleep(1000.0)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def measure(arcs, torch, gate, w, name, steps, warmup, event_launches, graph=False):
    run = Runner(arcs, torch, w)
    for i in range(warmup):
        run.step(i)
    torch.cuda.synchronize()
    ms, enq, full = time_steps(torch, gate, run, warmup, steps)
    n_ev = max(1, event_launches)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for i, (a, b) in enumerate(evs):
        a.record()
        run.step(warmup + steps + i)
        b.record()
    torch.cuda.synchronize()
    iso = sorted(a.elapsed_time(b) for a, b in evs)
    graph_ms = time_graph(torch, gate, run, warmup, steps) if graph else None
    alg = algorithmic_bytes(w)
    achieved = alg / (ms * 1e-3) / 1e9
    traffic = read_traffic(name, kernel_kind(w))
    rec = {
        "workload": name, "B": w.B, "V": w.V, "logits_dtype": w.dtype, "entry_point": entry_point(w),
        "kernel": kernel_name(w), "steps": steps, "us_per_step": ms * 1e3, "rows_per_s": w.B / (ms * 1e-3),
        "isolated_launch_us": float(np.mean(iso)) * 1e3, "host_enqueue_us_per_step": enq,
        "queue_full_before_timing": full, "logit_buffers_rotated": run.nbuf,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg},
    }
    if graph_ms is not None:
        rec["graph_us_per_step"] = graph_ms * 1e3
        rec["graph_rows_per_s"] = w.B / (graph_ms * 1e-3)
    log(f"[bench] {name}: {ms * 1e3:.2f} us/step ({achieved:.0f} GB/s, {achieved / HBM_PEAK_GBPS:.1%}), "
        f"isolated launch {rec['isolated_launch_us']:.2f} us, enqueue {enq:.2f} us/step, queue full {full}"
        + (f", graph {graph_ms * 1e3:.2f} us/step" if graph_ms is not None else ""))
    del run
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def nucleus_ab(arcs, torch, gate, widths=(1, 8, 64, 512, 4096, 12928), B=1, V=129_280, launches=20,
               budget=32):
    """Nucleus sampling on rows whose mass sits on `width` tokens (the pages'
    support-width sweep for their device selector): arcs_sample with top_p
    0.95 against the baseline hybrid selector (enumeration up to `budget` ids,
    then 32-step bisection), µs per launch of each (HIP events, gated)."""
    from workloads import f32_to_bf16_bits, make_params
    rng = np.random.default_rng(7)
    dev = torch.device("cuda:0")
    out = []
    for wdt in widths:
        z = np.full((B, V), -60.0, dtype=np.float32)
        for b in range(B):
            z[b, rng.choice(V, size=wdt, replace=False)] = rng.normal(0.0, 0.5, wdt)
        logits = torch.from_numpy(f32_to_bf16_bits(z).view(np.int16)).view(torch.bfloat16).to(dev)
        params = arcs.params_to_device(make_params(B, temperature=1.0, top_p=0.95), dev)
        T = torch.full((B,), 1.0, dtype=torch.float32, device=dev)
        P = torch.full((B,), 0.95, dtype=torch.float32, device=dev)
        ids = torch.empty(B, dtype=torch.int32, device=dev)
        kept = torch.empty(B, dtype=torch.int32, device=dev)
        ws = arcs.workspace_bytes(B, V, arcs.DTYPE_BF16)
        wsb = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        runs = {
            "arcs_sample_us": lambda i: arcs.sample(logits, params, seed=1, step=i, out=ids, workspace=wsb),
            "hybrid_us": lambda i: arcs.sample_hybrid_nucleus(logits, T, P, budget, seed=1, step=i, out=ids,
                                                              out_kept=kept),
        }
        rec = {"support_width": wdt, "B": B, "V": V, "top_p": 0.95, "budget": budget}
        for name, fn in runs.items():
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gate.sleep(500.0 + 40.0 * launches)
            e0.record()
            for i in range(launches):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            rec[name] = e0.elapsed_time(e1) / launches * 1e3
        rec["hybrid_kept"] = int(kept[0].item())
        rec["hybrid_path"] = "enumeration" if rec["hybrid_kept"] <= budget else "bisection"
        log(f"[bench] nucleus width {wdt}: arcs_sample {rec['arcs_sample_us']:.1f} us, "
            f"hybrid {rec['hybrid_us']:.1f} us ({rec['hybrid_path']}, kept {rec['hybrid_kept']})")
        out.append(rec)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true", help="time --workload alone (no sub-records)")
    ap.add_argument("--sub-steps", type=int, default=100)
    ap.add_argument("--event-launches", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--cpu-cores", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(rows would shard across GPUs with no exchange; see DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    from workloads import WORKLOAD_NAMES, make_workload
    if args.workload not in WORKLOAD_NAMES:
        print(f"unknown workload {args.workload}; one of {', '.join(WORKLOAD_NAMES)}", file=sys.stderr)
        sys.exit(2)

    # the CPU baseline first, before anything initialises the GPU
    cpu = None
    if not args.no_cpu_baseline and not args.calibrate_copy:
        cores = max(1, min(args.cpu_cores, os.cpu_count() or 1))
        log(f"[bench] cpu baseline: oracle, 1 thread for ~{args.cpu_seconds:.0f} s, then {cores} processes")
        B0 = make_workload(args.workload, rows=[0]).B
        single, n1, el1, mc, mc_desc = cpu_baseline(args.workload, B0, args.cpu_seconds, args.cpu_seconds / 2,
                                                    cores)
        cpu = {"value": mc if mc is not None else single, "unit": "rows/s",
               "cores": cores if mc is not None else 1, "kind": "oracle",
               "sample": (mc_desc + "; " if mc_desc else "") +
                         f"single thread: {n1} rows (the first 64 rows, cycled) in {el1:.1f} s",
               "single_thread_value": single, "cpu_model": cpu_model(),
               "note": "plain numpy fp64 oracle (a full-vocabulary sort per row), as it stands"}

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import decode_step_token_row_amd as arcs
    arcs.library()  # fails loudly when the HIP library is missing

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy * 2**20, max(args.steps, 1))
        return

    gate = Gate(torch)
    log(f"[bench] generating workload {args.workload}")
    w = make_workload(args.workload)
    head = measure(arcs, torch, gate, w, args.workload, args.steps, args.warmup, args.event_launches,
                   graph=not args.only)
    subs = []
    if not args.only:
        for name in SUB_CONFIGS:
            if name == args.workload:
                continue
            log(f"[bench] generating workload {name}")
            ws = make_workload(name)
            subs.append(measure(arcs, torch, gate, ws, name, min(args.steps, args.sub_steps),
                                min(args.warmup, 10), min(args.event_launches, 20)))
    ab = nucleus_ab(arcs, torch, gate) if not args.only else None

    ms_per_step = head["us_per_step"] * 1e-3
    roof = dict(head["roofline"])
    roof.update({"avg_launch_us": head["us_per_step"], "isolated_launch_us": head["isolated_launch_us"],
                 "kernel": head["kernel"]})
    res = {
        "metric": METRIC,
        "value": head["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # argmax compares raw 16-bit patterns as integers; sampling weighs in
        # fp32 (fp64 for rows without filters)
        "dtype": "i16" if (w.greedy_only and w.dtype == "bf16") else "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "B": w.B,
            "V": w.V,
            "logits_dtype": w.dtype,
            "entry_point": head["entry_point"],
            "logit_buffers_rotated": head["logit_buffers_rotated"],
            "parallelism": "single GPU, one workgroup per row",
        },
        "tokens_per_s": head["rows_per_s"],
        "step_GBps": roof["achieved"],
        "queue_full_before_timing": head["queue_full_before_timing"],
        "host_enqueue_us_per_step": head["host_enqueue_us_per_step"],
        "graph_us_per_step": head.get("graph_us_per_step"),
        "roofline": roof,
        "cpu_baseline": cpu,
        "sub_records": subs,
        "nucleus_ab": ab,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
