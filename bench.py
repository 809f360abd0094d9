"""Benchmark of the batched on-device sampler on one MI355X.

One step = one call of the hot path over one batch of synthetic logits that
are already resident in HBM: arcs_argmax for greedy-only workloads, else
arcs_sample (penalties, max/normaliser, top-k/top-p/min-p cutoff, SplitMix64
draw, output).  The default workload is the B=256, V=129,280 bf16 batch of
Zipf-shaped logits with greedy argmax on every row (66.2 MB read per step);
--workload picks another (e.g. the same logits with T=0.7, top_k=50,
top_p=0.9, min_p=0.05 on every row).  Launches rotate over enough copies of
the logits (>= 512 MiB, twice the 256 MiB Infinity Cache) that every step
reads its logits from HBM.

Prints ONE JSON line (rank 0): rows/s (= tokens/s), ms per step, the
roofline object of the sampling kernel (algorithmic bytes per launch over
its average launch duration measured with HIP events on the launch stream,
against MI355X's 8 TB/s HBM peak) and the CPU oracle timed on a bounded
sample of the same workload on this host.

Other modes: --calibrate-copy runs a plain device copy of known size (for
scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sampled rows/s and achieved HBM GB/s (% of peak) at B=256, V=129,280"
HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "zipf_b256_bf16_greedy"
ROTATE_BYTES = 512 * 2**20
# the sources each kernel is built from (with the launcher): a committed
# counter summary holds only while these are unchanged
KERNEL_SOURCES = {
    "argmax": ["device_common.hpp", "launch.hpp", "api.hip", "argmax_kernel.hip"],
    "sample": ["device_common.hpp", "launch.hpp", "api.hip", "sample_common.hpp", "sample_kernel.hip"],
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
        return "sample_summary_kernel"
    if w.dtype == "f32" and w.V % 4 == 0 and w.V <= 131072 and w.hist_ids is None:
        return "sample_f32_kernel"
    return "sample_kernel"


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


def cpu_baseline(w, seconds: float):
    from oracle import sampler as oracle
    rows = 0
    t0 = time.perf_counter()
    while True:
        i = rows % w.logits.shape[0]
        if w.top_n:
            oracle.top_logprobs_row(w.logits[i], w.dtype, float(w.params[i]["temperature"]), w.top_n)
        elif w.greedy_only:
            oracle.argmax(w.logits[i:i + 1], w.dtype)
        else:
            hist = None
            if w.hist_ids is not None:
                hist = w.hist_ids[int(w.hist_offsets[i]):int(w.hist_offsets[i + 1])]
            oracle.sample_row(w.logits[i], w.dtype, w.params[i], hist, w.seed, int(w.rows[i]), 0)
        rows += 1
        el = time.perf_counter() - t0
        if el >= seconds and rows >= 4:
            break
    return rows / el, rows, el


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--event-launches", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(rows would shard across GPUs with no exchange; see DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import decode_step_token_row_amd as arcs
    from workloads import make_workload
    arcs.library()  # fails loudly when the HIP library is missing

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy * 2**20, max(args.steps, 1))
        return

    log(f"[bench] generating workload {args.workload}")
    w = make_workload(args.workload)
    dev = torch.device("cuda:0")
    if w.dtype == "bf16":
        base = torch.from_numpy(w.logits.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        base = torch.from_numpy(w.logits).to(dev)
    nbuf = max(1, min(16, math.ceil(ROTATE_BYTES / base.numel() / base.element_size())))
    bufs = [base] + [base.clone() for _ in range(nbuf - 1)]
    params = arcs.params_to_device(w.params, dev)
    hist_ids = hist_offs = None
    if w.hist_ids is not None:
        hist_ids = torch.from_numpy(w.hist_ids).to(dev)
        hist_offs = torch.from_numpy(w.hist_offsets).to(dev)
    out = torch.empty(w.B, dtype=torch.int32, device=dev)
    if w.top_n:
        temps = torch.from_numpy(np.ascontiguousarray(w.params["temperature"], dtype=np.float32)).to(dev)
        lp_ids = torch.empty((w.B, w.top_n), dtype=torch.int32, device=dev)
        lp_vals = torch.empty((w.B, w.top_n), dtype=torch.float32, device=dev)

    def step(i):
        x = bufs[i % nbuf]
        if w.top_n:
            arcs.top_logprobs(x, w.top_n, temperature=temps, out_ids=lp_ids, out_logprobs=lp_vals)
        elif w.greedy_only:
            arcs.argmax(x, out=out)
        else:
            arcs.sample(x, params, hist_ids, hist_offs, seed=w.seed, step=i, out=out)

    log(f"[bench] warmup {args.warmup}, buffers {nbuf} x {base.numel() * base.element_size() / 1e6:.1f} MB")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    issue = time.perf_counter() - t0  # host time to enqueue the launches
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / args.steps

    # Isolated launches: event pairs around single launches on the launch
    # stream (torch's current stream), reported next to the timed-region average.
    n_ev = max(1, args.event_launches)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for i, (a, b) in enumerate(evs):
        a.record()
        step(args.warmup + args.steps + i)
        b.record()
    torch.cuda.synchronize()
    launch_ms = sorted(a.elapsed_time(b) for a, b in evs)
    avg_launch_ms = float(np.mean(launch_ms))

    alg = algorithmic_bytes(w)
    # one launch per step: the average launch duration over the timed region
    achieved = alg / (ms_per_step * 1e-3) / 1e9
    traffic = read_traffic(args.workload, kernel_kind(w))
    rows_per_s = w.B / (ms_per_step * 1e-3)
    log(f"[bench] {ms_per_step * 1e3:.2f} us/step, launch avg {avg_launch_ms * 1e3:.2f} us "
        f"(median {launch_ms[len(launch_ms) // 2] * 1e3:.2f}), {achieved:.0f} GB/s, wall {wall:.4f}s, "
        f"host enqueue {issue / args.steps * 1e6:.2f} us/step")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle for ~{args.cpu_seconds:.0f}s")
        sub = make_workload(args.workload, rows=np.arange(min(w.B, 64)))
        v, n, el = cpu_baseline(sub, args.cpu_seconds)
        cpu = {"value": v, "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} rows of {args.workload} (the first {len(sub.rows)} rows, cycled), "
                         f"{el:.1f} s, single-threaded numpy fp64 oracle"}

    res = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # argmax compares raw 16-bit patterns as integers; sampling weighs in fp32
        "dtype": "i16" if (w.greedy_only and w.dtype == "bf16") else "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "B": w.B,
            "V": w.V,
            "logits_dtype": w.dtype,
            "entry_point": ("arcs_top_logprobs" if w.top_n else
                            "arcs_argmax" if w.greedy_only else "arcs_sample"),
            "logit_buffers_rotated": nbuf,
            "parallelism": "single GPU, one workgroup per row",
        },
        "tokens_per_s": rows_per_s,
        "step_GBps": alg / (ms_per_step * 1e-3) / 1e9,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg,
            "avg_launch_us": ms_per_step * 1e3,
            "isolated_launch_us": avg_launch_ms * 1e3,
            "kernel": kernel_name(w),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
