#!/usr/bin/env python3
"""Throughput of the fused LM-head loss on one MI355X.

A step is one hl_forward_backward call (valid-row count, the fused kernel:
shared softmax, every loss and the gradient, then the batch reduction; GSPO
workloads call hl_forward_backward_segments) over one batch of synthetic
inputs already resident in HBM. Prints one JSON line on stdout; progress
goes to stderr.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1] [--no-grad]

--no-grad times metrics-only calls (no gradient buffer): the streaming
statistics kernel, one read of each valid row (GSPO: plus the segment step).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "tokens/s + achieved HBM GB/s (% peak), CE+z+GRPO+entropy, V=151936 bf16, 1 GPU"
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E, vendor figure
FUSED_KERNEL = "fused_kernel"
# with GSPO the timed bracket holds the forward, the segment step and the reloading backward
GSPO_KERNELS = "stream_stats_kernel (forward) + seam_kernel + fused_kernel (load mode)"
STREAM_KERNEL = "stream_stats_kernel"
GSPO_FWD_KERNELS = "stream_stats_kernel (forward) + seam_kernel"
LOSS_NAMES = {1: "CE", 2: "z", 4: "FKL", 8: "RKL", 64: "FDCE", 16: "GRPO", 128: "GSPO", 32: "entropy"}
HINTON_BIT = 1 << 17


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """The source without // and /* */ comments and without blank space, so
    that an edit of a comment does not invalidate stored counters. (String
    literals holding comment markers would be cut too; the kernel sources
    have none that change code.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash() -> str:
    """Hash of the kernel sources' code (tells whether stored counters still apply)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lm_head_vocab_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".cuh", ".h", ".cpp")):
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                h.update(name.encode())
                h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def plan_kwargs(w):
    wt = w.weights
    return dict(ce=wt.get("ce", 1.0), z=wt.get("z", 0.0), distill=wt.get("distill", 0.0),
                grpo=wt.get("grpo", 0.0), grad_scale=wt.get("grad_scale", 1.0),
                divisor=wt.get("divisor", 0.0), temperature=w.temperature, eps=w.eps,
                logit_scale=w.logit_scale, softcap=w.softcap)


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle, as it stands, on a bounded sample of rows
# ---------------------------------------------------------------------------
_SAMPLE = None   # (spec, flags, N, x, inputs): set before the worker processes fork


def _oracle_rows(bounds):
    """One task of the CPU baseline: the oracle's forward+backward on rows
    [r0, r1) of the sample (GSPO: those rows as one segment)."""
    import oracle

    spec, flags, N, x, d = _SAMPLE
    r0, r1 = bounds
    sub = {key: (v[r0:r1] if v is not None else None) for key, v in d.items()}
    if flags & oracle.GSPO:
        oracle.forward_backward(spec, x[r0:r1], seq_offsets=[0, r1 - r0], **sub)
    else:
        oracle.rows_forward_backward(spec, x[r0:r1], float(N), **sub)
    return r1 - r0


def cpu_baseline(w, budget_s: float, workers: int):
    import multiprocessing as mp

    import numpy as np

    import oracle

    global _SAMPLE
    spec = oracle.Spec(V=w.V, flags=w.flags, w_ce=w.weights.get("ce", 1.0), w_z=w.weights.get("z", 0.0),
                       w_distill=w.weights.get("distill", 0.0), w_grpo=w.weights.get("grpo", 0.0),
                       grad_scale=w.weights.get("grad_scale", 1.0), temperature=w.temperature,
                       eps=w.eps, logit_scale=w.logit_scale, softcap=w.softcap)
    rows_per_task = 2
    n_rows = 4 * workers * rows_per_task
    inp = workloads.generate(w, "cpu", seed=workloads.seed_for(w.name, 8), n_rows=n_rows)
    x = inp["logits"].double().numpy()
    y = inp["labels"].numpy() if inp["labels"] is not None else None
    d = dict(labels=y, mask=inp["mask"].numpy() if inp["mask"] is not None else None,
             teacher=inp["teacher"].double().numpy() if inp["teacher"] is not None else None,
             advantages=inp["advantages"].double().numpy() if inp["advantages"] is not None else None,
             grad_in=inp["grad_init"].double().numpy() if inp["grad_init"] is not None else None,
             old_logprobs=None)
    if w.flags & (oracle.GRPO | oracle.GSPO):
        d["old_logprobs"] = oracle.row_values(spec, x, y)["logp"] + inp["old_noise"].double().numpy()
    _SAMPLE = (spec, w.flags, w.N, x, d)
    tasks = [(r0, r0 + rows_per_task) for r0 in range(0, n_rows, rows_per_task)]
    log(f"cpu baseline: oracle on a {n_rows}-row sample x V={w.V}, {workers} worker processes, ~{budget_s:.0f} s")
    done = 0
    # fork: the workers inherit the sample; nothing has touched the GPU yet
    with mp.get_context("fork").Pool(processes=workers) as pool:
        t0 = time.perf_counter()
        while True:
            done += sum(pool.map(_oracle_rows, tasks, chunksize=1))
            dt = time.perf_counter() - t0
            if dt >= budget_s:
                break
    _SAMPLE = None
    return {"value": done / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "workers": workers, "host_cores": os.cpu_count(),
            "cpus_available": len(os.sched_getaffinity(0)),
            "sample": f"{done} row evaluations of a {n_rows}-row host-drawn sample of {w.name} (V={w.V}, same "
                      f"recipe), full forward+backward in numpy fp64, {workers} worker processes "
                      f"(host reports {os.cpu_count()} cores; the pool is capped at the 16-CPU share of one "
                      f"GPU), {dt:.1f} s"}


# ---------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------
def traffic_file(w, with_grad=True):
    """The committed counter summary of a workload's timed kernel(s)."""
    if with_grad:
        tag = "fused_seam" if w.flags & workloads.GSPO else FUSED_KERNEL
    else:
        tag = "stream_seam" if w.flags & workloads.GSPO else "stream_stats"
    return f"profiles/{tag}_{w.name}_pmc.json"


def stored_traffic(w, src_hash, with_grad=True):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, traffic_file(w, with_grad))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("src_hash") != src_hash:
        return None
    return d.get("traffic_bytes_per_launch")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=workloads.HEADLINE, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-separate", action="store_true")
    ap.add_argument("--chunks", type=int, default=0, help="force the split-vocab chunk count")
    ap.add_argument("--block", type=int, default=0, help="force the threads per workgroup (with --chunks)")
    ap.add_argument("--no-grad", action="store_true", help="metrics-only calls (no gradient buffer)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    w = workloads.WORKLOADS[args.workload]

    # The host baseline runs before anything touches the GPU.
    cpu = None
    if not args.no_cpu_baseline:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        cpu = cpu_baseline(w, args.cpu_seconds, workers)
        log(f"cpu baseline {cpu['value']:.1f} tokens/s")

    import torch

    import lm_head_vocab_amd as hl

    dev = torch.device("cuda:0")
    log(f"generating {w.name}: N={w.N} V={w.V} {w.dtype}")
    inp = workloads.generate(w, dev)
    if w.flags & (workloads.GRPO | workloads.GSPO):
        # old = label log-prob of the stored logits (fp32, torch) + noise: input synthesis
        N = w.N
        old = torch.empty(N, dtype=torch.float32, device=dev)
        y = inp["labels"].clamp(min=0)
        for r0 in range(0, N, 512):
            r1 = min(N, r0 + 512)
            xs = inp["logits"][r0:r1].float()
            s = w.softcap * torch.tanh(xs * (w.logit_scale / w.softcap)) if w.softcap > 0 else xs * w.logit_scale
            old[r0:r1] = torch.log_softmax(s, 1).gather(1, y[r0:r1, None])[:, 0]
        inp["old_logprobs"] = old + inp["old_noise"]
    labels = inp["labels"]
    valid = (labels >= 0) & (labels < w.V)
    if inp["mask"] is not None:
        valid &= inp["mask"] != 0
    n_valid = int(valid.sum().item())
    acc = bool(w.flags & workloads.ACCUMULATE)
    grad = None if args.no_grad else (inp["grad_init"].clone() if acc else torch.empty_like(inp["logits"]))
    plan = hl.Plan(w.V, w.torch_dtype, w.flags, **plan_kwargs(w))
    if args.chunks or args.block:
        plan.set_variant(args.chunks, args.block)
    geo = plan.describe()
    log(f"plan {geo}")

    def step(p=plan, g=grad):
        return p(inp["logits"], labels=labels, mask=inp["mask"], teacher=inp["teacher"],
                 old_logprobs=inp.get("old_logprobs"), advantages=inp["advantages"], grad=g,
                 seq_offsets=inp["seq_offsets"])

    # Context measurements first (they also bring the device to its working
    # clocks before the fused warm-up and timed steps).
    stream = torch.cuda.current_stream(dev)
    # plain device-to-device copy bandwidth, for context
    nb = 4 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * nb * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    separate = None
    if not args.no_separate and not args.no_grad:
        plans = []
        first = True
        for bit, lname in LOSS_NAMES.items():
            if not (w.flags & bit):
                continue
            kw = plan_kwargs(w)
            keep = {1: "ce", 2: "z", 4: "distill", 8: "distill", 64: "distill", 16: "grpo", 128: "grpo"}.get(bit)
            for key in ("ce", "z", "distill", "grpo"):
                if key != keep:
                    kw[key] = 0.0
            flags = bit
            if bit in (4, 8, 64):
                flags |= w.flags & HINTON_BIT     # the distillation pass keeps its temperature mode
            if bit != 32 and not first:
                flags |= hl.ACCUMULATE
            if bit == 32:
                plans.append((hl.Plan(w.V, w.torch_dtype, flags, **kw), None))
            else:
                if first and acc:
                    flags |= hl.ACCUMULATE
                plans.append((hl.Plan(w.V, w.torch_dtype, flags, **kw), grad))
                first = False

        def sep_step():
            for p, g in plans:
                step(p, g)
        for _ in range(max(1, args.warmup)):
            sep_step()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            sep_step()
        e1.record(stream)
        torch.cuda.synchronize()
        sep_ms = e0.elapsed_time(e1) / args.steps
        separate = {"ms_per_step": round(sep_ms, 5), "passes": [LOSS_NAMES[b] for b in LOSS_NAMES if w.flags & b]}
        log(f"separate passes: {sep_ms:.4f} ms/step")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    K = args.steps
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in kev:          # materialise the events before handing them to the library
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        plan.set_timing_events(*kev[i])
        step()
    t_stop.record(stream)
    torch.cuda.synchronize()
    plan.set_timing_events(None, None)
    ms_total = t_start.elapsed_time(t_stop)
    ms_step = ms_total / K
    kernel_ms = sorted(a.elapsed_time(b) for a, b in kev)
    kernel_avg = sum(kernel_ms) / K
    log(f"timed {K} steps: {ms_step:.4f} ms/step, fused kernel {kernel_avg:.4f} ms avg")

    algo_bytes = workloads.algorithmic_bytes(w, n_valid, with_grad=not args.no_grad)
    achieved = algo_bytes / (kernel_avg * 1e-3) / 1e9
    src_hash = source_hash()
    traffic = stored_traffic(w, src_hash, with_grad=not args.no_grad)
    tfile = traffic_file(w, with_grad=not args.no_grad)
    traffic_source = (f"{tfile}: rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, copy-calibrated, taken on "
                      f"these kernel sources (hash {src_hash}); not measured in this run"
                      if traffic is not None else
                      f"null: no counter summary for kernel source hash {src_hash} ({tfile})")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic, "traffic_source": traffic_source,
                "kernel": ((GSPO_KERNELS if w.flags & workloads.GSPO else FUSED_KERNEL) if not args.no_grad else
                           (GSPO_FWD_KERNELS if w.flags & workloads.GSPO else STREAM_KERNEL)),
                "kernel_ms_avg": round(kernel_avg, 5),
                "algorithmic_bytes_per_launch": algo_bytes}

    # The memory system's own rate for this traffic shape: a data-movement-only
    # kernel with the fused kernel's geometry (same block, loads per thread,
    # tensors read and written), over full tensors of this workload's size.
    ceiling = None
    if not args.no_grad and geo["block"] in (512, 1024):   # (256-thread variants: rows too short to stream)
        vpt = min((4, 6, 8, 9, 10) + ((13,) if geo["block"] == 512 else ()),
                  key=lambda v: (abs(v - geo["vec_per_thread"]), v))
        out = torch.empty_like(inp["logits"])
        reads = [inp["logits"]] + ([inp["teacher"]] if inp["teacher"] is not None else [])
        cms = hl.stream_ceiling(reads[0], reads[1] if len(reads) > 1 else None, out, geo["block"], vpt, reps=5)
        del out
        moved = (len(reads) + 1) * inp["logits"].numel() * inp["logits"].element_size()
        cgbps = moved / (cms * 1e-3) / 1e9
        ceiling = {"kernel": "hl_stream_ceiling", "reads": len(reads), "writes": 1, "block": geo["block"],
                   "vec_per_thread": vpt, "ms": round(cms, 5), "GBps": round(cgbps, 1),
                   "frac_of_peak": round(cgbps / PEAK_HBM_GBPS, 4), "fused_over_ceiling": round(achieved / cgbps, 4)}
        log(f"stream ceiling {cgbps:.0f} GB/s ({cgbps / PEAK_HBM_GBPS:.1%} of peak); fused/ceiling "
            f"{achieved / cgbps:.3f}")

    if separate is not None:
        separate["fused_speedup"] = round(separate["ms_per_step"] / ms_step, 3)
    tokens_s = w.N / (ms_step * 1e-3)
    line = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "N": w.N, "V": w.V, "dtype": w.dtype,
                   "losses": "+".join(LOSS_NAMES[b] for b in LOSS_NAMES if w.flags & b)
                             + (" (Hinton temperature)" if w.flags & HINTON_BIT else ""),
                   "accumulate": acc, "gradient": not args.no_grad, "n_valid": n_valid, "variant": geo},
        "hbm_GBps_step": round(algo_bytes / (ms_step * 1e-3) / 1e9, 1),
        "frac_peak_step": round(algo_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "copy_GBps": round(copy_gbps, 1),
        "roofline": roofline,
        "ceiling": ceiling,
        "cpu_baseline": cpu,
        "separate_pass": separate,
        "src_hash": src_hash,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
