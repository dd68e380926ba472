"""Benchmark of the verification hot path on one MI355X.

One step = one verification call (jsv_verify_stats then jsv_verify_sample) over one
synthetic block at the Qwen3-8B LM-head shape: d = 4096, V = 151936, K = 16 drafts,
batch 1, bf16 weights, T = 1 with the softmax proposal (draft logits read).  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

  python bench.py [--steps 50] [--warmup 5] [--config qwen8b_k16] [--no-cpu-baseline]
  python bench.py --copy-probe     # plain device copy of known size (counter calibration)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0


def algorithmic_bytes(cfg, T, mode_softmax):
    """Bytes the method must move per call: W once, hidden states, gamma, and the draft
    logits when the softmax proposal needs q."""
    esz = 2 if cfg.dtype == "bf16" else 4
    M = cfg.batch * (cfg.K + 1)
    b = cfg.vocab * cfg.hidden * esz + M * cfg.hidden * esz + cfg.hidden * esz
    if mode_softmax and T > 0:
        b += cfg.batch * cfg.K * cfg.vocab * 4
    return b


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen8b_k16")
    ap.add_argument("--temperature", type=float, default=1.0)
    ap.add_argument("--point", action="store_true", help="point-mass proposal instead of softmax")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the verification call runs on one device; see DESIGN.md for how it would shard)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        return copy_probe(torch)

    import draft_block_verification_rmsnorm_amd as jsv
    import synth

    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    T = args.temperature
    mode = jsv.PROPOSAL_POINT if args.point else jsv.PROPOSAL_SOFTMAX
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    head_cpu = synth.head_for(cfg)
    blk = synth.make_block(head_cpu, cfg.batch, cfg.K, cfg.sigma, T, seed=0)
    head = jsv.LMHead(head_cpu.weight.to(dev), head_cpu.norm_weight.to(dev), cfg.eps)
    hidden = blk.hidden.to(dev)
    drafts = blk.draft_tokens.to(dev)
    G = blk.draft_logits.to(dev) if mode == jsv.PROPOSAL_SOFTMAX else None
    ws = jsv.new_workspace(head, cfg.batch, cfg.K)
    out = jsv.VerifyOut(cfg.batch, cfg.K, dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        jsv.verify_stats(head, hidden, drafts, G, T, mode, 1234, i, ws, out=out, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        jsv.verify_sample(head, hidden, drafts, G, T, mode, 1234, i, ws, out=out, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k1 = sorted(e[0].elapsed_time(e[1]) for e in evs)
    k2 = sorted(e[1].elapsed_time(e[2]) for e in evs)
    call = sorted(e[0].elapsed_time(e[2]) for e in evs)
    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    ms_step = wall * 1e3 / args.steps
    positions = cfg.K * cfg.batch
    value = positions / (ms_step * 1e-3)
    abytes = algorithmic_bytes(cfg, T, mode == jsv.PROPOSAL_SOFTMAX)
    k1_ms = mean(k1)
    achieved = abytes / (k1_ms * 1e-3) / 1e9
    n_acc = int(out.n_accepted.sum())

    line = {
        "metric": "verified draft positions/s at Qwen3-8B LM-head shape; % of HBM roofline",
        "value": round(value, 1),
        "unit": "verified draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name + f" verify T={T} " + ("point-mass" if args.point else "softmax q"),
                   "hidden": cfg.hidden, "vocab": cfg.vocab, "K": cfg.K, "batch": cfg.batch,
                   "temperature": T},
        "latency_ms": {"call_median": round(call[len(call) // 2], 4),
                       "call_p90": round(call[int(0.9 * (len(call) - 1))], 4),
                       "stats_kernel_mean": round(k1_ms, 4), "accept_and_bonus_mean": round(mean(k2), 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "stats_kernel (fused RMSNorm + LM head + softmax statistics)",
                     "algorithmic_bytes": abytes},
        "accepted_last_step": n_acc,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, head_cpu, blk, T, mode)
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, head_cpu, blk, T, mode):
    """The oracle as it stands, on the host cores, over a bounded sample of the same
    workload: whole verification calls on the same block, until ~10 s have passed."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    oh = oracle.Head(head_cpu.weight, head_cpu.norm_weight, cfg.eps, cfg.dtype)
    dl = blk.draft_logits if mode == oracle.PROPOSAL_SOFTMAX else None
    times = []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < 10.0 and len(times) < 5):
        t0 = time.perf_counter()
        oracle.verify_block(oh, blk.hidden, blk.draft_tokens.numpy(), dl, T, mode, 1234, len(times))
        times.append(time.perf_counter() - t0)
    sec = float(np.median(times))
    return {"value": round(cfg.K * cfg.batch / sec, 3), "unit": "verified draft positions/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} whole verification calls of the benchmark block (float64 NumPy), "
                      f"median {sec:.2f} s per call"}


def copy_probe(torch):
    """A plain device-to-device copy of 1 GiB, five times: the bytes are known exactly, so
    its FETCH_SIZE / WRITE_SIZE counters calibrate the counters of the verification kernels."""
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "reps": 5}), flush=True)


if __name__ == "__main__":
    main()
