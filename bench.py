"""Benchmark of the verification hot path on one MI355X.

One step = one verification call (jsv_verify_stats then jsv_verify_sample) over one
synthetic block at the Qwen3-8B LM-head shape: d = 4096, V = 151936, K = 16 drafts,
batch 1, bf16 weights, T = 1 with the softmax proposal (draft logits read).  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

  python bench.py [--steps 50] [--warmup 5] [--config qwen8b_k16] [--no-cpu-baseline]
  python bench.py --copy-probe     # plain device copy of known size (counter calibration)
  python bench.py --next-rows      # latencies of anchor replacement, cache lookup,
                                   # calibrated lengths and the geometric fan-out
  python bench.py --pmc-summary DIR
      turn four rocprofv3 counter runs under DIR (bench_FETCH_SIZE, bench_WRITE_SIZE,
      copy_FETCH_SIZE, copy_WRITE_SIZE, each holding run_counter_collection.csv) into
      profiles/stats_kernel_<config>_traffic.{json,md}; the bench line reports that
      traffic only while the kernel sources still hash to what was measured.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))
KERNEL_SOURCES = ("draft_block_verification_rmsnorm_amd/csrc/jsv_kernels.hip",
                  "draft_block_verification_rmsnorm_amd/csrc/jsv_internal.h",
                  "draft_block_verification_rmsnorm_amd/csrc/jsv_api.hip")
COPY_PROBE_BYTES = 1 << 30

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0


def algorithmic_bytes(cfg, T, mode_softmax):
    """Bytes the method must move per call: W once (and its row scales for an fp8 head),
    hidden states, gamma, and the draft logits when the softmax proposal needs q."""
    wsz = {"bf16": 2, "f32": 4, "fp8": 1}[cfg.dtype]
    xsz = 4 if cfg.dtype == "f32" else 2
    M = cfg.batch * (cfg.K + 1)
    b = cfg.vocab * cfg.hidden * wsz + M * cfg.hidden * xsz + cfg.hidden * xsz
    if cfg.dtype == "fp8":
        b += cfg.vocab * 4
    if mode_softmax and T > 0:
        b += cfg.batch * cfg.K * cfg.vocab * 4
    return b


def lmhead_flops(cfg):
    """Dense flops of the LM-head product of one call: 2 M V d."""
    return 2 * cfg.batch * (cfg.K + 1) * cfg.vocab * cfg.hidden


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        h.update((ROOT / rel).read_bytes())
    return h.hexdigest()


def traffic_path(config):
    return ROOT / "profiles" / f"stats_kernel_{config}_traffic.json"


def measured_traffic(config):
    """HBM bytes per launch of the LM-head kernel from the committed counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    p = traffic_path(config)
    if not p.exists():
        return None
    t = json.loads(p.read_text())
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t["traffic_bytes_per_launch"]


def _counter_means(csv_path, name_prefix):
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if r["Kernel_Name"].startswith(name_prefix)]
    if not vals:
        raise SystemExit(f"no dispatch of {name_prefix!r} in {csv_path}")
    return sum(vals) / len(vals), len(vals)


# The LM-head kernels of jsv_verify_stats: the fused kernel, or for more rows than one pass
# holds (bf16) the split-d kernels.
LMHEAD_KERNELS = ("void jsv::stats_kernel", "jsv::xhat_kernel", "void jsv::wide_kernel",
                  "void jsv::wide_stats_kernel")


def wide_path(cfg):
    """True when verification of this workload takes the split-d LM head (bf16, 34..144
    rows, d a multiple of 1024 up to 5120)."""
    M = cfg.batch * (cfg.K + 1)
    return cfg.dtype == "bf16" and 33 < M <= 144 and cfg.hidden % 1024 == 0 and cfg.hidden <= 5120


def _lmhead_means(csv_path):
    """Sum over the LM-head kernels present of their mean counter value per dispatch."""
    total, n, names = 0.0, 0, []
    for k in LMHEAD_KERNELS:
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
                if r["Kernel_Name"].startswith(k)]
        if vals:
            total += sum(vals) / len(vals)
            n = max(n, len(vals))
            names.append(k.replace("void ", ""))
    if not names:
        raise SystemExit(f"no LM-head dispatch in {csv_path}")
    return total, n, names


def pmc_summary(pmc_dir, config):
    """Counter runs -> traffic summary.  FETCH_SIZE and WRITE_SIZE are KiB per dispatch;
    each is scaled by the factor that makes the 1 GiB copy read and write 1 GiB.  With the
    split-d LM head the three kernels of one call are added."""
    d = Path(pmc_dir)
    f_kib, nf, names = _lmhead_means(d / "bench_FETCH_SIZE" / "run_counter_collection.csv")
    w_kib, nw, _ = _lmhead_means(d / "bench_WRITE_SIZE" / "run_counter_collection.csv")
    kname = " + ".join(names)
    cf_kib, _ = _counter_means(d / "copy_FETCH_SIZE" / "run_counter_collection.csv", "__amd_rocclr_copyBuffer")
    cw_kib, _ = _counter_means(d / "copy_WRITE_SIZE" / "run_counter_collection.csv", "__amd_rocclr_copyBuffer")
    sf = COPY_PROBE_BYTES / (cf_kib * 1024.0)
    sw = COPY_PROBE_BYTES / (cw_kib * 1024.0)
    fetch = f_kib * 1024.0 * sf
    write = w_kib * 1024.0 * sw
    import synth
    cfg = synth.CONFIGS[config]
    abytes = algorithmic_bytes(cfg, 1.0, True)
    out = {"kernel": kname, "config": config, "kernel_source_sha256": kernel_source_hash(),
           "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": [nf, nw],
           "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib, "copy_bytes": COPY_PROBE_BYTES,
           "fetch_scale": sf, "write_scale": sw,
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "traffic_bytes_per_launch": fetch + write, "algorithmic_bytes": abytes}
    traffic_path(config).parent.mkdir(exist_ok=True)
    traffic_path(config).write_text(json.dumps(out, indent=1) + "\n")
    print(json.dumps(out, indent=1))


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
    ap.add_argument("--pmc-summary", metavar="DIR")
    ap.add_argument("--next-rows", action="store_true")
    args = ap.parse_args()
    if args.pmc_summary:
        return pmc_summary(args.pmc_summary, args.config)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(a verification call runs on one device)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        return copy_probe(torch)
    if args.next_rows:
        return next_rows(torch, args)

    import draft_block_verification_rmsnorm_amd as jsv
    import synth

    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    T = args.temperature
    mode = jsv.PROPOSAL_POINT if args.point else jsv.PROPOSAL_SOFTMAX
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    head_cpu = synth.head_for(cfg)
    blk = synth.make_block(head_cpu, cfg.batch, cfg.K, cfg.sigma, T, seed=0)
    ws_ = head_cpu.weight_scale
    head = jsv.LMHead(head_cpu.weight.to(dev), head_cpu.norm_weight.to(dev), cfg.eps,
                      weight_scale=None if ws_ is None else ws_.to(dev))
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
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(args.config) if (T > 0 and not args.point) else None,
                     "kernel": ("xhat_kernel + wide_kernel + wide_stats_kernel (split-d RMSNorm + LM head "
                                "+ softmax statistics)" if wide_path(cfg) else
                                "stats_kernel (fused RMSNorm + LM head + softmax statistics)"),
                     "algorithmic_bytes": abytes},
        "mfma": {"achieved": round(lmhead_flops(cfg) / (k1_ms * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(lmhead_flops(cfg) / (k1_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "flops": lmhead_flops(cfg)},
        "accepted_last_step": n_acc,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, head_cpu, blk, T, mode)
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, head_cpu, blk, T, mode):
    """The oracle as it stands, on the host cores, over a bounded sample of the same
    workload: whole verification calls on the same block, at least 3 and until ~12 s of
    CPU work have passed."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    oh = oracle.Head(head_cpu.weight, head_cpu.norm_weight, cfg.eps, cfg.dtype,
                     weight_scale=head_cpu.weight_scale)
    dl = blk.draft_logits if mode == oracle.PROPOSAL_SOFTMAX else None
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_start < 12.0 and len(times) < 50):
        t0 = time.perf_counter()
        oracle.verify_block(oh, blk.hidden, blk.draft_tokens.numpy(), dl, T, mode, 1234, len(times))
        times.append(time.perf_counter() - t0)
    sec = float(np.median(times))
    return {"value": round(cfg.K * cfg.batch / sec, 3), "unit": "verified draft positions/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} whole verification calls of the benchmark block (float64 NumPy), "
                      f"median {sec:.2f} s per call"}


def _event_median(torch, fn, n=50, warm=5):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    return times[len(times) // 2]


def next_rows(torch, args):
    """Latency of the next-row calls on the benchmark shape: anchor replacement on predicted
    states (one HBM stream over W, like verification), the cache hit test against a top-8
    list, the calibrated length score and the host fan-out (K = 16, cache of 16)."""
    import draft_block_verification_rmsnorm_amd as jsv
    import synth
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    head_cpu = synth.head_for(cfg)
    blk = synth.make_block(head_cpu, cfg.batch, cfg.K, cfg.sigma, 1.0, seed=0)
    ws_ = head_cpu.weight_scale
    head = jsv.LMHead(head_cpu.weight.to(dev), head_cpu.norm_weight.to(dev), cfg.eps,
                      weight_scale=None if ws_ is None else ws_.to(dev))
    hp = synth.predicted_hidden(blk.hidden, seed=0).to(dev)
    drafts = blk.draft_tokens.to(dev)
    G = blk.draft_logits.to(dev)
    ws = jsv.new_workspace(head, cfg.batch, cfg.K, 8)
    aout = jsv.AnchorOut(cfg.batch, dev)
    t_anchor = _event_median(torch, lambda: jsv.anchor_replace(head, hp, drafts, ws, out=aout), n=20)
    sc = jsv.score_outcomes(head, hp, drafts, G, 1.0, jsv.PROPOSAL_SOFTMAX, 8, ws)
    vo = jsv.verify_block(head, blk.hidden.to(dev), drafts, G, 1.0, jsv.PROPOSAL_SOFTMAX, 1, 0, ws)
    hit = torch.empty(cfg.batch, dtype=torch.int32, device=dev)
    t_lookup = _event_median(torch, lambda: jsv.cache_lookup(vo.n_accepted, vo.committed, sc.out_len,
                                                             sc.out_token, hit_index=hit))
    pt = torch.rand(cfg.batch, cfg.K, dtype=torch.float64, device=dev)
    lo = torch.empty(cfg.batch, cfg.K + 1, dtype=torch.float64, device=dev)
    lf = torch.empty(cfg.batch, dtype=torch.int32, device=dev)
    t_len = _event_median(torch, lambda: jsv.calibrated_lengths(pt, out=lo, flags=lf))
    t0 = time.perf_counter()
    for _ in range(1000):
        jsv.geometric_fanout(0.89, 1.0, cfg.K, 16)
    t_fan = (time.perf_counter() - t0) / 1000
    abytes = algorithmic_bytes(cfg, 0.0, False)
    print(json.dumps({"metric": "next-row call latency", "config": {"workload": cfg.name},
                      "anchor_replace_ms": round(t_anchor, 4),
                      "anchor_replace_hbm_frac": round(abytes / (t_anchor * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "cache_lookup_us": round(t_lookup * 1e3, 2),
                      "calibrated_lengths_us": round(t_len * 1e3, 2),
                      "geometric_fanout_host_us": round(t_fan * 1e6, 2)}), flush=True)


def copy_probe(torch):
    """A plain device-to-device copy of 1 GiB, five times: the bytes are known exactly, so
    its FETCH_SIZE / WRITE_SIZE counters calibrate the counters of the verification kernels."""
    n = COPY_PROBE_BYTES
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "reps": 5}), flush=True)


if __name__ == "__main__":
    main()
