"""Benchmark of the fused mHC pre-mapping forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one batch: pack the weights (phi with
gamma folded in) and run the fused forward, i.e. one mhc_pre_forward call with
unpacked phi. Inputs are seeded synthetic tensors (synth), resident in HBM before
timing. Prints one JSON line; the GPU timing, the roofline of the dominant launch
(HIP events on the launch stream) and the CPU oracle baseline are all measured in
this run.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
METRIC = "tokens/s and achieved HBM GB/s (% of peak) for fused mHC pre fwd, n=4"


def algorithmic_bytes(wl, *, intermediates: bool) -> int:
    """Bytes the method must move once: x, phi, alpha, bias, gamma, pre_mix read once,
    every requested output written once (per token: 2K + 2D + 4n + 4n^2, plus
    4 + 4M + 4n + 2it*4n + 2it*4n^2 with the backward intermediates)."""
    T, n, D, M, it = wl.T, wl.n, wl.D, wl.M, wl.num_iters
    K = n * D
    b = T * 2 * K + M * K * 4 + wl.n_alpha * 4 + M * 4
    if wl.gamma:
        b += K * 4
    if wl.pre_mix:
        b += T * n * 4
    b += T * D * 2 + T * n * 4                      # hIn, hPost
    if wl.n_alpha == 3:
        b += T * n * n * 4                          # hRes
    if intermediates:
        b += T * 4 + T * M * 4 + T * n * 4          # invRms, hMix, hPre
        if wl.n_alpha == 3:
            b += 2 * it * T * n * 4 + 2 * it * T * n * n * 4
    return b


def cpu_baseline(inp, max_tokens: int):
    import numpy as np

    import oracle
    T = inp.wl.T
    ntok = min(T, max_tokens)
    tokens = np.arange(ntok, dtype=np.int64)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.forward(inp.x, inp.phi, inp.alpha, inp.bias, inp.gamma, inp.pre_mix,
                   num_iters=inp.wl.num_iters, norm_eps=inp.wl.norm_eps, hc_eps=inp.wl.hc_eps,
                   tokens=tokens)
    dt = time.perf_counter() - t0
    return {"value": ntok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {ntok} of {T} tokens of the same workload, all outputs, "
                      f"fp64 C oracle, {threads} OpenMP threads, {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="large_prefill_bwd")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this operator has no cross-GPU step and the "
              f"build targets a single MI355X (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import mhc_hyper_connection_amd as mhc
    import synth

    wl = synth.WORKLOADS[args.workload]
    print(f"[bench] generating {wl.name}: T={wl.T} n={wl.n} D={wl.D}", file=sys.stderr, flush=True)
    inp = synth.generate(wl)
    dev = torch.device("cuda", 0)

    def up(a):
        if a is None:
            return None
        if a.dtype.name == "uint16":
            return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x, phi, alpha, bias, gamma, pre_mix = map(up, (inp.x, inp.phi, inp.alpha, inp.bias,
                                                   inp.gamma, inp.pre_mix))
    run = mhc.PreForward(wl.T, wl.n, wl.D, wl.n_alpha, num_iters=wl.num_iters,
                         norm_eps=wl.norm_eps, hc_eps=wl.hc_eps,
                         need_backward=wl.need_backward, device=dev)
    out = run.alloc_outputs()
    stream = torch.cuda.current_stream(dev)

    def step():
        run(x, phi, alpha, bias, gamma, pre_mix, out=out)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    # timed region: exactly K steps, bracketed by device synchronisation; per-step HIP
    # events on the launch stream give the launch-group duration for the roofline
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    ev_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    ms_step = elapsed * 1e3 / args.steps
    ev_avg = sum(ev_ms) / len(ev_ms)

    b_alg = algorithmic_bytes(wl, intermediates=wl.need_backward)
    achieved = b_alg / (ev_avg * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": wl.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "n": wl.n, "D": wl.D, "n_alpha": wl.n_alpha,
                   "gamma": wl.gamma, "pre_mix": wl.pre_mix, "need_backward": wl.need_backward,
                   "num_iters": wl.num_iters, "step": "weight pack + fused forward (one mhc_pre_forward call)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "mhc_pre_forward launch group (pack + projection + hIn)",
                     "algorithmic_bytes": b_alg, "avg_launch_ms": ev_avg,
                     "min_launch_ms": min(ev_ms)},
    }
    if not args.no_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
