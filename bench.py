"""Benchmark of the mHC pre-mapping forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one batch: pack the weights (phi with
gamma folded in) and run the forward, i.e. one mhc_pre_forward call with unpacked
phi (pack, projection, per-token epilogue, hIn kernels). Inputs are seeded synthetic
tensors (synth), resident in HBM before timing. Prints one JSON line.

Measured in this run:
  value        tokens/s over exactly K back-to-back steps, wall clock between two device
               syncs (inputs resident in HBM);
  roofline     of the dominant kernel (the one with the largest average duration), its
               duration from HIP events that the library records on the launch stream around
               each of its kernels (mhc_pre_forward_timed), in a second pass of K steps, each
               preceded (outside the events) by a 512 MiB read that evicts the 256 MB
               Infinity Cache, so that no step reads its inputs from the previous step's cache
               (a read leaves only clean lines behind: a write's dirty lines would be written
               back during the next kernel and charged to it)
               lines (decode is timed back to back without it);
  waits_timed_out  mhc_pre_wait_status after the timed steps (1: a single-read wait gave up);
  cpu_baseline the fp64 C oracle on the host cores, on a bounded sample of tokens.
Read from profiles/ (rocprofv3 runs of this same script, taken while the kernel sources hash
to the SHA-256 recorded beside the figures; otherwise null):
  roofline.traffic  HBM bytes per launch of that kernel from FETCH_SIZE and WRITE_SIZE, each
               divided by the factor the same counter reads for a plain device copy of known
               size;
  roofline.rocprof_avg_us / frac_rocprof  that kernel's average duration in the kernel
               trace, and the fraction of peak it gives.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
METRIC = "tokens/s and achieved HBM GB/s (% of peak) for fused mHC pre fwd, n=4"
KERNEL_SOURCES = ("mhc_hyper_connection_amd/csrc/mhc_kernels.hip",
                  "mhc_hyper_connection_amd/csrc/mhc_device.h",
                  "mhc_hyper_connection_amd/csrc/mhc_plan.h")
# the classic path: without pre_mix the epilogue writes hIn too, so no kernel runs in the
# hIn stage on any path
KERNEL_NAMES = {"pack": "prepack_kernel", "projection": "proj_kernel",
                "epilogue": "epilogue_kernel", "hin": "(none)"}
# the single-read path runs one kernel in the projection stage and none in the hIn stage
KERNEL_NAMES_SINGLE_READ = dict(KERNEL_NAMES, projection="fused_kernel", hin="(none)")
# the one-launch path of a few tokens: one kernel, timed as the projection stage
KERNEL_NAMES_ONE_LAUNCH = dict(pack="(none)", projection="decode_kernel", epilogue="(none)", hin="(none)")
# the streaming path packs the weights inside its projection kernel (no pack launch)
KERNEL_NAMES_STREAM = dict(KERNEL_NAMES, pack="(none)", projection="proj_stream_kernel")
PATH_NAMES = {0: "classic", 1: "single-read", 2: "one-launch", 3: "streaming"}


def algorithmic_bytes(wl, *, intermediates: bool) -> int:
    """Bytes the method must move once for the whole call: x, phi, alpha, bias, gamma,
    pre_mix read once, every requested output written once (per token: 2K + 2D + 4n
    + 4n^2, plus 4 + 4M + 4n + 2it*4n + 2it*4n^2 with the backward intermediates)."""
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


def stage_bytes(wl, stage: str, single_read: bool = False, one_launch: bool = False) -> int:
    """Algorithmic bytes of one launch of a kernel: what that step of the method must
    read and write once. Intermediates of this implementation (packed weights, partial
    records, the hIn weights, the values exchanged between workgroups) are not counted.
      pack        phi (+ gamma) read once: 4MK (+ 4K)
      projection  x read once (2K per token) and phi once (4MK); with pre_mix it also
                  reads pre_mix (4n per token) and writes hIn (2D per token); the
                  single-read kernel writes hIn too (2D per token)
      epilogue    the per-token outputs: hPost, hRes, and the requested intermediates;
                  without pre_mix on the classic and streaming paths also x read once
                  and hIn written once (2K + 2D per token)
      hin         nothing (no path launches a kernel there)
    On the one-launch path the projection stage's kernel is the whole call
    (algorithmic_bytes) and the other stages launch nothing."""
    T, n, D, M, it = wl.T, wl.n, wl.D, wl.M, wl.num_iters
    K = n * D
    if one_launch:
        return algorithmic_bytes(wl, intermediates=wl.need_backward) if stage == "projection" else 0
    if stage == "pack":
        return M * K * 4 + (K * 4 if wl.gamma else 0)
    if stage == "projection":
        b = T * 2 * K + M * K * 4
        if wl.pre_mix:
            b += T * n * 4 + T * D * 2
        elif single_read:
            b += T * D * 2
        return b
    if stage == "epilogue":
        b = T * n * 4 + (T * n * n * 4 if wl.n_alpha == 3 else 0)
        if wl.need_backward:
            b += T * 4 + T * M * 4 + T * n * 4
            if wl.n_alpha == 3:
                b += 2 * it * T * n * 4 + 2 * it * T * n * n * 4
        if not (wl.pre_mix or single_read):
            b += T * 2 * K + T * D * 2
        return b
    if stage == "hin":
        return 0
    raise ValueError(stage)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/<kernel>_<workload>_counters.md, or None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip().strip("`").strip()
            if ":" in line and line.split(":", 1)[0].strip() in (
                    "source_sha256", "fetch_kib_per_dispatch", "write_kib_per_dispatch",
                    "fetch_factor", "write_factor"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    try:
        if vals["source_sha256"] != kernel_source_sha():
            return None, "kernel changed since the counters were taken"
        fetch = float(vals["fetch_kib_per_dispatch"]) * 1024 / float(vals["fetch_factor"])
        write = float(vals["write_kib_per_dispatch"]) * 1024 / float(vals["write_factor"])
    except (KeyError, ValueError):
        return None, "counter summary incomplete"
    return fetch + write, os.path.relpath(path, ROOT)


def trace_average(kernel: str, workload: str):
    """rocprofv3 average duration (µs) of `kernel` from profiles/<kernel>_<workload>_trace.md,
    or None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_trace.md")
    if not os.path.exists(path):
        return None, "no trace summary"
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip().strip("`").strip()
            if ":" in line and line.split(":", 1)[0].strip() in ("source_sha256", "avg_us"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    try:
        if vals["source_sha256"] != kernel_source_sha():
            return None, "kernel changed since the trace was taken"
        return float(vals["avg_us"]), os.path.relpath(path, ROOT)
    except (KeyError, ValueError):
        return None, "trace summary incomplete"


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
                   x_f16=inp.wl.x_f16, tokens=tokens)
    dt = time.perf_counter() - t0
    return {"value": ntok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {ntok} of {T} tokens of the same workload, all outputs, "
                      f"fp64 C oracle, {threads} OpenMP threads, {dt:.2f} s"}


def calibration_copy(torch, dev, mib: int, reps: int = 3):
    """A plain device copy of `mib` MiB, `reps` times: the known-size reference the
    counter runs divide FETCH_SIZE and WRITE_SIZE by (src read once, dst written once)."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    del src, dst


BWD_METRIC = "tokens/s and achieved HBM GB/s (% of peak) for the MhcPre(Sinkhorn) backward, n=4"


def bwd_algorithmic_bytes(T, n, D, gamma=False, x_post=False, num_iters=0) -> int:
    """Bytes the MhcPre backward must move once: x, gradHIn read and gradX written once
    (2K + 2D + 2K per token), the per-token gradients and saved values (gradHPost,
    gradHRes, invRms, hMix, hPre, hPost), phi read and gradPhi written once (4MK each),
    alpha / gradAlpha, gradBias, and with gamma: gamma read and gradGamma written (4K
    each); with gradXPost: it is read once (2K per token); with Sinkhorn iterations the
    saved planes are read once (2 it (4n + 4n^2) per token)."""
    M, K = n * n + 2 * n, n * D
    b = T * (2 * K + 2 * D + 2 * K + 4 * n + 4 * n * n + 4 + 4 * M + 4 * n + 4 * n)
    b += 2 * M * K * 4 + 3 * 4 * 2 + M * 4
    if gamma:
        b += 2 * K * 4
    if x_post:
        b += T * 2 * K
    b += T * 2 * num_iters * (4 * n + 4 * n * n)
    return b


def cpu_baseline_bwd(bi, max_tokens: int):
    """The fp64 oracle on the first tokens of the same inputs, as a problem of its own
    (every gradient over those tokens)."""
    import oracle
    ntok = min(bi.T, max_tokens)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    it = bi.num_iters
    oracle.backward(bi.x[:ntok], bi.phi, bi.alpha, bi.grad_h_in[:ntok], bi.grad_h_post[:ntok],
                    bi.grad_h_res[:ntok], bi.inv_rms[:ntok], bi.h_mix[:ntok], bi.h_pre[:ntok],
                    bi.h_post[:ntok], bi.gamma, None if bi.grad_x_post is None else bi.grad_x_post[:ntok],
                    hc_eps=bi.hc_eps, num_iters=it,
                    sum_out=bi.sum_out[:, :ntok] if it else None,
                    norm_out=bi.norm_out[:, :ntok] if it else None, x_f16=bi.x_f16)
    dt = time.perf_counter() - t0
    return {"value": ntok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {ntok} of {bi.T} tokens as a problem of their own, every gradient, "
                      f"fp64 C oracle, {threads} OpenMP threads, {dt:.2f} s"}


def main_backward(args):
    """--op backward: one step = one mhc_pre_backward call at the large prefill shape
    (T = 16384, n = 4, D = 7168, no gamma, no gradXPost), through --bwd-iters Sinkhorn
    iterations (20, as the forward's; 0 = the MhcPre backward); --bwd-f16: x, gradHIn and
    gradX in fp16."""
    import torch

    import mhc_hyper_connection_amd as mhc
    import synth

    T, n, D = 16384, 4, 7168
    print(f"[bench] generating backward inputs T={T} n={n} D={D}", file=sys.stderr, flush=True)
    it = args.bwd_iters
    f16 = args.bwd_f16
    bi = synth.backward_inputs(T, n, D, sinkhorn_iters=it, seed=1003, x_f16=f16)
    dev = torch.device("cuda", 0)

    def up(a):
        if a is None:
            return None
        if a.dtype.name == "uint16":
            return torch.from_numpy(a.view("int16")).view(torch.float16 if f16 else torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    args_dev = [up(a) for a in (bi.x, bi.phi, bi.alpha, bi.grad_h_in, bi.grad_h_post, bi.grad_h_res,
                                bi.inv_rms, bi.h_mix, bi.h_pre, bi.h_post, bi.gamma, bi.grad_x_post)]
    run = mhc.PreBackward(T, n, D, hc_eps=bi.hc_eps, num_iters=it, x_f16=f16, device=dev)
    out = run.alloc_outputs(bi.gamma is not None)
    planes = {"sum_out": up(bi.sum_out), "norm_out": up(bi.norm_out)} if it else {}
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run(*args_dev, out=out, **planes)
    torch.cuda.synchronize(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        run(*args_dev, out=out, **planes)
        b.record(stream)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    call_us = sum(a.elapsed_time(b) for a, b in evs) * 1e3 / len(evs)
    ab = bwd_algorithmic_bytes(T, n, D, num_iters=it)
    achieved = ab / (call_us * 1e-6) / 1e9
    line = {
        "metric": BWD_METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16" if f16 else "bf16",
        "data": "synthetic",
        "config": {"workload": "large_prefill_backward" + ("_f16" if f16 else ""), "T": T, "n": n, "D": D,
                   "gamma": False,
                   "grad_x_post": False, "num_iters": it,
                   "step": "one mhc_pre_backward call (all of its kernels)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "whole call",
                     "algorithmic_bytes": ab, "avg_launch_us": call_us},
    }
    if not args.no_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_bwd(bi, args.cpu_tokens_bwd)
    print(json.dumps(line), flush=True)


POST_METRIC = "tokens/s and achieved HBM GB/s (% of peak) for hc_post (the mHC post-mapping), n=4"


def post_algorithmic_bytes(T, n, D) -> int:
    """hc_post moves x (2D) and the n streams (2nD) in, the n output streams (2nD) out,
    plus post (4n) and comb (4n^2), once per token."""
    return T * (2 * D + 2 * n * D + 4 * n + 4 * n * n + 2 * n * D)


def main_post(args):
    """--op post: one step = one mhc_post call at the large prefill shape (T = 16384,
    n = 4, D = 7168)."""
    import numpy as np
    import torch

    import mhc_hyper_connection_amd as mhc
    import synth

    T, n, D = 16384, 4, 7168
    print(f"[bench] generating hc_post inputs T={T} n={n} D={D}", file=sys.stderr, flush=True)
    pi = synth.post_inputs(T, n, D, seed=1004)
    dev = torch.device("cuda", 0)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x, res, post, comb = (up(a) for a in (pi.x, pi.residual, pi.post, pi.comb))
    out = torch.empty((T, n, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        mhc.mhc_post(x, res, post, comb, out=out)
    torch.cuda.synchronize(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        mhc.mhc_post(x, res, post, comb, out=out)
        b.record(stream)
    torch.cuda.synchronize(dev)
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    call_us = sum(a.elapsed_time(b) for a, b in evs) * 1e3 / len(evs)
    ab = post_algorithmic_bytes(T, n, D)
    achieved = ab / (call_us * 1e-6) / 1e9
    line = {
        "metric": POST_METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "large_prefill_post", "T": T, "n": n, "D": D,
                   "step": "one mhc_post call (one kernel)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "post_kernel",
                     "algorithmic_bytes": ab, "avg_launch_us": call_us},
    }
    if not args.no_cpu:
        import oracle
        ntok = min(T, 4096)
        threads = oracle.max_threads()
        c0 = time.perf_counter()
        oracle.post(pi.x[:ntok], pi.residual[:ntok], pi.post[:ntok], pi.comb[:ntok])
        dt = time.perf_counter() - c0
        line["cpu_baseline"] = {"value": ntok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                                "sample": f"first {ntok} of {T} tokens, fp64 C oracle, {threads} OpenMP threads, "
                                          f"{dt:.2f} s"}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="large_prefill_bwd",
                    help="a synth workload; a name ending in _f16 runs that workload with x and "
                         "hIn in binary16")
    ap.add_argument("--cpu-tokens", type=int, default=65536,
                    help="tokens of the workload the CPU oracle baseline runs on (bounded)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--graph-replays", type=int, default=0,
                    help="after the timed steps, capture one step into a HIP graph and report "
                         "its per-replay time over this many replays")
    ap.add_argument("--prepacked-calls", type=int, default=0,
                    help="after the timed steps, time this many back-to-back calls with weights "
                         "packed once beforehand (mhc_pre_prepack), as a serving loop calls it")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="size of the read that evicts the Infinity Cache before each step of the "
                         "per-kernel pass (0: none; decode never flushes)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run a plain copy of this size first (for counter calibration)")
    ap.add_argument("--op", choices=("forward", "backward", "post"), default="forward",
                    help="forward (default): the pre-mapping forward line; backward: the "
                         "MhcPre backward at the large prefill shape; post: hc_post at that shape")
    ap.add_argument("--bwd-iters", type=int, default=20,
                    help="Sinkhorn iterations of the backward (0: the MhcPre backward)")
    ap.add_argument("--bwd-f16", action="store_true",
                    help="the backward with x, gradHIn and gradX in fp16 (else bf16)")
    ap.add_argument("--cpu-tokens-bwd", type=int, default=16384,
                    help="tokens the CPU oracle baseline of the backward runs on (bounded)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the forward has no cross-GPU step and this "
              f"build runs on a single MI355X (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.op == "backward":
        main_backward(args)
        return
    if args.op == "post":
        main_post(args)
        return

    import torch

    import mhc_hyper_connection_amd as mhc
    import synth

    f16 = args.workload.endswith("_f16")
    wl = synth.WORKLOADS[args.workload[:-4] if f16 else args.workload]
    if f16:
        import dataclasses
        wl = dataclasses.replace(wl, name=args.workload, x_f16=True)
    print(f"[bench] generating {wl.name}: T={wl.T} n={wl.n} D={wl.D}", file=sys.stderr, flush=True)
    inp = synth.generate(wl)
    dev = torch.device("cuda", 0)

    def up(a):
        if a is None:
            return None
        if a.dtype.name == "uint16":
            return torch.from_numpy(a.view("int16")).view(torch.float16 if f16 else torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x, phi, alpha, bias, gamma, pre_mix = map(up, (inp.x, inp.phi, inp.alpha, inp.bias,
                                                   inp.gamma, inp.pre_mix))
    run = mhc.PreForward(wl.T, wl.n, wl.D, wl.n_alpha, num_iters=wl.num_iters,
                         norm_eps=wl.norm_eps, hc_eps=wl.hc_eps,
                         need_backward=wl.need_backward, device=dev, x_f16=f16)
    out = run.alloc_outputs()
    stream = torch.cuda.current_stream(dev)
    path = run.path(pre_mix is not None)
    single_read, one_launch, streaming = path == 1, path == 2, path == 3
    names = (KERNEL_NAMES_ONE_LAUNCH if one_launch else KERNEL_NAMES_SINGLE_READ if single_read
             else KERNEL_NAMES_STREAM if streaming else KERNEL_NAMES)

    if args.calib_copy_mib > 0:
        print(f"[bench] calibration copy {args.calib_copy_mib} MiB", file=sys.stderr, flush=True)
        calibration_copy(torch, dev, args.calib_copy_mib)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run(x, phi, alpha, bias, gamma, pre_mix, out=out)
    torch.cuda.synchronize(dev)

    # timed region: exactly K back-to-back steps, bracketed by device synchronisation
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run(x, phi, alpha, bias, gamma, pre_mix, out=out)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    waits_timed_out = run.wait_status()
    if waits_timed_out:
        print("[bench] WARNING: a kernel's wait gave up (its tokens hold NaN)", file=sys.stderr, flush=True)

    # per-kernel durations: a second pass of K steps with HIP events on the launch stream;
    # one set of events per step, each recorded once here so that its HIP event exists
    # before the library records it. Boundaries around a stage that launches nothing (the
    # pack and hIn stages of the single-read path, the pack stage of the streaming path and
    # its hIn stage with pre_mix; all but the one kernel of the one-launch
    # path) are not recorded: each record costs a few microseconds on the stream. Before each step (outside its events) a 512 MiB
    # read evicts the Infinity Cache, except for decode (launch-bound, back to back). A read,
    # not a write: a write would leave 256 MB of dirty lines that the next kernel's misses
    # write back to HBM, charging that kernel with traffic that is not its own (a 32 µs
    # projection measured 56 µs after such a write). The buffer is filled once, and the sync
    # below lets those dirty lines drain before the pass.
    flush = None
    flush_sink = None
    if args.flush_mib > 0 and wl.name != "decode":
        flush = torch.full((args.flush_mib << 18,), 1, dtype=torch.int32, device=dev)
        flush_sink = torch.empty((), dtype=torch.int32, device=dev)
        torch.sum(flush, dim=0, dtype=torch.int32, out=flush_sink)
    wanted = [True] * mhc.FORWARD_EVENTS
    if single_read:
        wanted[0] = wanted[-1] = False
    if streaming:
        wanted[0] = False
    if not one_launch:
        wanted[-1] = False   # no path launches a kernel in the hIn stage
    if one_launch:
        wanted = [False, True, True, False, False]
    evs = [[torch.cuda.Event(enable_timing=True) if w else None for w in wanted]
           for _ in range(args.steps)]
    for row in evs:
        for e in row:
            if e is not None:
                e.record(stream)
    torch.cuda.synchronize(dev)
    print(f"[bench] per-kernel pass {args.steps} steps" + (" (cache flushed)" if flush is not None else ""),
          file=sys.stderr, flush=True)
    for step, row in enumerate(evs):
        if flush is not None:
            torch.sum(flush, dim=0, dtype=torch.int32, out=flush_sink)
        run(x, phi, alpha, bias, gamma, pre_mix, out=out, events=row)
    torch.cuda.synchronize(dev)
    waits_timed_out |= run.wait_status()
    del flush, flush_sink

    kernels = {}
    for i, stage in enumerate(mhc.STAGES):
        if not (wanted[i] and wanted[i + 1]):
            kernels[stage] = {"kernel": names[stage], "avg_us": 0.0, "min_us": 0.0,
                              "algorithmic_bytes": stage_bytes(wl, stage, single_read, one_launch),
                              "note": "launches nothing on this path; not recorded"}
            continue
        ms = [row[i].elapsed_time(row[i + 1]) for row in evs]
        kernels[stage] = {"kernel": names[stage], "avg_us": 1e3 * sum(ms) / len(ms),
                          "min_us": 1e3 * min(ms),
                          "algorithmic_bytes": stage_bytes(wl, stage, single_read, one_launch)}
    first, last = wanted.index(True), len(wanted) - 1 - wanted[::-1].index(True)
    call_us = [1e3 * row[first].elapsed_time(row[last]) for row in evs]
    dom = max(kernels, key=lambda s: kernels[s]["avg_us"])
    kd = kernels[dom]
    achieved = kd["algorithmic_bytes"] / (kd["avg_us"] * 1e-6) / 1e9
    traffic, traffic_src = counter_traffic(names[dom], wl.name)
    rp_us, rp_src = trace_average(names[dom], wl.name)
    b_call = algorithmic_bytes(wl, intermediates=wl.need_backward)
    call_avg = sum(call_us) / len(call_us)

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
        "dtype": "f16" if f16 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "n": wl.n, "D": wl.D, "n_alpha": wl.n_alpha,
                   "gamma": wl.gamma, "pre_mix": wl.pre_mix, "need_backward": wl.need_backward,
                   "num_iters": wl.num_iters,
                   "path": PATH_NAMES[path],
                   "step": "weight pack + forward (one mhc_pre_forward call, unpacked phi)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kd["kernel"], "algorithmic_bytes": kd["algorithmic_bytes"],
                     "avg_launch_us": kd["avg_us"], "traffic_source": traffic_src,
                     "rocprof_avg_us": rp_us,
                     "frac_rocprof": None if rp_us is None else kd["algorithmic_bytes"] / (rp_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                     "rocprof_source": rp_src},
        "waits_timed_out": waits_timed_out,
        "call": {"algorithmic_bytes": b_call, "avg_us": call_avg,
                 "achieved_GBs": b_call / (call_avg * 1e-6) / 1e9,
                 "frac": b_call / (call_avg * 1e-6) / 1e9 / HBM_PEAK_GBS},
        "kernels": kernels,
    }
    if args.prepacked_calls > 0:
        # serving-loop form: weights packed once, then back-to-back calls, HIP events around
        # all of them on the launch stream (outside the timed region)
        print(f"[bench] prepacked calls {args.prepacked_calls}", file=sys.stderr, flush=True)
        pk = run.prepack(phi, gamma)
        for _ in range(10):
            run(x, None, alpha, bias, None, pre_mix, phi_packed=pk, out=out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.prepacked_calls):
            run(x, None, alpha, bias, None, pre_mix, phi_packed=pk, out=out)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        waits_timed_out |= run.wait_status()
        line["waits_timed_out"] = waits_timed_out
        us = 1e3 * e0.elapsed_time(e1) / args.prepacked_calls
        line["prepacked"] = {"calls": args.prepacked_calls, "us_per_call": us, "tokens_per_s": wl.T / (us * 1e-6)}
    if args.graph_replays > 0:
        # launch-bound sizes: the same step replayed from a captured graph (outside the
        # timed region)
        print(f"[bench] graph replays {args.graph_replays}", file=sys.stderr, flush=True)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(x, phi, alpha, bias, gamma, pre_mix, out=out)
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.graph_replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize(dev)
        us = 1e3 * e0.elapsed_time(e1) / args.graph_replays
        line["graph"] = {"replays": args.graph_replays, "us_per_call": us,
                         "tokens_per_s": wl.T / (us * 1e-6)}
    if not args.no_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
