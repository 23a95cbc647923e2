"""Helpers for the GPU parity tests: run the HIP library through the C-ABI (via the
thin binding) and compare with the fp64 oracle.

Acceptance rule (written here once, used by every GPU test):
  fp32 outputs (invRms, hMix, hPre, hPost, hRes, normOut, sumOut), every element:
      |gpu - ref| <= 1e-6 + 2e-4 * |ref|
  hIn (bf16), every element: within 1 bf16 ulp of the oracle's correctly rounded value
      (ordered-integer distance <= 1), or, where the exact sum cancels, within the error
      that the fp32 weights carry into it:  |gpu - ref| <= 2^-20 * sum_i |w_i * x_i,d|.
      The second branch only matters when |hIn| is far below its terms; the report
      counts how many elements needed it.
"""
from __future__ import annotations

import numpy as np

import oracle
from synth import Inputs, bf16_bits_to_f32

FP32_ATOL = 1e-6
FP32_RTOL = 2e-4
HIN_CANCEL = 2.0 ** -20


def torch_mod():
    import torch
    return torch


def device():
    torch = torch_mod()
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda", 0)


def to_dev(a, dev, f16=False):
    """numpy -> device tensor; uint16 arrays are bf16 bits (fp16 bits with f16)."""
    torch = torch_mod()
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.float16 if f16 else torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host(t):
    torch = torch_mod()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def gpu_forward(inp: Inputs, *, need_backward=None, intermediates=True, packed=False,
                runner=None, repeat=1):
    """Run the library on `inp`. Returns numpy outputs (h_in as bf16 bits)."""
    import mhc_hyper_connection_amd as mhc
    torch = torch_mod()
    dev = device()
    wl = inp.wl
    nb = wl.need_backward if need_backward is None else need_backward
    if runner is None:
        runner = mhc.PreForward(wl.T, wl.n, wl.D, wl.n_alpha, num_iters=wl.num_iters,
                                norm_eps=wl.norm_eps, hc_eps=wl.hc_eps, need_backward=nb,
                                device=dev, x_f16=wl.x_f16)
    x = to_dev(inp.x, dev, wl.x_f16)
    phi = to_dev(inp.phi, dev)
    alpha = to_dev(inp.alpha, dev)
    bias = to_dev(inp.bias, dev)
    gamma = to_dev(inp.gamma, dev)
    pre_mix = to_dev(inp.pre_mix, dev)
    pk = runner.prepack(phi, gamma) if packed else None
    out = runner.alloc_outputs(intermediates=intermediates or nb)
    results = []
    for _ in range(repeat):
        for v in out.values():
            if v.dtype in (torch.bfloat16, torch.float16):
                v.view(torch.int16).fill_(0x7FC0 if v.dtype == torch.bfloat16 else 0x7E00)   # NaN
            else:
                v.fill_(float("nan"))
        runner(x, None if packed else phi, alpha, bias, None if packed else gamma, pre_mix,
               phi_packed=pk, out=out)
        torch.cuda.synchronize(dev)
        results.append({k: to_host(v) for k, v in out.items()})
    return results if repeat > 1 else results[0]


def run_oracle(inp: Inputs, tokens=None, want_steps=True):
    wl = inp.wl
    return oracle.forward(inp.x, inp.phi, inp.alpha, inp.bias, inp.gamma, inp.pre_mix,
                          num_iters=wl.num_iters, norm_eps=wl.norm_eps, hc_eps=wl.hc_eps, x_f16=wl.x_f16,
                          tokens=tokens, want_sinkhorn_steps=want_steps)


def _fp32_check(name, g, r, report):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
    err = np.abs(g - r)
    lim = FP32_ATOL + FP32_RTOL * np.abs(r)
    bad = ~(err <= lim)          # NaN counts as a failure
    worst = int(np.argmax(np.where(np.isnan(err), np.inf, err / lim))) if err.size else 0
    report[name] = dict(n=int(err.size), fail=int(bad.sum()),
                        max_abs=float(np.nanmax(err)) if err.size else 0.0,
                        max_ratio=float(np.nanmax(err / lim)) if err.size else 0.0,
                        worst=(np.unravel_index(worst, err.shape), float(g.flat[worst]),
                               float(r.flat[worst])) if err.size else None)


def bf16_ordered(bits):
    b = np.asarray(bits).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _hin_check(g_bits, ref_double, ref_bits, scale, report, f16=False):
    # sign-magnitude 16-bit formats: the ordered distance counts ulps in bf16 and fp16 alike
    dist = np.abs(bf16_ordered(g_bits) - bf16_ordered(ref_bits))
    g = (np.asarray(g_bits, np.uint16).view(np.float16) if f16 else bf16_bits_to_f32(g_bits)).astype(np.float64)
    within_ulp = dist <= 1
    within_cancel = np.abs(g - ref_double) <= HIN_CANCEL * scale
    ok = within_ulp | within_cancel
    report["h_in"] = dict(n=int(dist.size), fail=int((~ok).sum()), max_ulp=int(dist.max()) if dist.size else 0,
                          ulp_gt_1_but_cancel_ok=int((~within_ulp & within_cancel).sum()),
                          exact=int((dist == 0).sum()))


def compare(gpu: dict, orc, inp: Inputs, tokens=None, *, check_steps=True):
    """Elementwise acceptance of `gpu` (full-T outputs) against `orc` (for `tokens`).
    Returns the report; raises AssertionError listing every failing output."""
    wl = inp.wl
    tok = np.arange(wl.T) if tokens is None else np.asarray(tokens)
    rep = {}
    _fp32_check("h_post", gpu["h_post"][tok], orc.h_post, rep)
    if wl.n_alpha == 3:
        _fp32_check("h_res", gpu["h_res"][tok], orc.h_res, rep)
    elif "h_res" in gpu:
        rep["h_res_zero"] = dict(n=int(gpu["h_res"].size), fail=int((gpu["h_res"] != 0).sum()))
    if "inv_rms" in gpu:
        _fp32_check("inv_rms", gpu["inv_rms"][tok], orc.inv_rms, rep)
    if "h_mix" in gpu:
        _fp32_check("h_mix", gpu["h_mix"][tok], orc.h_mix, rep)
    if "h_pre" in gpu:
        _fp32_check("h_pre", gpu["h_pre"][tok], orc.h_pre, rep)
    if check_steps and "sum_out" in gpu and orc.sum_out is not None:
        _fp32_check("sum_out", gpu["sum_out"][:, tok], orc.sum_out, rep)
        _fp32_check("norm_out", gpu["norm_out"][:, tok], orc.norm_out, rep)
    x = (inp.x[tok].view(np.float16) if wl.x_f16 else bf16_bits_to_f32(inp.x[tok])).astype(np.float64)
    w = (inp.pre_mix[tok].astype(np.float64) if inp.pre_mix is not None else orc.h_pre)
    scale = np.einsum("ti,tid->td", np.abs(w), np.abs(x))
    _hin_check(gpu["h_in"][tok], orc.h_in, orc.h_in_bf16, scale, rep, wl.x_f16)
    failing = {k: v for k, v in rep.items() if v.get("fail", 0)}
    if failing:
        raise AssertionError(f"parity failures: {failing}")
    return rep


def summary(rep) -> str:
    parts = []
    for k, v in rep.items():
        if "max_ratio" in v:
            parts.append(f"{k}: max|d|={v['max_abs']:.2e} ratio={v['max_ratio']:.3f}")
        elif k == "h_in":
            parts.append(f"h_in: max_ulp={v['max_ulp']} exact={v['exact']}/{v['n']} "
                         f"cancel={v['ulp_gt_1_but_cancel_ok']}")
    return "; ".join(parts)
