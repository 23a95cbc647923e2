"""GPU parity of the MhcPre backward: the HIP library (through the C-ABI) against the
fp64 oracle (oracle/mhc_oracle_bwd.c), on seeded synthetic inputs (synth.backward_inputs).

Acceptance rule, derived from the arithmetic of the GPU path:
  gradX (bf16, or fp16 with fp16 inputs), every element: within 1 ulp of the oracle's
      correctly rounded value, or |gpu - ref| <= 2^-18 * A, A = the sum of |terms| of the
      element (the oracle's grad_x_abs). gradX is formed in fp32 from five terms, one of
      them a split-bf16 matrix-core product accurate to ~2^-22 of its terms, so the fp32
      error e is far below 2^-18 A. Rounding a value within e of the exact one lands within
      1 ulp of the correctly rounded result whenever e < 1 ulp; otherwise the result is
      within half an ulp + e <= 1.5 e of the exact value. The rule is the same for both
      formats; the branch matters only where the terms cancel.
  gradPhi, gradGamma (f32), every element: |gpu - ref| <= 2e-4 |ref| + 2^-14 A, A the
      oracle's sum of |terms|. Each is an fp32 sum over the tokens of one group (up to a
      few hundred rounding steps into the accumulator, each <= 2^-24 of a partial sum
      <= A), then an fp64 sum over groups; 2^-14 A leaves a 4x margin over that bound,
      and 2e-4 |ref| is the forward's relative tolerance.
  gradAlpha, gradBias (f32): fp64 per-token terms summed in fp64, one rounding to f32:
      |gpu - ref| <= 1e-6 |ref| + 2^-30 A.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import bf16_ordered, device, to_dev, to_host
from synth import bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def gpu_backward(bi, repeat=1):
    import mhc_hyper_connection_amd as mhc
    import torch
    dev = device()
    it = bi.num_iters
    r = mhc.PreBackward(bi.T, bi.n, bi.D, hc_eps=bi.hc_eps, num_iters=it, x_f16=bi.x_f16, device=dev)
    args = [to_dev(a, dev, bi.x_f16) for a in (bi.x, bi.phi, bi.alpha, bi.grad_h_in, bi.grad_h_post,
                                     bi.grad_h_res, bi.inv_rms, bi.h_mix, bi.h_pre, bi.h_post,
                                     bi.gamma, bi.grad_x_post)]
    planes = {}
    if it:
        planes = {"sum_out": to_dev(bi.sum_out, dev), "norm_out": to_dev(bi.norm_out, dev)}
    out = r.alloc_outputs(bi.gamma is not None)
    results = []
    for _ in range(repeat):
        for v in out.values():
            if v.dtype in (torch.bfloat16, torch.float16):   # NaN: anything not written shows
                v.view(torch.int16).fill_(0x7FC0 if v.dtype == torch.bfloat16 else 0x7E00)
            else:
                v.fill_(float("nan"))
        r(*args, out=out, **planes)
        torch.cuda.synchronize(dev)
        results.append({k: to_host(v) for k, v in out.items()})
    return results if repeat > 1 else results[0]


def run_oracle(bi, tokens=None):
    return oracle.backward(bi.x, bi.phi, bi.alpha, bi.grad_h_in, bi.grad_h_post, bi.grad_h_res,
                           bi.inv_rms, bi.h_mix, bi.h_pre, bi.h_post, bi.gamma, bi.grad_x_post,
                           hc_eps=bi.hc_eps, tokens=tokens, num_iters=bi.num_iters,
                           sum_out=bi.sum_out, norm_out=bi.norm_out, x_f16=bi.x_f16)


def sinkhorn_inputs(T, n, D, it, *, gamma=False, post=False, seed=31, f16=False):
    """MhcPreSinkhorn backward inputs: the forward's saved values (invRms, hMix, hPre,
    hPost, sumOut, normOut) come from the fp64 oracle forward on seeded inputs, rounded
    to float32 as the forward emits them; the incoming gradients are seeded draws."""
    inp = synth.custom(T, n, D, gamma=gamma, need_backward=True, num_iters=it, seed=seed, x_f16=f16)
    f = oracle.forward(inp.x, inp.phi, inp.alpha, inp.bias, inp.gamma, num_iters=it,
                       want_h_in=False, x_f16=f16)
    g = synth.backward_inputs(T, n, D, x_post=post, seed=seed + 1000, x_f16=f16)
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return synth.BwdInputs(T, n, D, inp.x, inp.phi, inp.alpha, g.grad_h_in, g.grad_h_post,
                           g.grad_h_res, f32(f.inv_rms), f32(f.h_mix), f32(f.h_pre), f32(f.h_post),
                           inp.gamma, g.grad_x_post, num_iters=it, sum_out=f32(f.sum_out),
                           norm_out=f32(f.norm_out), x_f16=f16)


def _bound_check(name, g, r, a, rtol, atab, rep):
    g = np.asarray(g, dtype=np.float64)
    err = np.abs(g - r)
    lim = rtol * np.abs(r) + atab * a
    bad = ~(err <= lim)
    ratio = np.where(lim > 0, err / np.where(lim > 0, lim, 1), np.where(err > 0, np.inf, 0))
    rep[name] = dict(n=int(err.size), fail=int(bad.sum()), max_abs=float(np.nanmax(err)) if err.size else 0,
                     max_ratio=float(np.nanmax(ratio)) if err.size else 0)


def compare(g, o, bi, tokens=None):
    tok = np.arange(bi.T) if tokens is None else np.asarray(tokens)
    rep = {}
    gx_all = g["grad_x"][tok]
    nel = fails = max_ulp = cancel_used = 0
    for r0 in range(0, len(tok), 1024):   # rows in chunks: bounded temporaries at the large shape
        sl = slice(r0, min(len(tok), r0 + 1024))
        gx = gx_all[sl]
        dist = np.abs(bf16_ordered(gx) - bf16_ordered(o.grad_x_bits[sl]))
        gv = gx.view(np.float16) if bi.x_f16 else bf16_bits_to_f32(gx)
        cancel = np.abs(gv.astype(np.float64) - o.grad_x[sl]) <= 2.0 ** -18 * o.grad_x_abs[sl]
        ok = (dist <= 1) | cancel
        nel += int(dist.size)
        fails += int((~ok).sum())
        max_ulp = max(max_ulp, int(dist.max()) if dist.size else 0)
        cancel_used += int(((dist > 1) & cancel).sum())
    rep["grad_x"] = dict(n=nel, fail=fails, max_ulp=max_ulp, cancel_branch=cancel_used)
    _bound_check("grad_phi", g["grad_phi"], o.grad_phi, o.grad_phi_abs, 2e-4, 2.0 ** -14, rep)
    _bound_check("grad_alpha", g["grad_alpha"], o.grad_alpha, o.grad_alpha_abs, 1e-6, 2.0 ** -30, rep)
    _bound_check("grad_bias", g["grad_bias"], o.grad_bias, o.grad_bias_abs, 1e-6, 2.0 ** -30, rep)
    if bi.gamma is not None:
        _bound_check("grad_gamma", g["grad_gamma"], o.grad_gamma, o.grad_gamma_abs, 2e-4, 2.0 ** -14, rep)
    print(f"[parity-bwd] " + " ".join(f"{k}:fail={v['fail']}/{v['n']}" for k, v in rep.items()),
          file=sys.stderr, flush=True)
    bad = {k: v for k, v in rep.items() if v["fail"]}
    assert not bad, f"backward parity failures: {bad}"
    return rep


CASES = [
    # (name, T, n, D, gamma, grad_x_post, seed)
    ("T1_D8", 1, 4, 8, False, False, 1),
    ("T10_D8_gamma_post", 10, 4, 8, True, True, 2),
    ("T65_D40_ragged", 65, 4, 40, False, True, 3),
    ("T130_D512_gamma", 130, 4, 512, True, False, 4),
    ("T64_D7168", 64, 4, 7168, False, False, 5),
    ("T200_D7168_gamma_post", 200, 4, 7168, True, True, 6),
    ("T300_D1000", 300, 4, 1000, False, False, 7),
    ("n8_T17_D24", 17, 8, 24, False, False, 8),
    ("n8_T70_D256_gamma_post", 70, 8, 256, True, True, 9),
    ("n8_T129_D2048", 129, 8, 2048, False, False, 10),
    ("T4097_D256_groups", 4097, 4, 256, True, False, 11),
    # n = 6 (48 phi rows: two 32-row K-steps, two streams per main-pass workgroup)
    ("n6_T1_D8", 1, 6, 8, False, False, 71),
    ("n6_T17_D24", 17, 6, 24, False, False, 72),
    ("n6_T70_D256_gamma_post", 70, 6, 256, True, True, 73),
    ("n6_T129_D2048", 129, 6, 2048, False, False, 74),
    ("n6_T300_D7168_gamma", 300, 6, 7168, True, False, 75),
    ("n6_T4097_D256_groups_post", 4097, 6, 256, False, True, 76),
    # the largest D the backward takes, for each n
    ("Dmax_T70_D16384_gamma_post", 70, 4, 16384, True, True, 91),
    ("n6_Dmax_T33_D16384", 33, 6, 16384, False, False, 92),
    ("n8_Dmax_T20_D16384_gamma", 20, 8, 16384, True, False, 93),
]


@pytest.mark.parametrize("name,T,n,D,gamma,post,seed", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(name, T, n, D, gamma, post, seed):
    print(f"[case] backward {name} T={T} n={n} D={D} gamma={gamma} post={post}", file=sys.stderr, flush=True)
    bi = synth.backward_inputs(T, n, D, gamma=gamma, x_post=post, seed=seed)
    compare(gpu_backward(bi), run_oracle(bi), bi)


F16_CASES = [
    # fp16 x, gradHIn, gradXPost and gradX: (name, T, n, D, gamma, grad_x_post, seed)
    ("f16_T1_D8", 1, 4, 8, False, False, 61),
    ("f16_T65_D40_ragged_gamma_post", 65, 4, 40, True, True, 62),
    ("f16_T200_D7168_gamma_post", 200, 4, 7168, True, True, 63),
    ("f16_T300_D1000", 300, 4, 1000, False, False, 64),
    ("f16_n8_T70_D256_gamma_post", 70, 8, 256, True, True, 65),
    ("f16_n8_T129_D2048", 129, 8, 2048, False, False, 66),
    ("f16_T4097_D256_groups", 4097, 4, 256, True, False, 67),
    ("f16_n6_T65_D512_gamma_post", 65, 6, 512, True, True, 69),
    ("f16_Dmax_T40_D16384_gamma_post", 40, 4, 16384, True, True, 94),
]


@pytest.mark.parametrize("name,T,n,D,gamma,post,seed", F16_CASES, ids=[c[0] for c in F16_CASES])
def test_backward_parity_f16(name, T, n, D, gamma, post, seed):
    print(f"[case] backward {name} T={T} n={n} D={D} gamma={gamma} post={post}", file=sys.stderr, flush=True)
    bi = synth.backward_inputs(T, n, D, gamma=gamma, x_post=post, seed=seed, x_f16=True)
    compare(gpu_backward(bi), run_oracle(bi), bi)


def test_backward_f16_through_the_wrapper():
    # mhc_pre_backward picks fp16 from x's dtype, on [B, S, n, D] tensors: the same bits
    # as the launcher it builds
    import mhc_hyper_connection_amd as mhc
    print("[case] backward f16 wrapper B=2 S=33 n=4 D=512", file=sys.stderr, flush=True)
    bi = synth.backward_inputs(66, 4, 512, gamma=True, x_post=True, seed=68, x_f16=True)
    want = gpu_backward(bi)
    dev = device()
    t = lambda a: to_dev(a, dev, True)
    got = mhc.mhc_pre_backward(t(bi.x).reshape(2, 33, 4, 512), t(bi.phi), t(bi.alpha),
                               t(bi.grad_h_in).reshape(2, 33, 512), t(bi.grad_h_post).reshape(2, 33, 4),
                               t(bi.grad_h_res).reshape(2, 33, 4, 4), t(bi.inv_rms).reshape(2, 33),
                               t(bi.h_mix).reshape(2, 33, -1), t(bi.h_pre).reshape(2, 33, 4),
                               t(bi.h_post).reshape(2, 33, 4), t(bi.gamma),
                               t(bi.grad_x_post).reshape(2, 33, 4, 512), hc_eps=bi.hc_eps)
    import torch
    assert got["grad_x"].dtype == torch.float16 and got["grad_x"].shape == (2, 33, 4, 512)
    for k, v in got.items():
        h = to_host(v.reshape(want[k].shape))
        assert np.array_equal(h.view(np.uint8), want[k].view(np.uint8)), k


def test_backward_empty_tokens():
    print("[case] backward T=0", file=sys.stderr, flush=True)
    bi = synth.backward_inputs(0, 4, 256, gamma=True, seed=12)
    g = gpu_backward(bi)
    for k in ("grad_phi", "grad_alpha", "grad_bias", "grad_gamma"):
        assert np.all(g[k] == 0.0), k


def test_backward_bitwise_reproducible():
    print("[case] backward determinism T=300 D=2048", file=sys.stderr, flush=True)
    bi = synth.backward_inputs(300, 4, 2048, gamma=True, x_post=True, seed=13)
    a, b = gpu_backward(bi, repeat=2)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


def test_backward_mid_workload_shape():
    # the mid prefill shape (T = 4096, n = 4, D = 4096, gamma): every gradient, every row
    print("[case] backward mid T=4096 D=4096 gamma", file=sys.stderr, flush=True)
    bi = synth.backward_inputs(4096, 4, 4096, gamma=True, seed=14)
    compare(gpu_backward(bi), run_oracle(bi), bi)


def test_backward_large_workload_shape():
    # the large prefill shape (T = 16384, n = 4, D = 7168), as the benchmark runs it:
    # every gradient in full, every row of gradX
    print("[case] backward large T=16384 D=7168", file=sys.stderr, flush=True)
    bi = synth.backward_inputs(16384, 4, 7168, seed=15)
    rep = compare(gpu_backward(bi), run_oracle(bi), bi)
    assert rep["grad_x"]["n"] == 16384 * 4 * 7168


SINKHORN_CASES = [
    # (name, T, n, D, iterations, gamma, grad_x_post, seed)
    ("sk_T64_D256_20it", 64, 4, 256, 20, False, False, 41),
    ("sk_T130_D512_3it_gamma_post", 130, 4, 512, 3, True, True, 42),
    ("sk_T1_D8_1it", 1, 4, 8, 1, False, False, 43),
    ("sk_n8_T17_D64_2it", 17, 8, 64, 2, True, False, 44),
    ("sk_n8_T70_D256_20it", 70, 8, 256, 20, False, True, 45),
    ("sk_T200_D7168_20it", 200, 4, 7168, 20, False, False, 46),
    ("sk_n6_T1_D8_1it", 1, 6, 8, 1, False, False, 77),
    ("sk_n6_T17_D64_2it_gamma", 17, 6, 64, 2, True, False, 78),
    ("sk_n6_T70_D256_20it_post", 70, 6, 256, 20, False, True, 79),
    ("sk_Dmax_T30_D16384_20it_gamma", 30, 4, 16384, 20, True, False, 95),
]


@pytest.mark.parametrize("name,T,n,D,it,gamma,post,seed", SINKHORN_CASES, ids=[c[0] for c in SINKHORN_CASES])
def test_sinkhorn_backward_parity(name, T, n, D, it, gamma, post, seed):
    print(f"[case] sinkhorn backward {name} T={T} n={n} D={D} it={it}", file=sys.stderr, flush=True)
    bi = sinkhorn_inputs(T, n, D, it, gamma=gamma, post=post, seed=seed)
    compare(gpu_backward(bi), run_oracle(bi), bi)


def test_sinkhorn_backward_f16():
    print("[case] sinkhorn backward f16 T=130 n=4 D=512 it=3 gamma post", file=sys.stderr, flush=True)
    bi = sinkhorn_inputs(130, 4, 512, 3, gamma=True, post=True, seed=48, f16=True)
    compare(gpu_backward(bi), run_oracle(bi), bi)


def test_backward_large_workload_shape_f16():
    # the large prefill shape with fp16 x and gradients: every gradient, every row
    print("[case] backward large f16 T=16384 D=7168", file=sys.stderr, flush=True)
    bi = synth.backward_inputs(16384, 4, 7168, seed=16, x_f16=True)
    rep = compare(gpu_backward(bi), run_oracle(bi), bi)
    assert rep["grad_x"]["n"] == 16384 * 4 * 7168


def test_sinkhorn_backward_large_workload_shape():
    # the large prefill shape with its 20 Sinkhorn iterations: the training step's backward
    print("[case] sinkhorn backward large T=16384 D=7168 it=20", file=sys.stderr, flush=True)
    bi = sinkhorn_inputs(16384, 4, 7168, 20, seed=47)
    rep = compare(gpu_backward(bi), run_oracle(bi), bi)
    assert rep["grad_x"]["n"] == 16384 * 4 * 7168
