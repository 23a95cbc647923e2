"""GPU parity of the two standalone stages through the C-ABI -- mhc_pre_inv_rms and
mhc_pre_sinkhorn (from given mixes and invRms) -- against the fp64 oracle's
oracle.inv_rms / oracle.pre_sinkhorn on seeded inputs (synth.stage_inputs).

Acceptance: the rule of gpu_helpers for every f32 output and for hIn; invRms, whose
squares and sums run in fp64 on both sides, must also be the correctly rounded f32 of
the oracle's value within one f32 rounding (relative error <= 2^-23)."""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import _fp32_check, _hin_check, device, summary, to_dev, to_host
from synth import bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def gpu_inv_rms(x_bits):
    import mhc_hyper_connection_amd as mhc
    import torch
    dev = device()
    out = mhc.mhc_pre_inv_rms(to_dev(x_bits, dev))
    torch.cuda.synchronize(dev)
    return to_host(out)


INV_CASES = [("T1_n4_D8", 1, 4, 8), ("T7_n4_D40", 7, 4, 40), ("T130_n8_D24", 130, 8, 24),
             ("T65_n8_D7168", 65, 8, 7168), ("T300_n4_D7168", 300, 4, 7168), ("T5_n4_D16384", 5, 4, 16384),
             ("T33_n6_D520", 33, 6, 520)]


@pytest.mark.parametrize("name,T,n,D", INV_CASES, ids=[c[0] for c in INV_CASES])
def test_inv_rms_parity(name, T, n, D):
    print(f"[case] inv_rms {name}", file=sys.stderr, flush=True)
    si = synth.stage_inputs(T, n, D, seed=40 + T)
    g = gpu_inv_rms(si.x)
    r = oracle.inv_rms(si.x)
    rep = {}
    _fp32_check("inv_rms", g, r, rep)
    rel = float(np.max(np.abs(g.astype(np.float64) - r) / r))
    print(f"[parity-inv-rms] {summary(rep)} max_rel={rel:.2e}", file=sys.stderr, flush=True)
    assert rep["inv_rms"]["fail"] == 0
    assert rel <= 2.0 ** -23


def test_inv_rms_large_every_token():
    # a long-prefill slice at the widest hidden size: 8192 tokens of n = 4, D = 7168,
    # every token against the oracle
    T, n, D = 8192, 4, 7168
    print(f"[case] inv_rms T{T}_n{n}_D{D} every token", file=sys.stderr, flush=True)
    si = synth.stage_inputs(T, n, D, seed=47)
    g = gpu_inv_rms(si.x)
    r = oracle.inv_rms(si.x)
    rel = float(np.max(np.abs(g.astype(np.float64) - r) / r))
    print(f"[parity-inv-rms] every token max_rel={rel:.2e}", file=sys.stderr, flush=True)
    assert rel <= 2.0 ** -23


def gpu_sinkhorn(si, num_iters, need_backward):
    import mhc_hyper_connection_amd as mhc
    import torch
    dev = device()
    d = lambda a: None if a is None else to_dev(a, dev)
    h_in, h_pre, h_post, h_res, ex = mhc.mhc_pre_sinkhorn(
        d(si.x), d(si.h_mix), d(si.inv_rms), d(si.alpha), d(si.bias), d(si.pre_mix),
        num_iters=num_iters, need_backward=need_backward)
    torch.cuda.synchronize(dev)
    out = {"h_in": to_host(h_in), "h_pre": to_host(h_pre), "h_post": to_host(h_post), "h_res": to_host(h_res)}
    out.update({k: to_host(v) for k, v in ex.items()})
    return out


SK_CASES = [  # name, T, n, D, n_alpha, pre_mix, need_backward, num_iters
    ("T1_n4_D8", 1, 4, 8, 3, False, True, 20),
    ("T9_n4_D40_tail", 9, 4, 40, 3, False, True, 20),
    ("T33_n8_D24", 33, 8, 24, 3, False, True, 20),
    ("T17_n4_D64_alpha2", 17, 4, 64, 2, False, False, 20),
    ("T20_n8_D32_alpha2_premix", 20, 8, 32, 2, True, False, 20),
    ("T70_n4_D520_premix", 70, 4, 520, 3, True, True, 20),
    ("T300_n4_D7168", 300, 4, 7168, 3, False, True, 20),
    ("T64_n8_D4096_it3", 64, 8, 4096, 3, False, True, 3),
    ("T13_n6_D48", 13, 6, 48, 3, False, True, 20),
    ("T21_n6_D64_alpha2_premix", 21, 6, 64, 2, True, False, 20),
]


@pytest.mark.parametrize("name,T,n,D,na,pm,nb,it", SK_CASES, ids=[c[0] for c in SK_CASES])
def test_sinkhorn_parity(name, T, n, D, na, pm, nb, it):
    print(f"[case] sinkhorn {name}", file=sys.stderr, flush=True)
    si = synth.stage_inputs(T, n, D, n_alpha=na, pre_mix=pm, seed=50 + T)
    g = gpu_sinkhorn(si, it, nb)
    r = oracle.pre_sinkhorn(si.x, si.h_mix, si.inv_rms, si.alpha, si.bias, si.pre_mix, num_iters=it)
    rep = {}
    _fp32_check("h_pre", g["h_pre"], r.h_pre, rep)
    _fp32_check("h_post", g["h_post"], r.h_post, rep)
    if na == 3:
        _fp32_check("h_res", g["h_res"], r.h_res, rep)
    else:
        rep["h_res_zero"] = dict(n=int(g["h_res"].size), fail=int((g["h_res"] != 0).sum()))
    if nb and na == 3:
        _fp32_check("sum_out", g["sum_out"], r.sum_out, rep)
        _fp32_check("norm_out", g["norm_out"], r.norm_out, rep)
    x = bf16_bits_to_f32(si.x).astype(np.float64)
    w = si.pre_mix.astype(np.float64) if si.pre_mix is not None else r.h_pre
    _hin_check(g["h_in"], r.h_in, r.h_in_bf16, np.einsum("ti,tid->td", np.abs(w), np.abs(x)), rep)
    print(f"[parity-sinkhorn] {summary(rep)}", file=sys.stderr, flush=True)
    failing = {k: v for k, v in rep.items() if v.get("fail", 0)}
    assert not failing, f"parity failures: {failing}"


def test_stages_empty_input():
    import mhc_hyper_connection_amd as mhc
    si = synth.stage_inputs(0, 4, 64)
    assert mhc.mhc_pre_inv_rms(to_dev(si.x, device())).shape == (0,)
    d = lambda a: to_dev(a, device())
    h_in, h_pre, h_post, h_res, ex = mhc.mhc_pre_sinkhorn(d(si.x), d(si.h_mix), d(si.inv_rms), d(si.alpha),
                                                          d(si.bias), need_backward=True)
    assert h_in.shape == (0, 64) and ex["norm_out"].shape == (40, 0, 4, 4)


@pytest.mark.parametrize("T,n,D,na,pm", [(33, 4, 520, 3, False), (20, 8, 64, 2, True), (11, 6, 48, 3, True)])
def test_stages_f16(T, n, D, na, pm):
    # binary16 x and hIn through both standalone stages
    import mhc_hyper_connection_amd as mhc
    import torch
    print(f"[case] stages f16 T={T} n={n} D={D} alpha={na} pre_mix={pm}", file=sys.stderr, flush=True)
    dev = device()
    si = synth.stage_inputs(T, n, D, n_alpha=na, pre_mix=pm, seed=90 + T, x_f16=True)
    x = to_dev(si.x, dev, True)
    g_inv = to_host(mhc.mhc_pre_inv_rms(x))
    r_inv = oracle.inv_rms(si.x, x_f16=True)
    assert float(np.max(np.abs(g_inv.astype(np.float64) - r_inv) / r_inv)) <= 2.0 ** -23
    d = lambda a: None if a is None else to_dev(a, dev)
    h_in, h_pre, h_post, h_res, ex = mhc.mhc_pre_sinkhorn(x, d(si.h_mix), d(si.inv_rms), d(si.alpha), d(si.bias),
                                                          d(si.pre_mix), need_backward=True)
    torch.cuda.synchronize(dev)
    assert h_in.dtype == torch.float16
    r = oracle.pre_sinkhorn(si.x, si.h_mix, si.inv_rms, si.alpha, si.bias, si.pre_mix, x_f16=True)
    rep = {}
    _fp32_check("h_pre", to_host(h_pre), r.h_pre, rep)
    _fp32_check("h_post", to_host(h_post), r.h_post, rep)
    if na == 3:
        _fp32_check("h_res", to_host(h_res), r.h_res, rep)
        _fp32_check("norm_out", to_host(ex["norm_out"]), r.norm_out, rep)
    xf = si.x.view(np.float16).astype(np.float64)
    w = si.pre_mix.astype(np.float64) if si.pre_mix is not None else r.h_pre
    _hin_check(to_host(h_in), r.h_in, r.h_in_bf16, np.einsum("ti,tid->td", np.abs(w), np.abs(xf)), rep, True)
    print(f"[parity-stages-f16] {summary(rep)}", file=sys.stderr, flush=True)
    failing = {k: v for k, v in rep.items() if v.get("fail", 0)}
    assert not failing, f"parity failures: {failing}"
