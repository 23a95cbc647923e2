"""The five measured workloads at their full sizes, in the launch configuration the
benchmark times (one mhc_pre_forward call with unpacked weights).

Every token of every workload is compared element by element against the oracle: the
small ones in one oracle call, the large prefill (with all 40 Sinkhorn planes), the wide
pre_mix workload and the fp16 large prefill in oracle calls of 1024 tokens that bound
host memory. Properties that hold at any size are checked on every token as well: gate
ranges, Sinkhorn column sums after the last (column) step, and the step relation
normOut[k] = normOut[k-1] / sumOut[k] between the emitted planes.
"""
import dataclasses
import sys

import numpy as np
import pytest

import synth
from gpu_helpers import compare, gpu_forward, run_oracle, summary

pytestmark = pytest.mark.gpu

_CACHE = {}


def _inputs(name):
    if name not in _CACHE:
        _CACHE.clear()
        if name.endswith("_f16"):   # the same workload with x and hIn in binary16
            wl = dataclasses.replace(synth.WORKLOADS[name[:-4]], name=name, x_f16=True)
        else:
            wl = synth.WORKLOADS[name]
        _CACHE[name] = synth.generate(wl)
    return _CACHE[name]


def _merge(total, rep):
    """Accumulates per-chunk reports: counts add up, maxima are kept."""
    for k, v in rep.items():
        if k not in total:
            total[k] = {f: val for f, val in v.items() if f != "worst"}
            continue
        t = total[k]
        for f, val in v.items():
            if f in ("n", "fail", "ulp_gt_1_but_cancel_ok", "exact"):
                t[f] += val
            elif f in ("max_abs", "max_ratio", "max_ulp"):
                t[f] = max(t[f], val)
    return total


def compare_chunked(g, inp, chunk=1024):
    """Every token against the oracle, `chunk` tokens per oracle call (compare raises on
    the first chunk with a failure)."""
    total = {}
    for t0 in range(0, inp.wl.T, chunk):
        tok = np.arange(t0, min(inp.wl.T, t0 + chunk))
        _merge(total, compare(g, run_oracle(inp, tokens=tok), inp, tokens=tok))
    return total


def _log(name, rep):
    print(f"[workload] {name}: {summary(rep)}", file=sys.stderr, flush=True)


@pytest.mark.parametrize("name", ["tiny", "mid_prefill", "decode"])
def test_workload_full_compare(name):
    inp = _inputs(name)
    print(f"[case] {name} full compare", file=sys.stderr, flush=True)
    g = gpu_forward(inp, intermediates=True)
    rep = compare(g, run_oracle(inp), inp)
    _log(name, rep)


@pytest.mark.parametrize("name", ["large_prefill_bwd", "wide_premix", "large_prefill_bwd_f16"])
def test_workload_every_token_and_properties(name):
    inp = _inputs(name)
    wl = inp.wl
    print(f"[case] {name} every-token compare", file=sys.stderr, flush=True)
    g = gpu_forward(inp, intermediates=True)
    rep = compare_chunked(g, inp)
    assert rep["h_in"]["n"] == wl.T * wl.D, rep["h_in"]
    _log(name, rep)

    eps = wl.hc_eps
    h_pre, h_post = g["h_pre"].astype(np.float64), g["h_post"].astype(np.float64)
    assert np.all((h_pre > eps) & (h_pre < 1 + eps + 1e-6))
    if wl.n_alpha == 3:
        assert np.all((h_post > 0) & (h_post < 2))
        cols = g["h_res"].astype(np.float64).sum(axis=1)            # [T, n]
        assert np.all(np.abs(cols - 1.0) <= 1e-5), float(np.abs(cols - 1).max())
        no, so = g["norm_out"].astype(np.float64), g["sum_out"].astype(np.float64)
        for k in range(1, no.shape[0]):
            axis_b = (slice(None), None, slice(None)) if k % 2 else (slice(None), slice(None), None)
            pred = no[k - 1] / so[k][axis_b]
            assert np.all(np.abs(no[k] - pred) <= 1e-6 + 1e-5 * np.abs(pred)), k
        assert np.array_equal(g["h_res"], g["norm_out"][-1])
    else:
        assert np.all((h_post > eps) & (h_post < 2 + eps + 1e-6))
        assert np.all(g["h_res"] == 0.0)
