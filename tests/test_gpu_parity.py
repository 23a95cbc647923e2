"""GPU parity: the HIP library (through the C-ABI) against the fp64 oracle.

Acceptance rule: see gpu_helpers (fp32 outputs |d| <= 1e-6 + 2e-4 |ref|; hIn within
1 bf16 ulp, with the cancellation bound). Inputs are seeded and synthetic (synth).
"""
import json
import os
import sys

import numpy as np
import pytest

import synth
from gpu_helpers import compare, gpu_forward, run_oracle, summary, to_dev, to_host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_shapes.json")


def _log(name, rep):
    print(f"[parity] {name}: {summary(rep)}", file=sys.stderr, flush=True)


def _check(inp, name, **kw):
    print(f"[case] {name} T={inp.wl.T} n={inp.wl.n} D={inp.wl.D} alpha={inp.wl.n_alpha} "
          f"gamma={inp.gamma is not None} pre_mix={inp.pre_mix is not None}",
          file=sys.stderr, flush=True)
    g = gpu_forward(inp, **kw)
    rep = compare(g, run_oracle(inp), inp)
    _log(name, rep)
    return g


SMALL = [
    ("tiny_workload", lambda: synth.generate(synth.WORKLOADS["tiny"])),
    ("ragged_D7168_bwd", lambda: synth.custom(200, 4, 7168, need_backward=True, seed=21)),
    ("gamma_D4096", lambda: synth.custom(130, 4, 4096, gamma=True, seed=22)),
    ("n8_alpha2_premix", lambda: synth.custom(100, 8, 2048, n_alpha=2, pre_mix=True, seed=23)),
    ("n8_alpha3_bwd", lambda: synth.custom(70, 8, 256, need_backward=True, seed=24)),
    ("n4_alpha2", lambda: synth.custom(50, 4, 512, n_alpha=2, need_backward=True, seed=25)),
    ("n4_alpha3_premix_gamma", lambda: synth.custom(90, 4, 1024, gamma=True, pre_mix=True, seed=26)),
    ("D8_T10", lambda: synth.custom(10, 4, 8, need_backward=True, seed=27)),
    ("D40_partial_chunk", lambda: synth.custom(33, 4, 40, need_backward=True, seed=28)),
    ("D2056_tail", lambda: synth.custom(65, 4, 2056, gamma=True, seed=29)),
    ("n8_D24_partial", lambda: synth.custom(17, 8, 24, n_alpha=2, pre_mix=True, seed=30)),
    # the largest D for each n and alpha length: n = 8 with alpha[3] stops at 8192
    ("n8_alpha3_Dmax8192", lambda: synth.custom(20, 8, 8192, need_backward=True, seed=31)),
    ("n8_alpha2_Dmax16384", lambda: synth.custom(9, 8, 16384, n_alpha=2, seed=32)),
    ("n4_Dmax16384_T130_gamma", lambda: synth.custom(130, 4, 16384, gamma=True, need_backward=True, seed=33)),
    ("T1", lambda: synth.custom(1, 4, 7168, seed=31)),
    ("T2", lambda: synth.custom(2, 4, 4096, seed=32)),
    ("T7", lambda: synth.custom(7, 4, 5120, seed=33)),
    ("T63", lambda: synth.custom(63, 4, 5120, seed=34)),
    ("T513", lambda: synth.custom(513, 4, 4096, seed=35)),
    ("iters1", lambda: synth.custom(64, 4, 256, need_backward=True, num_iters=1, seed=36)),
    ("iters3", lambda: synth.custom(64, 4, 256, need_backward=True, num_iters=3, seed=37)),
    # n = 6 (the third stream count the aclnnMhcPreV2 guide allows): 36-entry Sinkhorn
    # matrices, 12-step slices, padded records
    ("n6_alpha3_bwd", lambda: synth.custom(130, 6, 1024, need_backward=True, seed=60)),
    ("n6_alpha3_D7168_gamma", lambda: synth.custom(70, 6, 7168, gamma=True, need_backward=True, seed=61)),
    ("n6_alpha2_premix_D520", lambda: synth.custom(65, 6, 520, n_alpha=2, pre_mix=True, need_backward=True, seed=62)),
    ("n6_alpha3_premix_D24_T9", lambda: synth.custom(9, 6, 24, pre_mix=True, need_backward=True, seed=63)),
    ("n6_D16384_T3", lambda: synth.custom(3, 6, 16384, need_backward=True, seed=64)),
    # binary16 x and hIn: fp16 matrix-core products against weights split into three
    # scaled fp16 terms
    ("f16_n4_alpha3_bwd", lambda: synth.custom(130, 4, 1024, need_backward=True, x_f16=True, seed=80)),
    ("f16_n4_D7168_gamma", lambda: synth.custom(70, 4, 7168, gamma=True, need_backward=True, x_f16=True, seed=81)),
    ("f16_n8_alpha2_premix_D520", lambda: synth.custom(65, 8, 520, n_alpha=2, pre_mix=True, need_backward=True,
                                                       x_f16=True, seed=82)),
    ("f16_n6_D40_T9", lambda: synth.custom(9, 6, 40, need_backward=True, x_f16=True, seed=83)),
    ("f16_n4_T1024_D4096_gamma", lambda: synth.custom(1024, 4, 4096, gamma=True, x_f16=True, seed=84)),
]


@pytest.mark.parametrize("name,make", SMALL, ids=[s[0] for s in SMALL])
def test_parity_small(name, make):
    _check(make(), name)


def _page_cases():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("case", _page_cases(), ids=lambda c: c["name"])
def test_parity_page_example_shapes(case):
    inp = synth.custom(case["T"], case["n"], case["D"], gamma=case.get("gamma", False),
                       need_backward=case.get("need_backward", False), seed=40)
    if case.get("all_ones"):
        one = synth.f32_to_bf16_bits(np.ones(1, np.float32))[0]
        inp.x[...] = one
        for a in (inp.phi, inp.alpha, inp.bias, inp.gamma):
            a[...] = 1.0
    g = _check(inp, case["name"])
    if case.get("all_ones"):
        # closed form of the all-ones example: hIn = 4 (1 + eps) -> bf16 4.0; hPost = 2
        assert np.all(g["h_in"] == 0x4080)
        assert np.allclose(g["h_post"], 2.0, rtol=0, atol=1e-6)


def test_bsnd_layout_matches_tnd():
    import torch

    import mhc_hyper_connection_amd as mhc
    from gpu_helpers import device, to_dev, to_host
    inp = synth.custom(24, 4, 256, gamma=True, seed=41)
    dev = device()
    x = to_dev(inp.x, dev)
    args = [to_dev(a, dev) for a in (inp.phi, inp.alpha, inp.bias, inp.gamma)]
    h1, p1, r1, _ = mhc.mhc_pre(x, *args)
    h2, p2, r2, e2 = mhc.mhc_pre(x.reshape(2, 12, 4, 256), *args, need_backward=True)
    torch.cuda.synchronize()
    assert h2.shape == (2, 12, 256) and p2.shape == (2, 12, 4) and r2.shape == (2, 12, 4, 4)
    assert e2["sum_out"].shape == (40, 2, 12, 4) and e2["inv_rms"].shape == (2, 12)
    assert np.array_equal(to_host(h1), to_host(h2).reshape(24, 256))
    assert np.array_equal(to_host(p1), to_host(p2).reshape(24, 4))
    assert np.array_equal(to_host(r1), to_host(r2).reshape(24, 4, 4))


def test_deterministic_and_flag_invariant():
    inp = synth.custom(520, 4, 7168, need_backward=True, seed=42)
    runs = gpu_forward(inp, repeat=3)
    for k in runs[0]:
        for r in runs[1:]:
            assert np.array_equal(runs[0][k].view(np.uint8), r[k].view(np.uint8)), k
    lean = gpu_forward(inp, need_backward=False, intermediates=False)
    for k in ("h_in", "h_post", "h_res"):
        assert np.array_equal(lean[k].view(np.uint8), runs[0][k].view(np.uint8)), k
    packed = gpu_forward(inp, packed=True)
    for k in runs[0]:
        assert np.array_equal(packed[k].view(np.uint8), runs[0][k].view(np.uint8)), k


def test_timed_forward_with_unrecorded_boundaries():
    # mhc_pre_forward_timed skips NULL event entries: the outputs equal the untimed call's
    # bit for bit, and the recorded pairs give positive durations
    import mhc_hyper_connection_amd as mhc
    import torch
    print("[case] timed forward with NULL events", file=sys.stderr, flush=True)
    inp = synth.custom(300, 4, 1024, need_backward=True, seed=96)
    plain = gpu_forward(inp)
    dev = torch.device("cuda", 0)
    wl = inp.wl
    r = mhc.PreForward(wl.T, wl.n, wl.D, wl.n_alpha, need_backward=True, device=dev)
    x, phi, alpha, bias = (to_dev(a, dev) for a in (inp.x, inp.phi, inp.alpha, inp.bias))
    ev = [torch.cuda.Event(enable_timing=True) if i in (0, 2, 4) else None for i in range(mhc.FORWARD_EVENTS)]
    for e in ev:
        if e is not None:
            e.record()
    torch.cuda.synchronize(dev)
    out = r(x, phi, alpha, bias, events=ev)
    torch.cuda.synchronize(dev)
    assert ev[0].elapsed_time(ev[2]) > 0 and ev[2].elapsed_time(ev[4]) > 0
    for k, v in out.items():
        assert np.array_equal(to_host(v).view(np.uint8), plain[k].view(np.uint8)), k
