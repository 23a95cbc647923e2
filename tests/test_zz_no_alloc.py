"""mhc_pre_forward_noalloc (the forward with the library's per-GPU scratch array as its
workspace, for callers that cannot allocate) against mhc_pre_forward, both through the
C-ABI: two calls in a row, the second with fewer tokens, each bit for bit equal to the
regular entry point on the same inputs and within the oracle's acceptance rule. (Its host
checks, among them the refusal of a workspace beyond the array, run in test_boundary.)"""
import sys

import numpy as np
import pytest

import synth
from gpu_helpers import compare, device, gpu_forward, run_oracle, summary

pytestmark = pytest.mark.gpu


def _run(inp, noalloc, packed=False):
    import mhc_hyper_connection_amd as mhc
    wl = inp.wl
    r = mhc.PreForward(wl.T, wl.n, wl.D, wl.n_alpha, num_iters=wl.num_iters, norm_eps=wl.norm_eps,
                       hc_eps=wl.hc_eps, need_backward=wl.need_backward, device=device())

    class _Caller:   # gpu_forward's runner protocol, routed to the chosen entry point
        def __getattr__(self, name):
            return getattr(r, name)

        def __call__(self, *args, **kw):
            return r(*args, noalloc=noalloc, **kw)

    return gpu_forward(inp, runner=_Caller(), intermediates=True, packed=packed)


@pytest.mark.parametrize("first,second", [((3000, 2048, True, 71), (500, 2048, True, 72)),
                                          ((2100, 7168, False, 73), (64, 7168, False, 74))])
def test_noalloc_matches_forward_on_two_calls(first, second):
    for (T, D, gamma, seed) in (first, second):
        print(f"[case] noalloc T={T} D={D} gamma={gamma}", file=sys.stderr, flush=True)
        inp = synth.custom(T, 4, D, gamma=gamma, need_backward=True, seed=seed)
        got = _run(inp, True)
        want = _run(inp, False)
        for k in want:
            assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), (T, D, k)
        rep = compare(got, run_oracle(inp), inp)
        print(f"[noalloc] T={T} D={D}: {summary(rep)}", file=sys.stderr, flush=True)


def test_noalloc_one_launch_grid_changes():
    # the one-launch kernel through the shared array with its grid changing from call to
    # call: 224 workgroups (weights split in the kernel), 112 (packed weights passed in:
    # two d-blocks a workgroup), 224 again; the tags in the array's flag words stay in
    # step, and each call equals the regular entry point called the same way
    inp = synth.custom(64, 4, 7168, gamma=True, need_backward=True, seed=75)
    orc = run_oracle(inp)
    for packed in (False, True, False):
        print(f"[case] noalloc one-launch T=64 D=7168 packed={packed}", file=sys.stderr, flush=True)
        got = _run(inp, True, packed)
        want = _run(inp, False, packed)
        for k in want:
            assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), (packed, k)
        compare(got, orc, inp)
