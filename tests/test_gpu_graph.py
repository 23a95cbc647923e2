"""The forward captured into a HIP graph (torch.cuda.CUDAGraph on torch's current stream):
no path records a memset or a host synchronisation, so each can be captured (the
one-launch path in the first two cases, whose kernel clears its barrier counters in the
workspace at its end; the streaming path at 4096 tokens, with packed and unpacked weights;
the classic path, forced by MHC_FORWARD_PATH=classic; the single-read path forced by
MHC_FORWARD_PATH=fused in the last case: its kernel
and the epilogue keep the call counter and the per-XCD arrival counters in the workspace,
which each replay advances and clears as an eager call does). Every replay, with eager work of
the program between replays, must equal the eager call bit for bit (the forward is
deterministic), and the eager call meets the oracle."""
import sys

import numpy as np
import pytest

import synth
from gpu_helpers import compare, device, run_oracle, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,D,packed,path", [(64, 7168, True, 2), (64, 7168, False, 2), (64, 7168, True, 0),
                                              (4096, 1024, True, 3), (4096, 1024, False, 3), (4096, 1024, True, 0),
                                              (1500, 2048, False, 1)])
def test_graph_replays_match_eager(T, D, packed, path, monkeypatch):
    import mhc_hyper_connection_amd as mhc
    import torch
    monkeypatch.delenv("MHC_FORWARD_PATH", raising=False)
    if path == 1:
        monkeypatch.setenv("MHC_FORWARD_PATH", "fused")
    elif path == 0:
        monkeypatch.setenv("MHC_FORWARD_PATH", "classic")
    print(f"[case] graph T={T} D={D} packed={packed} path={path}", file=sys.stderr, flush=True)
    dev = device()
    inp = synth.custom(T, 4, D, need_backward=True, seed=95)
    wl = inp.wl
    r = mhc.PreForward(wl.T, wl.n, wl.D, wl.n_alpha, num_iters=wl.num_iters, need_backward=True, device=dev)
    assert r.path() == path
    x, phi, alpha, bias = (to_dev(a, dev) for a in (inp.x, inp.phi, inp.alpha, inp.bias))
    pk = r.prepack(phi) if packed else None
    eager = r(x, None if packed else phi, alpha, bias, phi_packed=pk)
    torch.cuda.synchronize(dev)
    want = {k: to_host(v) for k, v in eager.items()}
    compare(want, run_oracle(inp), inp)

    out = r.alloc_outputs()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):      # warm the captured call once on the capture stream
        r(x, None if packed else phi, alpha, bias, phi_packed=pk, out=out)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r(x, None if packed else phi, alpha, bias, phi_packed=pk, out=out)
    torch.cuda.synchronize(dev)
    for rep in range(4):
        for v in out.values():   # clobber the outputs between replays with eager work
            v.view(torch.int16).fill_(0x7FC0) if v.dtype == torch.bfloat16 else v.fill_(float("nan"))
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        for k, v in out.items():
            assert np.array_equal(to_host(v).view(np.uint8), want[k].view(np.uint8)), f"replay {rep}: {k}"
