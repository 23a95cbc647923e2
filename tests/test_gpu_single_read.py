"""The single-read forward kernel (n = 4, alpha[3], no pre_mix, 32 to 224 d-blocks of 32
positions, T >= 8192, bf16 or fp16 x; one group of 32 workgroups per XCD): path selection on the device,
and parity with the fp64 oracle under the acceptance rule of gpu_helpers, at the sizes
where it is chosen by itself (the large workload test covers that at full size) and,
forced by MHC_FORWARD_PATH=fused, at small and ragged sizes: partial last tiles of 16
tokens, fewer tiles than groups, groups with unequal numbers of tiles, members with
unequal numbers of d-blocks (compute waves with a block or none), a partial last d-block,
gamma, and the output set without intermediates. The wait time-out is driven from the
host (a test switch makes every exchange wait accept no tag, so each gives up at its
poll limit; all kernels exit normally) and must show through mhc_pre_wait_status."""
import sys

import numpy as np
import pytest

import synth
from gpu_helpers import compare, device, gpu_forward, run_oracle, summary

pytestmark = pytest.mark.gpu


def _runner(wl, nb):
    import mhc_hyper_connection_amd as mhc
    return mhc.PreForward(wl.T, wl.n, wl.D, wl.n_alpha, num_iters=wl.num_iters, norm_eps=wl.norm_eps,
                          hc_eps=wl.hc_eps, need_backward=nb, device=device(), x_f16=wl.x_f16)


def _timeout_flag(runner):
    # the library's wait time-out flag, read and cleared through the C-ABI
    return runner.wait_status()


@pytest.mark.parametrize("T,D,pre_mix,n,n_alpha,want", [
    (16384, 7168, False, 4, 3, 1), (8192, 4096, False, 4, 3, 1), (8192, 1024, False, 4, 3, 1),
    (64, 7168, False, 4, 3, 2), (8191, 7168, False, 4, 3, 3), (8192, 7168, False, 4, 3, 1),
    (4096, 4096, False, 4, 3, 3), (16384, 7168, True, 4, 3, 0), (8192, 8192, False, 4, 3, 3),
    (8192, 992, False, 4, 3, 3), (8192, 1016, False, 4, 3, 1), (8192, 2048, False, 8, 3, 0),
    (8192, 2048, False, 4, 2, 3), (32768, 2048, True, 8, 2, 0), (8192, 2048, False, 6, 2, 3),
    (8192, 1000, False, 4, 3, 1), (8192, 1000, True, 4, 3, 0),
    (8192, 2048, False, 6, 3, 0)])
@pytest.mark.parametrize("f16", [False, True])
def test_path_selection(T, D, pre_mix, n, n_alpha, want, f16, monkeypatch):
    # the same choice for bf16 and fp16 x
    import mhc_hyper_connection_amd as mhc
    monkeypatch.delenv("MHC_FORWARD_PATH", raising=False)
    device()
    p = mhc.make_params(T, n, D, n_alpha, x_f16=f16)
    assert mhc.forward_path(p, pre_mix) == want


CASES = [
    # (name, T, D, gamma, need_backward, intermediates, fp16 x, seed)
    ("T1_D1024", 1, 1024, False, True, True, False, 51),
    ("T17_D1024_bwd", 17, 1024, False, True, True, False, 52),
    ("T100_D1032_gamma", 100, 1032, True, False, True, False, 53),
    ("T129_D2048_no_intermediates", 129, 2048, False, False, False, False, 54),
    ("T300_D4096_gamma_bwd", 300, 4096, True, True, True, False, 55),
    ("T1000_D7168_bwd", 1000, 7168, False, True, True, False, 56),
    ("T2100_D3000_gamma", 2100, 3000, True, False, True, False, 57),
    ("f16_T17_D1024_bwd", 17, 1024, False, True, True, True, 151),
    ("f16_T300_D4096_gamma_bwd", 300, 4096, True, True, True, True, 152),
    ("f16_T1000_D7168_bwd", 1000, 7168, False, True, True, True, 153),
    ("f16_T2100_D3000_gamma", 2100, 3000, True, False, True, True, 154),
]


@pytest.mark.parametrize("name,T,D,gamma,nb,inter,f16,seed", CASES, ids=[c[0] for c in CASES])
def test_forced_single_read_parity(name, T, D, gamma, nb, inter, f16, seed, monkeypatch):
    monkeypatch.setenv("MHC_FORWARD_PATH", "fused")
    print(f"[case] single-read {name} T={T} D={D} gamma={gamma} need_backward={nb} f16={f16}", file=sys.stderr, flush=True)
    inp = synth.custom(T, 4, D, gamma=gamma, need_backward=nb, seed=seed, x_f16=f16)
    r = _runner(inp.wl, nb)
    assert r.path() == 1
    gpu = gpu_forward(inp, runner=r, intermediates=inter)
    rep = compare(gpu, run_oracle(inp), inp)
    print(f"[single-read] {name}: {summary(rep)}", file=sys.stderr, flush=True)
    assert _timeout_flag(r) == 0


def test_single_read_reproducible_and_repeated_calls(monkeypatch):
    # several calls through one workspace (the call counter advances each time): bitwise
    # equal results, and no wait ever timed out
    monkeypatch.setenv("MHC_FORWARD_PATH", "fused")
    print("[case] single-read repeated T=3000 D=2048", file=sys.stderr, flush=True)
    inp = synth.custom(3000, 4, 2048, gamma=True, need_backward=True, seed=58)
    r = _runner(inp.wl, True)
    runs = gpu_forward(inp, runner=r, repeat=3)
    for k in runs[0]:
        for other in runs[1:]:
            assert np.array_equal(runs[0][k].view(np.uint8), other[k].view(np.uint8)), k
    compare(runs[-1], run_oracle(inp), inp)
    assert _timeout_flag(r) == 0


def test_classic_path_still_served(monkeypatch):
    # the classic path on a shape the single-read kernel would take
    monkeypatch.setenv("MHC_FORWARD_PATH", "classic")
    print("[case] classic forced T=8192 D=2048", file=sys.stderr, flush=True)
    inp = synth.custom(8192, 4, 2048, need_backward=True, seed=59)
    r = _runner(inp.wl, True)
    assert r.path() == 0
    compare(gpu_forward(inp, runner=r), run_oracle(inp), inp)


@pytest.mark.parametrize("f16", [False, True])
def test_single_read_with_prepacked_weights(f16, monkeypatch):
    # phi packed once by mhc_pre_prepack and passed in (the kernel then copies the packed
    # slices instead of packing phi itself): same acceptance, and the same bits as packing
    # inside the kernel
    monkeypatch.setenv("MHC_FORWARD_PATH", "fused")
    print(f"[case] single-read prepacked T=500 D=2048 gamma f16={f16}", file=sys.stderr, flush=True)
    inp = synth.custom(500, 4, 2048, gamma=True, need_backward=True, seed=60, x_f16=f16)
    r = _runner(inp.wl, True)
    g_packed = gpu_forward(inp, runner=r, packed=True)
    compare(g_packed, run_oracle(inp), inp)
    g_inline = gpu_forward(inp, runner=r, packed=False)
    for k in g_packed:
        assert np.array_equal(g_packed[k].view(np.uint8), g_inline[k].view(np.uint8)), k
    assert _timeout_flag(r) == 0


def test_wait_time_out_is_reported(monkeypatch):
    # every exchange wait made to give up (the kernel then never sees the tag it waits for,
    # and stops polling at its limit, about 0.3 s): the call still returns, hIn holds NaN
    # (hPre, which the epilogue computes from the stored records, stays finite), and
    # mhc_pre_wait_status reports the time-out once, then clears it
    import mhc_hyper_connection_amd as mhc
    monkeypatch.setenv("MHC_FORWARD_PATH", "fused")
    monkeypatch.setenv("MHC_TEST_EXCHANGE_NEVER_READY", "1")
    print("[case] single-read forced wait time-out T=1000 D=2048", file=sys.stderr, flush=True)
    inp = synth.custom(1000, 4, 2048, need_backward=True, seed=61)
    r = _runner(inp.wl, True)
    assert r.path() == 1
    g = gpu_forward(inp, runner=r)
    assert r.wait_status() == 1
    assert r.wait_status() == 0
    hin = g["h_in"].view(np.int16)
    assert np.all((hin & 0x7F80) == 0x7F80) and np.all((hin & 0x7F) != 0)   # bf16 NaN everywhere
    assert np.all(np.isfinite(g["h_pre"]))
    monkeypatch.delenv("MHC_TEST_EXCHANGE_NEVER_READY")
    compare(gpu_forward(inp, runner=r), run_oracle(inp), inp)
    assert r.wait_status() == 0
