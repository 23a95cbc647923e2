"""The one-launch forward of a few tokens (n = 4, alpha[3], no pre_mix, T <= 64, bf16 or
fp16 x): path selection on the device, and parity with the fp64 oracle under the acceptance rule of
gpu_helpers over the sizes it serves: one token, tokens that fill 1 to 4 matrix-row waves
and ragged counts, fewer tokens than workgroups and more (a workgroup then takes several
tokens), a single d-block, a partial last d-block, the largest D (512 workgroups), gamma,
the output set without intermediates, packed and unpacked weights, repeated
calls through one workspace (each call's tag comes from flag words every call advances),
packed weights passed in (then two d-blocks a workgroup where there are still as many
workgroups as tokens: one token, an odd block count, a partial last block, 512 blocks),
the same inputs on the classic path, and a wait time-out driven from the host (a test
switch makes every poll accept no tag, so each gives up at its limit; every workgroup
still exits normally) that must leave NaN outputs and show through mhc_pre_wait_status."""
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


@pytest.mark.parametrize("T,D,pre_mix,n,n_alpha,want", [
    (1, 7168, False, 4, 3, 2), (64, 7168, False, 4, 3, 2), (65, 7168, False, 4, 3, 3),
    (64, 7168, True, 4, 3, 0), (64, 16384, False, 4, 3, 2), (8, 8, False, 4, 3, 2),
    (16, 1024, False, 4, 2, 3), (16, 1024, False, 8, 3, 0), (16, 1024, False, 6, 3, 0)])
@pytest.mark.parametrize("f16", [False, True])
def test_path_selection(T, D, pre_mix, n, n_alpha, want, f16, monkeypatch):
    import mhc_hyper_connection_amd as mhc
    monkeypatch.delenv("MHC_FORWARD_PATH", raising=False)
    device()
    p = mhc.make_params(T, n, D, n_alpha, x_f16=f16)
    assert mhc.forward_path(p, pre_mix) == want


def test_path_override(monkeypatch):
    import mhc_hyper_connection_amd as mhc
    device()
    p = mhc.make_params(64, 4, 7168, 3)
    monkeypatch.setenv("MHC_FORWARD_PATH", "classic")
    assert mhc.forward_path(p, False) == 0
    monkeypatch.setenv("MHC_FORWARD_PATH", "fused")
    assert mhc.forward_path(p, False) == 1


CASES = [
    # (name, T, D, gamma, need_backward, intermediates, fp16 x, seed)
    ("T1_D7168", 1, 7168, False, False, True, False, 151),
    ("T2_D1024_bwd", 2, 1024, False, True, True, False, 152),
    ("T16_D4096_gamma_bwd", 16, 4096, True, True, True, False, 153),
    ("T17_D7168_bwd", 17, 7168, False, True, True, False, 154),
    ("T33_D40_partial_block", 33, 40, False, True, True, False, 155),
    ("T48_D8_one_block", 48, 8, True, True, True, False, 156),
    ("T63_D5128_gamma", 63, 5128, True, False, True, False, 157),
    ("T64_D7168_bwd", 64, 7168, False, True, True, False, 158),
    ("T64_D1024_two_tokens_per_wg", 64, 1024, True, True, True, False, 159),
    ("T64_D16384", 64, 16384, False, True, True, False, 160),
    ("T40_D2048_no_intermediates", 40, 2048, False, False, False, False, 161),
    ("f16_T1_D7168", 1, 7168, False, False, True, True, 171),
    ("f16_T33_D40_partial_block", 33, 40, True, True, True, True, 172),
    ("f16_T64_D7168_gamma_bwd", 64, 7168, True, True, True, True, 173),
]


@pytest.mark.parametrize("name,T,D,gamma,nb,inter,f16,seed", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(name, T, D, gamma, nb, inter, f16, seed, monkeypatch):
    monkeypatch.delenv("MHC_FORWARD_PATH", raising=False)
    print(f"[case] one-launch {name} T={T} D={D} gamma={gamma} need_backward={nb} f16={f16}", file=sys.stderr, flush=True)
    inp = synth.custom(T, 4, D, gamma=gamma, need_backward=nb, seed=seed, x_f16=f16)
    r = _runner(inp.wl, nb)
    assert r.path() == 2
    gpu = gpu_forward(inp, runner=r, intermediates=inter)
    rep = compare(gpu, run_oracle(inp), inp)
    print(f"[one-launch] {name}: {summary(rep)}", file=sys.stderr, flush=True)
    assert r.wait_status() == 0


PACKED_CASES = [
    # (name, T, D, gamma, fp16 x, seed); packed weights passed in: two d-blocks a workgroup
    # wherever ceil(nblk / 2) >= T, else one
    ("T1_D7168_two_blocks", 1, 7168, False, False, 181),
    ("T4_D216_odd_block_count", 4, 216, True, False, 182),     # 7 blocks: the last workgroup has one
    ("T3_D168_partial_last", 3, 168, False, False, 183),
    ("T64_D7168_gamma", 64, 7168, True, False, 184),
    ("T64_D16384", 64, 16384, False, False, 185),
    ("T64_D3072_one_block", 64, 3072, True, False, 186),       # 96 blocks, 48 < 64 tokens: one each
    ("f16_T33_D7168_gamma", 33, 7168, True, True, 187),
]


@pytest.mark.parametrize("name,T,D,gamma,f16,seed", PACKED_CASES, ids=[c[0] for c in PACKED_CASES])
def test_decode_parity_packed(name, T, D, gamma, f16, seed, monkeypatch):
    monkeypatch.delenv("MHC_FORWARD_PATH", raising=False)
    print(f"[case] one-launch packed {name} T={T} D={D} gamma={gamma} f16={f16}", file=sys.stderr, flush=True)
    inp = synth.custom(T, 4, D, gamma=gamma, need_backward=True, seed=seed, x_f16=f16)
    r = _runner(inp.wl, True)
    assert r.path() == 2
    runs = gpu_forward(inp, runner=r, packed=True, repeat=2)
    for k in runs[0]:
        assert np.array_equal(runs[0][k].view(np.uint8), runs[1][k].view(np.uint8)), k
    rep = compare(runs[-1], run_oracle(inp), inp)
    print(f"[one-launch packed] {name}: {summary(rep)}", file=sys.stderr, flush=True)
    assert r.wait_status() == 0


@pytest.mark.parametrize("D", [7168, 3072])
def test_decode_repeated_calls_and_prepacked(D, monkeypatch):
    # several calls through one workspace: bitwise equal results, no wait timed out. Where
    # the packed weights passed in still leave one d-block a workgroup (D = 3072: 48 pairs
    # of blocks for 64 tokens) they give the same bits as packing inside the kernel; where
    # they take two (D = 7168) the fp32 sums group the other way and each meets the oracle.
    monkeypatch.delenv("MHC_FORWARD_PATH", raising=False)
    print(f"[case] one-launch repeated / prepacked T=64 D={D}", file=sys.stderr, flush=True)
    inp = synth.custom(64, 4, D, gamma=True, need_backward=True, seed=162)
    r = _runner(inp.wl, True)
    assert r.path() == 2
    runs = gpu_forward(inp, runner=r, repeat=3)
    for k in runs[0]:
        for other in runs[1:]:
            assert np.array_equal(runs[0][k].view(np.uint8), other[k].view(np.uint8)), k
    orc = run_oracle(inp)
    compare(runs[-1], orc, inp)
    g_packed = gpu_forward(inp, runner=r, packed=True)
    if D == 3072:
        for k in g_packed:
            assert np.array_equal(g_packed[k].view(np.uint8), runs[0][k].view(np.uint8)), k
    else:
        compare(g_packed, orc, inp)
    assert r.wait_status() == 0


def test_decode_and_four_kernel_path_agree_with_oracle(monkeypatch):
    # the same inputs through both paths (different summation groupings): each meets the
    # oracle's acceptance rule
    print("[case] one-launch vs classic T=37 D=3072", file=sys.stderr, flush=True)
    inp = synth.custom(37, 4, 3072, gamma=True, need_backward=True, seed=163)
    orc = run_oracle(inp)
    monkeypatch.delenv("MHC_FORWARD_PATH", raising=False)
    r = _runner(inp.wl, True)
    assert r.path() == 2
    compare(gpu_forward(inp, runner=r), orc, inp)
    monkeypatch.setenv("MHC_FORWARD_PATH", "classic")
    assert r.path() == 0
    compare(gpu_forward(inp, runner=r), orc, inp)


def test_decode_wait_time_out_is_reported(monkeypatch):
    # every poll made to give up (about 0.3 s each): the call still returns, every output is
    # NaN (the records every output comes from are never accepted), and
    # mhc_pre_wait_status reports the time-out once, then clears it; the next normal call
    # through the same workspace meets the oracle
    monkeypatch.delenv("MHC_FORWARD_PATH", raising=False)
    monkeypatch.setenv("MHC_TEST_EXCHANGE_NEVER_READY", "1")
    print("[case] one-launch forced wait time-out T=20 D=2048", file=sys.stderr, flush=True)
    inp = synth.custom(20, 4, 2048, need_backward=True, seed=164)
    r = _runner(inp.wl, True)
    assert r.path() == 2
    g = gpu_forward(inp, runner=r)
    assert r.wait_status() == 1
    assert r.wait_status() == 0
    hin = g["h_in"].view(np.int16)
    assert np.all((hin & 0x7F80) == 0x7F80) and np.all((hin & 0x7F) != 0)   # bf16 NaN everywhere
    for k in ("h_pre", "h_post", "h_res", "inv_rms", "h_mix"):
        assert np.all(np.isnan(g[k])), k
    monkeypatch.delenv("MHC_TEST_EXCHANGE_NEVER_READY")
    compare(gpu_forward(inp, runner=r), run_oracle(inp), inp)
    assert r.wait_status() == 0
