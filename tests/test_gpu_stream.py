"""The streaming projection (path 3: persistent workgroups that keep a slice's packed weights
in LDS and load the next task's x while the current one is on the matrix cores; each slice a
contiguous run of K-steps of the flattened row), the projection of every call without pre_mix,
with D a multiple of 32, that the single-read and one-launch kernels do not take: n = 4
(alpha[3] and alpha[2]), n = 8 and n = 6 with alpha[2], bf16 or fp16 x. Parity with the fp64
oracle under the acceptance rule of gpu_helpers at small and ragged sizes: a partial last
64-token tile, fewer tiles than the workgroups of a slice (halves with no task), a partial last
slice (K-steps past the data), gamma, packed and unpacked weights. Its slices group the
partial sums differently from the classic path's, so the two agree with the oracle, not
bit for bit; the weights it splits itself must give the same bits as weights packed
beforehand (gathered from the d-block-major packed layout), and repeated calls the same bits.
With pre_mix, or D not a multiple of 32, the classic path serves."""
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


CASES = [
    # (name, T, n, D, n_alpha, gamma, need_backward, fp16 x, seed)
    ("n4_T65_D992_gamma", 65, 4, 992, 3, True, True, False, 302),
    ("n4_T700_D4096_gamma_bwd", 700, 4, 4096, 3, True, True, False, 303),
    ("n4_T4100_D2048", 4100, 4, 2048, 3, False, False, False, 304),
    ("n4_T300_D7168_bwd", 300, 4, 7168, 3, False, True, False, 305),
    ("n4a2_T999_D3008_gamma", 999, 4, 3008, 2, True, True, False, 306),
    ("n8a2_T1100_D2048", 1100, 8, 2048, 2, False, True, False, 307),
    ("n8a2_T129_D1024_gamma", 129, 8, 1024, 2, True, False, False, 308),
    ("n6a2_T500_D1536", 500, 6, 1536, 2, False, True, False, 309),
    ("n6a2_T77_D992_gamma", 77, 6, 992, 2, True, True, False, 310),
    ("f16_n4_T700_D4096_gamma_bwd", 700, 4, 4096, 3, True, True, True, 311),
    ("f16_n8a2_T1100_D2048", 1100, 8, 2048, 2, False, True, True, 312),
]


@pytest.mark.parametrize("name,T,n,D,na,gamma,nb,f16,seed", CASES, ids=[c[0] for c in CASES])
def test_stream_parity(name, T, n, D, na, gamma, nb, f16, seed, monkeypatch):
    monkeypatch.delenv("MHC_FORWARD_PATH", raising=False)
    monkeypatch.delenv("MHC_PROJECTION", raising=False)
    print(f"[case] streaming {name} T={T} n={n} D={D} alpha[{na}] gamma={gamma} need_backward={nb} f16={f16}",
          file=sys.stderr, flush=True)
    inp = synth.custom(T, n, D, n_alpha=na, gamma=gamma, need_backward=nb, seed=seed, x_f16=f16)
    r = _runner(inp.wl, nb)
    assert r.path(False) == 3
    rep = compare(gpu_forward(inp, runner=r), run_oracle(inp), inp)
    print(f"[streaming] {name}: {summary(rep)}", file=sys.stderr, flush=True)


@pytest.mark.parametrize("T,n,D,na,pm,want", [(300, 4, 7168, 3, True, 0), (300, 8, 2048, 2, True, 0),
                                             (4100, 8, 2048, 2, True, 0), (300, 4, 1000, 3, False, 0),
                                             (300, 4, 992, 3, False, 3)])
def test_stream_not_taken(T, n, D, na, pm, want, monkeypatch):
    # with pre_mix or D not a multiple of 32 the classic path serves, and meets the oracle
    # (n = 8, alpha[2] with pre_mix at T = 4100: its 32-K-step slices and a partial last tile)
    monkeypatch.delenv("MHC_FORWARD_PATH", raising=False)
    print(f"[case] path T={T} n={n} D={D} alpha[{na}] pre_mix={pm}", file=sys.stderr, flush=True)
    inp = synth.custom(T, n, D, n_alpha=na, pre_mix=pm, need_backward=True, seed=330 + n)
    r = _runner(inp.wl, True)
    assert r.path(pm) == want
    compare(gpu_forward(inp, runner=r), run_oracle(inp), inp)


@pytest.mark.parametrize("n,na,D,f16", [(4, 3, 2048, False), (8, 2, 2048, False), (4, 3, 992, True),
                                        (6, 2, 992, False)])
def test_stream_prepacked_same_bits(n, na, D, f16, monkeypatch):
    # phi packed once by mhc_pre_prepack and copied into LDS, against the split inside the
    # kernel: the same bits; and repeated calls through one workspace give the same bits
    monkeypatch.delenv("MHC_FORWARD_PATH", raising=False)
    print(f"[case] streaming prepacked n={n} alpha[{na}] D={D} f16={f16}", file=sys.stderr, flush=True)
    inp = synth.custom(1500, n, D, n_alpha=na, gamma=True, need_backward=True, seed=320 + n, x_f16=f16)
    r = _runner(inp.wl, True)
    assert r.path(False) == 3
    g_packed = gpu_forward(inp, runner=r, packed=True)
    compare(g_packed, run_oracle(inp), inp)
    runs = gpu_forward(inp, runner=r, packed=False, repeat=2)
    for other in runs:
        for k in g_packed:
            assert np.array_equal(g_packed[k].view(np.uint8), other[k].view(np.uint8)), k
