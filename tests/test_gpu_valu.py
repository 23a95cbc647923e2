"""The projection on the VALU (fp32 FMA, MHC_PROJECTION=valu) on the classic path,
against the fp64 oracle under the acceptance rule of gpu_helpers: every M <= 32 variant
(n = 4 with alpha[3] and alpha[2], n = 8 and n = 6 with alpha[2]), pre_mix (hIn written
by the projection), gamma, partial last d-blocks and tiles, fp16 x, and both slice sizes
of n = 4 with alpha[2]; plus the wide workload at full size on sampled tokens. The choice
between this path and the matrix cores is made by measurement (bench.py per workload)."""
import sys

import pytest

import synth
from gpu_helpers import compare, gpu_forward, run_oracle, summary

pytestmark = pytest.mark.gpu

CASES = [
    # (name, T, n, D, n_alpha, gamma, pre_mix, need_backward, f16, seed)
    ("n4a3_D7168_bwd", 200, 4, 7168, 3, False, False, True, False, 71),
    ("n4a3_gamma_D4096", 130, 4, 4096, 3, True, False, False, False, 72),
    ("n4a3_premix_D1032", 90, 4, 1032, 3, True, True, False, False, 73),
    ("n4a2_D512_bwd", 50, 4, 512, 2, False, False, True, False, 74),
    ("n4a2_big_slices", 4100, 4, 1024, 2, False, False, False, False, 75),
    ("n8a2_premix_D2048", 100, 8, 2048, 2, False, True, False, False, 76),
    ("n8a2_premix_D24_T17", 17, 8, 24, 2, False, True, False, False, 77),
    ("n6a2_premix_D520", 65, 6, 520, 2, False, True, True, False, 78),
    ("n4a3_f16_D2056", 65, 4, 2056, 3, True, False, True, True, 79),
    ("n8a2_f16_premix", 40, 8, 1024, 2, False, True, False, True, 80),
]


@pytest.mark.parametrize("name,T,n,D,na,gamma,pm,nb,f16,seed", CASES, ids=[c[0] for c in CASES])
def test_valu_projection_parity(name, T, n, D, na, gamma, pm, nb, f16, seed, monkeypatch):
    monkeypatch.setenv("MHC_PROJECTION", "valu")
    monkeypatch.setenv("MHC_FORWARD_PATH", "classic")
    print(f"[case] valu {name} T={T} n={n} D={D} alpha={na}", file=sys.stderr, flush=True)
    inp = synth.custom(T, n, D, n_alpha=na, gamma=gamma, pre_mix=pm, need_backward=nb, seed=seed,
                       x_f16=f16)
    rep = compare(gpu_forward(inp), run_oracle(inp), inp)
    print(f"[valu] {name}: {summary(rep)}", file=sys.stderr, flush=True)
