"""GPU parity of hc_post (mhc_post through the C-ABI) against the fp64 oracle
(oracle/mhc_oracle_post.c) on seeded inputs (synth.post_inputs).

Acceptance rule: every output element within 1 bf16 ulp of the oracle's correctly rounded
value, or, where the sum cancels, |gpu - ref| <= 2^-20 * sum of |terms| (the same rule as
hIn: fp32 fused multiply-adds of n + 1 products, each exact in fp32 up to the bf16 inputs'
8 bits times the f32 weights' 24, so the fp32 error stays far below 2^-20 of the terms)."""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import bf16_ordered, device, to_dev, to_host
from synth import bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def gpu_post(pi, repeat=1):
    import mhc_hyper_connection_amd as mhc
    import torch
    dev = device()
    x, res, post, comb = (to_dev(a, dev) for a in (pi.x, pi.residual, pi.post, pi.comb))
    out = torch.empty((pi.T, pi.n, pi.D), dtype=torch.bfloat16, device=dev)
    results = []
    for _ in range(repeat):
        out.view(torch.int16).fill_(0x7FC0)   # NaN: anything not written shows
        mhc.mhc_post(x, res, post, comb, out=out)
        torch.cuda.synchronize(dev)
        results.append(to_host(out))
    return results if repeat > 1 else results[0]


def check(g, pi, tokens=None):
    tok = np.arange(pi.T) if tokens is None else np.asarray(tokens)
    ref = oracle.post(pi.x[tok], pi.residual[tok], pi.post[tok], pi.comb[tok])
    gt = g[tok]
    dist = np.abs(bf16_ordered(gt) - bf16_ordered(ref.out_bf16))
    cancel = np.abs(bf16_bits_to_f32(gt).astype(np.float64) - ref.out) <= 2.0 ** -20 * ref.out_abs
    bad = ~((dist <= 1) | cancel)
    print(f"[parity-post] fail={int(bad.sum())}/{bad.size} max_ulp={int(dist.max()) if dist.size else 0} "
          f"exact={int((dist == 0).sum())}", file=sys.stderr, flush=True)
    assert not bad.any(), f"{int(bad.sum())} outputs out of tolerance"


CASES = [("T1_D8_n4", 1, 4, 8, 1), ("T3_D40_n4", 3, 4, 40, 2), ("T65_D520_n4", 65, 4, 520, 3),
         ("T17_D24_n8", 17, 8, 24, 4), ("T70_D2048_n8", 70, 8, 2048, 5), ("T300_D7168_n4", 300, 4, 7168, 6),
         ("T37_D1032_n6", 37, 6, 1032, 7),
         # the largest D hc_post takes
         ("T9_D16384_n4", 9, 4, 16384, 8), ("T20_D16384_n8", 20, 8, 16384, 9)]


@pytest.mark.parametrize("name,T,n,D,seed", CASES, ids=[c[0] for c in CASES])
def test_post_parity(name, T, n, D, seed):
    print(f"[case] post {name}", file=sys.stderr, flush=True)
    pi = synth.post_inputs(T, n, D, seed=seed)
    check(gpu_post(pi), pi)


def test_post_permutation_is_exact():
    # a non-symmetric permutation as comb and post = 0: output stream perm(i) is exactly
    # residual stream i (the sum runs over comb's first index)
    print("[case] post permutation", file=sys.stderr, flush=True)
    pi = synth.post_inputs(40, 4, 256, seed=7)
    pi.post[:] = 0.0
    pi.comb[:] = 0.0
    for i in range(4):
        pi.comb[:, i, (i + 1) % 4] = 1.0
    g = gpu_post(pi)
    for i in range(4):
        assert np.array_equal(g[:, (i + 1) % 4, :], pi.residual[:, i, :])


def test_post_empty_and_reproducible():
    import mhc_hyper_connection_amd as mhc
    import torch
    dev = device()
    e = torch.empty((0, 4, 64), dtype=torch.bfloat16, device=dev)
    out = mhc.mhc_post(torch.empty((0, 64), dtype=torch.bfloat16, device=dev), e,
                       torch.empty((0, 4), device=dev), torch.empty((0, 4, 4), device=dev))
    assert out.shape == (0, 4, 64)
    print("[case] post determinism T=500 D=4096", file=sys.stderr, flush=True)
    pi = synth.post_inputs(500, 4, 4096, seed=8)
    a, b = gpu_post(pi, repeat=2)
    assert np.array_equal(a, b)


def test_post_large_workload_shape():
    # the large prefill shape (T = 16384, n = 4, D = 7168), as the benchmark runs it:
    # every token against the oracle
    print("[case] post large T=16384 D=7168", file=sys.stderr, flush=True)
    pi = synth.post_inputs(16384, 4, 7168, seed=1004)
    g = gpu_post(pi)
    for t0 in range(0, pi.T, 2048):   # every token, in chunks that bound host memory
        check(g, pi, tokens=np.arange(t0, min(pi.T, t0 + 2048)))


@pytest.mark.parametrize("T,n,D", [(33, 4, 520), (17, 8, 64), (9, 6, 7168)])
def test_post_parity_f16(T, n, D):
    # binary16 x, residual and out
    import mhc_hyper_connection_amd as mhc
    import torch
    print(f"[case] post f16 T={T} n={n} D={D}", file=sys.stderr, flush=True)
    rng = np.random.default_rng(100 + T)
    x = rng.standard_normal((T, D), dtype=np.float32).astype(np.float16).view(np.uint16)
    res = rng.standard_normal((T, n, D), dtype=np.float32).astype(np.float16).view(np.uint16)
    post = rng.uniform(0.0, 2.0, (T, n)).astype(np.float32)
    comb = rng.uniform(0.05, 0.45, (T, n, n)).astype(np.float32)
    dev = device()
    out = mhc.mhc_post(to_dev(x, dev, True), to_dev(res, dev, True), to_dev(post, dev), to_dev(comb, dev))
    torch.cuda.synchronize(dev)
    assert out.dtype == torch.float16
    g = to_host(out)
    ref = oracle.post(x, res, post, comb, x_f16=True)
    dist = np.abs(bf16_ordered(g) - bf16_ordered(ref.out_bf16))
    cancel = np.abs(g.view(np.float16).astype(np.float64) - ref.out) <= 2.0 ** -20 * ref.out_abs
    bad = ~((dist <= 1) | cancel)
    print(f"[parity-post-f16] fail={int(bad.sum())}/{bad.size} max_ulp={int(dist.max())}", file=sys.stderr, flush=True)
    assert not bad.any()
