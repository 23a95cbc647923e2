"""Pins of the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes an oracle library handle (None = the real build)
and raises AssertionError on a mismatch. ``test_oracle_pins.py`` runs them on
the real oracle; ``test_oracle_mutants.py`` runs them on altered copies of the
oracle source and requires every alteration to be caught by at least one pin.

What pins what (expected values are closed forms derived by hand, special cases
that reduce to a library routine, or invariants of the mathematics):
  bf16 rounding   bit patterns of the IEEE binary32/bfloat16 definition
  invRms          x constant, x zero, one stream non-zero (fixes the n*D mean),
                  gamma does not enter invRms
  hMix            one-hot phi rows (transposition, gamma indexing), all-ones,
                  numpy float64 matmul at a small size (independent routine)
  gates           special values of the logistic function: sigma(0)=1/2,
                  sigma(ln 3)=3/4, sigma(-ln 3)=1/4, sigma(ln 7)=7/8, with invRms=1/2
                  exactly so the normalisation, alpha and bias indexing all show
  alpha of [2]    hRes == 0, hPost gets +hcEps
  Sinkhorn        uniform logits -> scalar recursion; rank-1 logits with hcEps=0 ->
                  softmax of the column offsets then 1/n; the last step normalises
                  columns; row shifts leave every plane unchanged; rows and columns
                  sum to 1 within 1e-3 on well-conditioned logits
  hIn             one-hot pre_mix returns the stream's x bit-exactly; dyadic weights
                  give exact sums; without pre_mix the weights are hPre
  page example    all inputs 1.0 at n=4, D=2560 (aclnnMhcPreV2 guide, section 9)
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits

EPS = 1e-6


def _bits(values) -> np.ndarray:
    v = np.asarray(values, dtype=np.float32)
    b = f32_to_bf16_bits(v)
    assert np.array_equal(bf16_bits_to_f32(b), v), "test value not exact in bf16"
    return b


def _close(got, want, rtol, atol=0.0, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    lim = atol + rtol * np.abs(want)
    if not np.all(err <= lim):
        i = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: worst |got-want|={err.flat[i]:.3e} at {i} "
                             f"(got {got.flat[i]!r}, want {want.flat[i]!r})")


def _run(x, phi, alpha, bias, gamma=None, pre_mix=None, lib=None, **kw):
    return oracle.forward(x, phi, alpha, bias, gamma, pre_mix, lib=lib, **kw)


def _zeros_params(n, D, n_alpha=3):
    M = n * n + 2 * n if n_alpha == 3 else 2 * n
    return (np.zeros((M, n * D), np.float32), np.zeros(n_alpha, np.float32),
            np.zeros(M, np.float32))


# ------------------------------------------------------------------ bf16 rounding

# (value, expected bits): binary32 has 1 sign, 8 exponent, 23 fraction bits; bf16
# keeps the top 16 of them. Ties go to the even fraction.
BF16_CASES = [
    (1.0, 0x3F80),
    (-2.0, 0xC000),
    (3.0, 0x4040),
    (1.0 + 2.0 ** -8, 0x3F80),                  # tie -> even (fraction 0)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),              # tie -> even (fraction 2)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),     # just above the tie
    (1.0 + 2.0 ** -8 - 2.0 ** -30, 0x3F80),     # just below the tie
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),     # largest finite
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),     # tie above the largest -> inf
    (2.0 ** -133, 0x0001),                      # smallest subnormal
    (2.0 ** -134, 0x0000),                      # tie between 0 and it -> even (0)
    (1.5 * 2.0 ** -134, 0x0001),
    (2.0 ** -130, 0x0008),
    (-0.0, 0x8000),
    (float("inf"), 0x7F80),
    (0.1, 0x3DCD),                              # 0.1 = 1.6 * 2^-4; 0.6*128 = 76.8 -> 77 = 0x4D
]


def pin_bf16_rounding(lib=None):
    for v, bits in BF16_CASES:
        got = oracle.bf16_from_double(v, lib=lib)
        assert got == bits, f"bf16({v!r}) = {got:#06x}, want {bits:#06x}"
    assert oracle.bf16_from_double(float("nan"), lib=lib) & 0x7FC0 == 0x7FC0
    for bits in (0x3F80, 0xC000, 0x0001, 0x7F7F, 0x3DCD):
        v = oracle.bf16_to_double(bits, lib=lib)
        assert oracle.bf16_from_double(v, lib=lib) == bits


# ------------------------------------------------------------------ invRms

def pin_inv_rms(lib=None):
    n, D = 4, 8
    phi, alpha, bias = _zeros_params(n, D)
    # x == 0.5 everywhere: mean of squares is 0.25
    x = _bits(np.full((2, n, D), 0.5))
    r = _run(x, phi, alpha, bias, lib=lib, want_h_in=False)
    _close(r.inv_rms, 1.0 / math.sqrt(0.25 + EPS), 1e-15, what="invRms x=0.5")
    # gamma scales only the projection input, never the RMS statistic
    gamma = np.full((n, D), 2.0, np.float32)
    r = _run(x, phi, alpha, bias, gamma=gamma, lib=lib, want_h_in=False)
    _close(r.inv_rms, 1.0 / math.sqrt(0.25 + EPS), 1e-15, what="invRms with gamma")
    # x == 0: invRms = normEps^(-1/2) = 1000
    x = _bits(np.zeros((1, n, D)))
    r = _run(x, phi, alpha, bias, lib=lib, want_h_in=False)
    _close(r.inv_rms, 1000.0, 1e-12, what="invRms x=0")
    # stream 0 == 1, stream 1 == 3, streams 2, 3 == 0: the mean runs over n*D entries,
    # (D*1 + D*9) / (4*D) = 2.5
    xv = np.zeros((1, n, D), np.float32)
    xv[0, 0, :] = 1.0
    xv[0, 1, :] = 3.0
    r = _run(_bits(xv), phi, alpha, bias, lib=lib, want_h_in=False)
    _close(r.inv_rms, 1.0 / math.sqrt(2.5 + EPS), 1e-15, what="invRms one stream")


# ------------------------------------------------------------------ hMix

def pin_hmix_one_hot(lib=None):
    n, D = 4, 8
    K = n * D
    M = n * n + 2 * n
    rng = np.random.default_rng(11)
    x = f32_to_bf16_bits(rng.standard_normal((3, n, D), dtype=np.float32))
    gamma = rng.uniform(0.5, 1.5, size=(n, D)).astype(np.float32)
    phi = np.zeros((M, K), np.float32)
    ks = [(7 * m + 3) % K for m in range(M)]      # spread over all four streams
    for m, k in enumerate(ks):
        phi[m, k] = 1.0
    alpha = np.zeros(3, np.float32)
    bias = np.zeros(M, np.float32)
    xf = bf16_bits_to_f32(x).reshape(3, K).astype(np.float64)
    gf = gamma.reshape(K).astype(np.float64)
    r = _run(x, phi, alpha, bias, lib=lib, want_h_in=False)
    _close(r.h_mix, xf[:, ks], 0.0, what="hMix one-hot")
    r = _run(x, phi, alpha, bias, gamma=gamma, lib=lib, want_h_in=False)
    _close(r.h_mix, xf[:, ks] * gf[ks], 0.0, what="hMix one-hot with gamma")


def pin_hmix_all_ones(lib=None):
    n, D = 4, 8
    M = n * n + 2 * n
    x = _bits(np.ones((2, n, D)))
    phi = np.ones((M, n * D), np.float32)
    r = _run(x, phi, np.zeros(3, np.float32), np.zeros(M, np.float32), lib=lib,
             want_h_in=False)
    _close(r.h_mix, np.full((2, M), float(n * D)), 0.0, what="hMix all ones")


def pin_hmix_matmul(lib=None):
    # Independent evaluation with numpy's float64 matrix product.
    n, D, T = 4, 16, 5
    M = n * n + 2 * n
    rng = np.random.default_rng(12)
    x = f32_to_bf16_bits(rng.standard_normal((T, n, D), dtype=np.float32))
    phi = rng.standard_normal((M, n * D)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, size=(n, D)).astype(np.float32)
    xg = bf16_bits_to_f32(x).reshape(T, n * D).astype(np.float64) * gamma.reshape(-1)
    want = xg @ phi.astype(np.float64).T
    r = _run(x, phi, np.zeros(3, np.float32), np.zeros(M, np.float32), gamma=gamma,
             lib=lib, want_h_in=False)
    _close(r.h_mix, want, 1e-12, 1e-13, what="hMix vs numpy matmul")


# ------------------------------------------------------------------ gates

LN3 = math.log(3.0)
LN7 = math.log(7.0)


def pin_gates_bias_only(lib=None):
    # alpha == 0: hPre = sigma(b) + eps, hPost = 2 sigma(b), whatever x is.
    n, D = 4, 8
    M = n * n + 2 * n
    rng = np.random.default_rng(13)
    x = f32_to_bf16_bits(rng.standard_normal((2, n, D), dtype=np.float32))
    phi = rng.standard_normal((M, n * D)).astype(np.float32)
    bias = np.zeros(M, np.float32)
    bias[0:4] = [0.0, LN3, -LN3, LN7]
    bias[4:8] = [LN7, 0.0, -LN3, LN3]
    r = _run(x, phi, np.zeros(3, np.float32), bias, lib=lib, want_h_in=False)
    _close(r.h_pre, np.tile([0.5 + EPS, 0.75 + EPS, 0.25 + EPS, 0.875 + EPS], (2, 1)),
           0.0, 1e-7, what="hPre alpha=0")
    _close(r.h_post, np.tile([1.75, 1.0, 0.5, 1.5], (2, 1)), 0.0, 2e-7, what="hPost alpha=0")


def pin_gates_affine(lib=None):
    # x == 2 everywhere and normEps = 0 give invRms = 1/2 exactly; phi rows of v/64
    # give hMix = v exactly (K = 32 entries of 2 * v/64), so w = v/2. The bias is set
    # so that each gate argument lands on a special value of the logistic function.
    n, D = 4, 8
    K = n * D
    M = n * n + 2 * n
    a0, a1 = 0.5, 2.0
    v_pre = np.array([1.0, 2.0, 3.0, 4.0])
    v_post = np.array([-1.0, -2.0, 1.0, 2.0])
    z_pre = np.array([LN3, 0.0, -LN3, LN7])
    z_post = np.array([-LN3, LN3, 0.0, LN7])
    phi = np.zeros((M, K), np.float32)
    phi[0:4, :] = (v_pre / 64.0)[:, None]
    phi[4:8, :] = (v_post / 64.0)[:, None]
    bias = np.zeros(M, np.float32)
    bias[0:4] = z_pre - a0 * v_pre / 2.0
    bias[4:8] = z_post - a1 * v_post / 2.0
    alpha = np.array([a0, a1, 0.0], np.float32)
    x = _bits(np.full((1, n, D), 2.0))
    r = _run(x, phi, alpha, bias, lib=lib, want_h_in=False, norm_eps=0.0)
    _close(r.inv_rms, 0.5, 0.0, what="invRms x=2")
    _close(r.h_mix[0, :8], np.concatenate([v_pre, v_post]), 0.0, what="hMix rows")
    _close(r.h_pre[0], np.array([0.75, 0.5, 0.25, 0.875]) + EPS, 0.0, 1e-7, what="hPre")
    _close(r.h_post[0], [0.5, 1.5, 1.0, 1.75], 0.0, 2e-7, what="hPost")


def pin_alpha2_branch(lib=None):
    n, D = 4, 8
    rng = np.random.default_rng(14)
    x = f32_to_bf16_bits(rng.standard_normal((3, n, D), dtype=np.float32))
    phi = rng.standard_normal((2 * n, n * D)).astype(np.float32)
    bias = np.zeros(2 * n, np.float32)
    r = _run(x, phi, np.zeros(2, np.float32), bias, lib=lib, want_h_in=False)
    assert r.sum_out is None and r.norm_out is None
    assert np.all(r.h_res == 0.0), "hRes must be 0 with a 2-entry alpha"
    _close(r.h_pre, 0.5 + EPS, 0.0, 1e-15, what="hPre alpha[2]")
    _close(r.h_post, 1.0 + EPS, 0.0, 1e-15, what="hPost alpha[2] gets +hcEps")


# ------------------------------------------------------------------ Sinkhorn

def _sinkhorn_inputs(logits, n, D=8, T=None, seed=15):
    """Inputs whose res logits are exactly `logits` ([T, n, n]): alpha2 = 0, so the
    logits are the res part of the bias, which is per-entry, not per-token; hence T=1."""
    M = n * n + 2 * n
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal((1, n, D), dtype=np.float32))
    phi = rng.standard_normal((M, n * D)).astype(np.float32)
    bias = np.zeros(M, np.float32)
    bias[2 * n:] = np.asarray(logits, np.float32).reshape(-1)
    assert np.array_equal(bias[2 * n:].astype(np.float64), np.asarray(logits, np.float64).reshape(-1))
    return x, phi, np.array([1.0, 1.0, 0.0], np.float32), bias


def pin_sinkhorn_uniform(lib=None):
    # Equal logits: every entry follows a_0 = 1/n + eps, a_k = a_{k-1} / (n a_{k-1} + eps);
    # every sum of step k >= 1 is n a_{k-1} + eps; the softmax denominator is n.
    n, it = 4, 20
    x, phi, alpha, bias = _sinkhorn_inputs(np.full((n, n), 0.375), n)
    r = _run(x, phi, alpha, bias, lib=lib, want_h_in=False, num_iters=it)
    a = [1.0 / n + EPS]
    for _ in range(1, 2 * it):
        a.append(a[-1] / (n * a[-1] + EPS))
    assert r.norm_out.shape == (2 * it, 1, n, n) and r.sum_out.shape == (2 * it, 1, n)
    for k in range(2 * it):
        _close(r.norm_out[k], np.full((1, n, n), a[k]), 1e-14, what=f"normOut[{k}]")
        want_s = float(n) if k == 0 else n * a[k - 1] + EPS
        _close(r.sum_out[k], np.full((1, n), want_s), 1e-14, what=f"sumOut[{k}]")
    _close(r.h_res, np.full((1, n, n), a[-1]), 1e-14, what="hRes uniform")


def pin_sinkhorn_rank1(lib=None):
    # hcEps = 0 and L[r][c] = u_r + v_c: the row softmax gives q_c = softmax(v)_c in
    # every row; the column step then makes every entry 1/n, a fixed point.
    n, it = 4, 3
    u = np.array([0.0, 0.5, -1.0, 2.0])
    v = np.array([0.25, -0.75, 1.5, 0.0])
    x, phi, alpha, bias = _sinkhorn_inputs(u[:, None] + v[None, :], n)
    r = _run(x, phi, alpha, bias, lib=lib, want_h_in=False, num_iters=it, hc_eps=0.0)
    e = np.exp(v - v.max())
    q = e / e.sum()
    _close(r.norm_out[0, 0], np.tile(q, (n, 1)), 1e-14, what="normOut[0] rank-1")
    _close(r.sum_out[0, 0], np.full(n, e.sum()), 1e-14, what="sumOut[0] rank-1")
    _close(r.sum_out[1, 0], n * q, 1e-14, what="sumOut[1] (per column)")
    for k in range(1, 2 * it):
        _close(r.norm_out[k, 0], np.full((n, n), 1.0 / n), 1e-14, what=f"normOut[{k}]")
    for k in range(2, 2 * it):
        _close(r.sum_out[k, 0], np.ones(n), 1e-14, what=f"sumOut[{k}]")


def pin_sinkhorn_invariants(lib=None):
    n = 4
    rng = np.random.default_rng(16)
    # Well-conditioned logits: rows and columns of hRes sum to 1 within 1e-3.
    for trial in range(8):
        L = rng.uniform(-1.0, 1.0, size=(n, n)).astype(np.float32)
        x, phi, alpha, bias = _sinkhorn_inputs(L, n, seed=100 + trial)
        h = _run(x, phi, alpha, bias, lib=lib, want_h_in=False).h_res[0]
        assert np.all(np.abs(h.sum(axis=0) - 1.0) <= 1e-3), "columns must sum to 1"
        assert np.all(np.abs(h.sum(axis=1) - 1.0) <= 1e-3), "rows must sum to 1"
        assert np.all(h > 0.0)
    # Badly conditioned logits: after 2*numIters steps the last one normalised the
    # columns, so they sum to S/(S + eps) ~ 1 - eps, while the rows are still off.
    L = (4.0 * rng.standard_normal((n, n))).astype(np.float32)
    x, phi, alpha, bias = _sinkhorn_inputs(L, n, seed=200)
    h = _run(x, phi, alpha, bias, lib=lib, want_h_in=False).h_res[0]
    assert np.all(np.abs(h.sum(axis=0) - 1.0) <= 2.5 * EPS), "last step normalises columns"
    assert np.max(np.abs(h.sum(axis=1) - 1.0)) > 1e-4, "rows should not be converged here"


def pin_sinkhorn_row_shift(lib=None):
    # Adding c_r to row r of the logits changes no plane: the first step is a softmax
    # over each row (and its denominator is taken after subtracting the row max).
    n = 4
    rng = np.random.default_rng(17)
    L = np.round(rng.uniform(-2, 2, size=(n, n)) * 64) / 64
    shift = np.array([0.5, -1.25, 3.0, 0.0])[:, None]
    ra = _run(*_sinkhorn_inputs(L, n), lib=lib, want_h_in=False)
    rb = _run(*_sinkhorn_inputs(L + shift, n), lib=lib, want_h_in=False)
    _close(rb.norm_out, ra.norm_out, 1e-14, what="row-shift normOut")
    _close(rb.sum_out, ra.sum_out, 1e-14, what="row-shift sumOut")
    # A column shift does change the first softmax.
    rc = _run(*_sinkhorn_inputs(L + shift.T, n), lib=lib, want_h_in=False)
    assert np.max(np.abs(rc.norm_out[0] - ra.norm_out[0])) > 1e-3


# ------------------------------------------------------------------ hIn

def pin_hin_one_hot_premix(lib=None):
    n, D, T = 4, 16, 3
    rng = np.random.default_rng(18)
    x = f32_to_bf16_bits(rng.standard_normal((T, n, D), dtype=np.float32))
    M = n * n + 2 * n
    phi = rng.standard_normal((M, n * D)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, size=(n, D)).astype(np.float32)
    alpha = rng.uniform(0.5, 1.5, size=3).astype(np.float32)
    bias = rng.standard_normal(M).astype(np.float32)
    for j in range(n):
        pm = np.zeros((T, n), np.float32)
        pm[:, j] = 1.0
        r = _run(x, phi, alpha, bias, gamma=gamma, pre_mix=pm, lib=lib)
        assert np.array_equal(r.h_in_bf16, x[:, j, :]), f"one-hot pre_mix stream {j}"


def pin_hin_exact_sums(lib=None):
    n, D, T = 4, 8, 2
    rng = np.random.default_rng(19)
    xv = rng.integers(-8, 9, size=(T, n, D)).astype(np.float32)
    pm = np.array([[0.25, 0.5, 1.0, 0.0], [1.0, 0.0, 0.75, 0.5]], np.float32)
    phi, alpha, bias = _zeros_params(n, D)
    r = _run(_bits(xv), phi, alpha, bias, pre_mix=pm, lib=lib)
    want = np.einsum("ti,tid->td", pm.astype(np.float64), xv.astype(np.float64))
    _close(r.h_in, want, 0.0, what="hIn dyadic sums")
    assert np.array_equal(r.h_in_bf16, f32_to_bf16_bits(want.astype(np.float32)))


def pin_hin_uses_hpre(lib=None):
    # No pre_mix, alpha = 0, bias = 0: hPre = 1/2 + eps for every stream (hPost = 1).
    n, D, T = 4, 8, 2
    rng = np.random.default_rng(20)
    xv = rng.integers(-8, 9, size=(T, n, D)).astype(np.float32)
    phi, alpha, bias = _zeros_params(n, D)
    r = _run(_bits(xv), phi, alpha, bias, lib=lib)
    _close(r.h_in, (0.5 + EPS) * xv.astype(np.float64).sum(axis=1), 1e-15, what="hIn = hPre . x")


# ------------------------------------------------------------------ page example

def pin_v2_page_example(lib=None):
    # aclnnMhcPreV2 guide, section 9: n = 4, D = 2560, every input 1.0 (x, phi, alpha,
    # bias, gamma). hMix = n*D = 10240; invRms = (1 + 1e-6)^(-1/2); the gate arguments
    # are ~10241, so hPre = 1 + eps and hPost = 2; all res logits are equal, so hRes
    # follows the uniform recursion; hIn = 4 (1 + eps), which is 4.0 in bf16.
    n, D, T = 4, 2560, 3
    M = n * n + 2 * n
    x = _bits(np.ones((T, n, D)))
    phi = np.ones((M, n * D), np.float32)
    r = _run(x, phi, np.ones(3, np.float32), np.ones(M, np.float32),
             gamma=np.ones((n, D), np.float32), lib=lib)
    _close(r.h_mix, np.full((T, M), 10240.0), 0.0, what="hMix")
    _close(r.inv_rms, np.full(T, (1.0 + EPS) ** -0.5), 1e-15, what="invRms")
    _close(r.h_pre, np.full((T, n), 1.0 + EPS), 1e-15, what="hPre")
    _close(r.h_post, np.full((T, n), 2.0), 1e-15, what="hPost")
    a = 1.0 / n + EPS
    for _ in range(1, 40):
        a = a / (n * a + EPS)
    _close(r.h_res, np.full((T, n, n), a), 1e-14, what="hRes")
    _close(r.h_in, np.full((T, D), 4.0 * (1.0 + EPS)), 1e-15, what="hIn double")
    assert np.all(r.h_in_bf16 == 0x4080), "hIn rounds to 4.0"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
