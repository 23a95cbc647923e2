"""The oracle's two standalone stages -- invRms alone, and the Sinkhorn stage that starts
from given mixes and invRms (the HcPre guide's "function description" names both as
operators of their own) -- against what pins them, and the pins against planted mistakes.

Pins:
  inv_rms closed    x == 0.5, x == 0 and one stream at 1 with another at 3: invRms is
                    1/sqrt(mean + normEps) with the mean over all n*D entries.
  gates closed      per-token mixes and invRms chosen so that alpha * mix * invRms + bias
                    hits special values of the logistic function (sigma(0) = 1/2,
                    sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4); every token differs, so a
                    token read from the wrong row shows.
  uniform logits    res mixes equal within each token (a different value per token): the
                    scalar recursion a_0 = 1/n + eps, a_k = a_(k-1) / (n a_(k-1) + eps).
  rank-1 logits     hcEps = 0, invRms = 1, alpha2 = 1, L_t[r][c] = u_t[r] + v_t[c] with
                    u, v drawn per token: plane 0 is softmax(v_t) in every row, every later
                    plane is 1/n.
  permutation       permuting rows and columns of one token's logits permutes every
                    plane the same way (Sinkhorn treats rows and columns alike up to order).
  hIn               one-hot pre_mix returns the chosen stream's x bit-exactly; without
                    pre_mix hIn equals NumPy's float64 weighted sum with weights hPre.
  whole forward     the stage fed the whole forward's own hMix and invRms reproduces the
                    forward's gates, planes and hIn (whose own pins live beside them).
"""
from __future__ import annotations

import math
import os
import subprocess

import numpy as np
import pytest

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits

EPS = 1e-6
HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "mhc_oracle.c")
BWD = os.path.join(HERE, "mhc_oracle_bwd.c")
POST = os.path.join(HERE, "mhc_oracle_post.c")


def _close(got, want, rtol, atol=0.0, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    lim = atol + rtol * np.abs(want)
    if not np.all(err <= lim):
        i = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: worst |got-want|={err.flat[i]:.3e} at {i} "
                             f"(got {got.flat[i]!r}, want {want.flat[i]!r})")


def _bits(values) -> np.ndarray:
    v = np.asarray(values, dtype=np.float32)
    b = f32_to_bf16_bits(v)
    assert np.array_equal(bf16_bits_to_f32(b), v), "test value not exact in bf16"
    return b


def _x(T, n, D, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((T, n, D), dtype=np.float32))


def pin_inv_rms_closed(lib=None):
    n, D = 4, 8
    _close(oracle.inv_rms(_bits(np.full((3, n, D), 0.5)), lib=lib), 1.0 / math.sqrt(0.25 + EPS),
           1e-15, what="invRms x=0.5")
    _close(oracle.inv_rms(_bits(np.zeros((1, n, D))), lib=lib), 1000.0, 1e-12, what="invRms x=0")
    xv = np.zeros((2, n, D), np.float32)
    xv[0, 0, :] = 1.0
    xv[0, 1, :] = 3.0
    xv[1, 2, :] = 2.0     # token 1: (D * 4) / (4 D) = 1
    got = oracle.inv_rms(_bits(xv), lib=lib)
    _close(got, [1.0 / math.sqrt(2.5 + EPS), 1.0 / math.sqrt(1.0 + EPS)], 1e-15,
           what="invRms per token")


def pin_gates_closed(lib=None):
    # token t: invRms = 1/2 (t even) or 1/4 (t odd); the pre/post mixes are chosen so
    # that alpha * mix * invRms lands on 0, +ln 3 or -ln 3 after the bias.
    n, D, T = 4, 8, 4
    M = n * n + 2 * n
    alpha = np.array([2.0, 4.0, 1.0], np.float32)
    bias = np.zeros(M, np.float32)
    inv = np.array([0.5, 0.25, 0.5, 0.25])
    z_pre = np.array([[0.0, math.log(3), -math.log(3), 0.0]] * T)
    z_post = np.array([[math.log(3), 0.0, 0.0, -math.log(3)]] * T)
    for t in range(T):
        z_pre[t] = np.roll(z_pre[t], t)
        z_post[t] = np.roll(z_post[t], -t)
    h_mix = np.zeros((T, M))
    h_mix[:, :n] = z_pre / (alpha[0] * inv[:, None])
    h_mix[:, n:2 * n] = z_post / (alpha[1] * inv[:, None])
    sig = {0.0: 0.5, math.log(3): 0.75, -math.log(3): 0.25}
    r = oracle.pre_sinkhorn(_x(T, n, D, 3), h_mix, inv, alpha, bias, lib=lib)
    want_pre = np.vectorize(lambda z: sig[z])(z_pre) + EPS
    want_post = 2.0 * np.vectorize(lambda z: sig[z])(z_post)
    _close(r.h_pre, want_pre, 1e-14, what="hPre")
    _close(r.h_post, want_post, 1e-14, what="hPost")


def pin_uniform_logits(lib=None):
    n, D, T, it = 4, 8, 3, 6
    M = n * n + 2 * n
    h_mix = np.zeros((T, M))
    for t in range(T):
        h_mix[t, 2 * n:] = 0.5 * (t + 1) - 1.0
    alpha = np.array([1.0, 1.0, 1.5], np.float32)
    r = oracle.pre_sinkhorn(_x(T, n, D, 4), h_mix, np.full(T, 0.75), alpha, np.zeros(M, np.float32),
                            num_iters=it, lib=lib)
    a = [1.0 / n + EPS]
    for _ in range(1, 2 * it):
        a.append(a[-1] / (n * a[-1] + EPS))
    for k in range(2 * it):
        _close(r.norm_out[k], np.full((T, n, n), a[k]), 1e-14, what=f"normOut[{k}]")
        _close(r.sum_out[k], np.full((T, n), float(n) if k == 0 else n * a[k - 1] + EPS), 1e-14,
               what=f"sumOut[{k}]")
    _close(r.h_res, np.full((T, n, n), a[-1]), 1e-14, what="hRes")


def pin_rank1_logits(lib=None):
    n, D, T, it = 4, 8, 3, 2
    M = n * n + 2 * n
    rng = np.random.default_rng(5)
    u = rng.uniform(-1, 1, (T, n))
    v = rng.uniform(-2, 2, (T, n))
    h_mix = np.zeros((T, M))
    h_mix[:, 2 * n:] = (u[:, :, None] + v[:, None, :]).reshape(T, n * n)
    r = oracle.pre_sinkhorn(_x(T, n, D, 6), h_mix, np.ones(T), np.array([1.0, 1.0, 1.0], np.float32),
                            np.zeros(M, np.float32), num_iters=it, hc_eps=0.0, lib=lib)
    for t in range(T):
        e = np.exp(v[t] - v[t].max())
        _close(r.norm_out[0, t], np.tile(e / e.sum(), (n, 1)), 1e-13, what=f"plane 0 token {t}")
        for k in range(1, 2 * it):
            _close(r.norm_out[k, t], np.full((n, n), 1.0 / n), 1e-13, what=f"plane {k} token {t}")


def pin_permutation(lib=None):
    n, D, T = 4, 8, 2
    M = n * n + 2 * n
    rng = np.random.default_rng(7)
    L = rng.uniform(-1.5, 1.5, (n, n))
    P = [2, 0, 3, 1]          # a row order
    Q = [1, 3, 0, 2]          # a column order
    h_mix = np.zeros((T, M))
    h_mix[0, 2 * n:] = L.reshape(-1)
    h_mix[1, 2 * n:] = L[P][:, Q].reshape(-1)
    r = oracle.pre_sinkhorn(_x(T, n, D, 8), h_mix, np.ones(T), np.array([1.0, 1.0, 1.0], np.float32),
                            np.zeros(M, np.float32), num_iters=5, lib=lib)
    for k in range(r.norm_out.shape[0]):
        _close(r.norm_out[k, 1], r.norm_out[k, 0][P][:, Q], 1e-13, what=f"permuted plane {k}")
    _close(r.h_res[1], r.h_res[0][P][:, Q], 1e-13, what="permuted hRes")


def pin_hin(lib=None):
    n, D, T = 4, 16, 3
    M = n * n + 2 * n
    rng = np.random.default_rng(9)
    x = _x(T, n, D, 10)
    h_mix = rng.standard_normal((T, M))
    inv = rng.uniform(0.5, 2.0, T)
    alpha = np.array([0.7, 0.9, 1.1], np.float32)
    bias = rng.uniform(-0.5, 0.5, M).astype(np.float32)
    pick = [2, 0, 3]
    pre_mix = np.zeros((T, n), np.float32)
    pre_mix[np.arange(T), pick] = 1.0
    r = oracle.pre_sinkhorn(x, h_mix, inv, alpha, bias, pre_mix, lib=lib)
    for t in range(T):
        assert np.array_equal(r.h_in_bf16[t], x[t, pick[t]]), f"one-hot pre_mix, token {t}"
    r = oracle.pre_sinkhorn(x, h_mix, inv, alpha, bias, lib=lib)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    _close(r.h_in, np.einsum("ti,tid->td", r.h_pre, xf), 1e-12, atol=1e-300, what="hIn = hPre . x")


def pin_whole_forward(lib=None):
    for n, na in ((4, 3), (8, 3), (4, 2)):
        D, T = 16, 5
        M = n * n + 2 * n if na == 3 else 2 * n
        rng = np.random.default_rng(11 + n + na)
        x = _x(T, n, D, 12 + n)
        phi = (rng.standard_normal((M, n * D)) / (n * D)).astype(np.float32)
        alpha = rng.uniform(0.5, 1.5, na).astype(np.float32)
        bias = rng.uniform(-0.5, 0.5, M).astype(np.float32)
        f = oracle.forward(x, phi, alpha, bias, num_iters=4, lib=lib)
        s = oracle.pre_sinkhorn(x, f.h_mix, f.inv_rms, alpha, bias, num_iters=4, lib=lib)
        for name in ("h_pre", "h_post", "h_res", "h_in", "h_in_bf16"):
            assert np.array_equal(getattr(s, name), getattr(f, name)), f"{name} n={n} alpha={na}"
        if na == 3:
            assert np.array_equal(s.sum_out, f.sum_out) and np.array_equal(s.norm_out, f.norm_out)
        assert np.array_equal(oracle.inv_rms(x, lib=lib), f.inv_rms), "invRms alone"


PINS = [pin_inv_rms_closed, pin_gates_closed, pin_uniform_logits, pin_rank1_logits,
        pin_permutation, pin_hin, pin_whole_forward]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(None)


def test_rejects_bad_descriptions():
    with pytest.raises(ValueError):
        oracle.inv_rms(np.zeros((2, 4), np.uint16))
    with pytest.raises(ValueError):
        oracle.pre_sinkhorn(np.zeros((1, 4, 8), np.uint16), np.zeros((1, 24)), np.ones(1),
                            np.ones(3, np.float32), np.zeros(24, np.float32), num_iters=0)


# Mistakes local to the two standalone entry points (the per-token arithmetic they share
# with the whole forward is mutated by the forward's own mutant suite).
MUTANTS = {
    "mixes_of_token_0": ("finish_token(c, c->T, t, t, x, h_mix + t * M, inv_rms[t],",
                         "finish_token(c, c->T, t, t, x, h_mix, inv_rms[t],"),
    "inv_rms_of_token_0": ("finish_token(c, c->T, t, t, x, h_mix + t * M, inv_rms[t],",
                           "finish_token(c, c->T, t, t, x, h_mix + t * M, inv_rms[0],"),
    "x_of_token_0": ("inv_rms[t] = token_inv_rms(c, x + t * K, c->n, c->D, c->norm_eps);",
                     "inv_rms[t] = token_inv_rms(c, x, c->n, c->D, c->norm_eps);"),
    "rms_mean_over_D": ("ss / (double)K + norm_eps", "ss / (double)D + norm_eps"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(so_path),
                    str(c_path), BWD, POST, "-lm"], check=True)
    lib = oracle.load_library(str(so_path))
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
