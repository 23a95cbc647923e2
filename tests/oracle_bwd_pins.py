"""Pins of the fp64 MhcPre-backward oracle to facts other than itself.

Each ``pin_*`` function takes an oracle library handle (None = the real build) and
raises AssertionError on a mismatch. ``test_oracle_bwd.py`` runs them on the real
oracle and on altered copies of ``oracle/mhc_oracle_bwd.c`` (every alteration must be
caught by at least one pin).

What pins what:
  the whole backward   central finite differences of the scalar
                       L = <gradHIn, hIn> + <gradHPost, hPost> + <gradHRes, hRes>
                       through the fp64 MhcPre forward (every gradient is dL/d input),
                       with and without gamma, n = 4, 6 and 8
  the forward it uses  the bf16-input forward oracle (pinned on its own) on the same
                       bf16-exact inputs; hRes against its affine closed form
  alpha = 0            no gradient reaches hMix: gradPhi = gradGamma = 0 and
                       gradX = gradHIn * hPre + gradXPost exactly
  page example         every input 1.0 at T = 1024, n = 4, D = 512 (the MhcPreBackward
                       guide, section 7): closed forms derived by hand below
  summation scale      the returned sums of |terms| bound the sums and equal them
                       when every term is non-negative
  fp16 x / gradHIn     (gradX then takes fp16, the MhcPreBackward guide's section 8.2)
                       the same finite differences on fp16-exact inputs that bf16 cannot
                       hold; gradX's fp16 bits against numpy's correctly rounded float16
  Sinkhorn backward    (MhcPreSinkhorn: hRes is the Sinkhorn of the affine logits) the
                       same finite differences through the double forward with the
                       Sinkhorn steps, n = 4 and 8, 1 to 20 iterations; the double
                       forward's planes against the pinned bf16 forward oracle; adding a
                       constant to a row of logits changes no plane, so the logit
                       gradient (gradBias of the res entries) has zero row sums
"""
from __future__ import annotations

import numpy as np

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits

EPS = 1e-6


def _close(got, want, rtol, atol=0.0, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    lim = atol + rtol * np.abs(want)
    if not np.all(err <= lim):
        i = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: worst |got-want|={err.flat[i]:.3e} at {i} "
                             f"(got {got.flat[i]!r}, want {want.flat[i]!r})")


def _bf16(a):
    bits = f32_to_bf16_bits(np.asarray(a, dtype=np.float32))
    return bits, bf16_bits_to_f32(bits).astype(np.float64)


def _f16(a):
    h = np.asarray(a, dtype=np.float16)
    return h.view(np.uint16).copy(), h.astype(np.float64)


def problem(T=3, n=4, D=8, gamma=True, x_post=True, seed=0, f16=False):
    """A small random MhcPre backward problem with bf16-exact (or, f16, fp16-exact) x,
    gradHIn, gradXPost."""
    rng = np.random.default_rng(seed)
    M, K = n * n + 2 * n, n * D
    x16 = _f16 if f16 else _bf16
    p = {"x_f16": f16}
    p["x_bits"], p["x"] = x16(rng.normal(0, 1, (T, n, D)))
    p["phi"] = rng.normal(0, K ** -0.5, (M, K)).astype(np.float32)
    p["alpha"] = np.array([0.8, 1.1, 0.9], np.float32)
    p["bias"] = rng.normal(0, 0.5, M).astype(np.float32)
    p["gamma"] = rng.uniform(0.5, 1.5, (n, D)).astype(np.float32) if gamma else None
    p["ghin_bits"], p["ghin"] = x16(rng.normal(0, 1, (T, D)))
    p["ghpost"] = rng.normal(0, 1, (T, n)).astype(np.float32)
    p["ghres"] = rng.normal(0, 1, (T, n, n)).astype(np.float32)
    if x_post:
        p["gxp_bits"], p["gxp"] = x16(rng.normal(0, 1, (T, n, D)))
    else:
        p["gxp_bits"], p["gxp"] = None, None
    return p


def forward64(p, x=None, phi=None, alpha=None, bias=None, gamma="same", lib=None):
    g = p["gamma"] if isinstance(gamma, str) else gamma
    return oracle.mhcpre_forward_f64(
        p["x"] if x is None else x, p["phi"] if phi is None else phi,
        p["alpha"] if alpha is None else alpha, p["bias"] if bias is None else bias,
        g, num_iters=p.get("num_iters", 0), lib=lib)


def loss(p, lib=None, **kw):
    f = forward64(p, lib=lib, **kw)
    return float(np.sum(p["ghin"] * f.h_in) + np.sum(p["ghpost"] * f.h_post)
                 + np.sum(p["ghres"] * f.h_res))


def backward(p, fwd=None, lib=None, **kw):
    f = fwd or forward64(p, lib=lib)
    it = p.get("num_iters", 0)
    return oracle.backward(p["x_bits"], p["phi"], p["alpha"], p["ghin_bits"], p["ghpost"],
                           p["ghres"], f.inv_rms, f.h_mix, f.h_pre, f.h_post, p["gamma"],
                           p["gxp_bits"], num_iters=it, sum_out=f.sum_out, norm_out=f.norm_out,
                           x_f16=p.get("x_f16", False), lib=lib, **kw)


def _fd(p, name, lib=None):
    """Central differences of the loss in every entry of input ``name``."""
    base = np.array(p[name] if name != "x" else p["x"], dtype=np.float64)
    g = np.empty(base.shape)
    flat = base.reshape(-1)
    for j in range(flat.size):
        v = flat[j]
        h = 1e-6 * (1.0 + abs(v))
        up, dn = flat.copy(), flat.copy()
        up[j], dn[j] = v + h, v - h
        lu = loss(p, lib=lib, **{name: up.reshape(base.shape)})
        ld = loss(p, lib=lib, **{name: dn.reshape(base.shape)})
        g.reshape(-1)[j] = (lu - ld) / (2 * h)
    return g


def _check_fd(p, lib=None):
    r = backward(p, lib=lib)
    gxp = p["gxp"] if p["gxp"] is not None else 0.0
    for name, got in (("x", r.grad_x - gxp), ("phi", r.grad_phi), ("alpha", r.grad_alpha),
                      ("bias", r.grad_bias)) + ((("gamma", r.grad_gamma),) if p["gamma"] is not None else ()):
        want = _fd(p, name, lib=lib)
        # the saved forward values reach the backward as float32 (~1e-7 relative)
        _close(got, want, 2e-5, 2e-6 * max(1.0, float(np.max(np.abs(want)))), what=f"d L / d {name}")


def pin_fd_n4_gamma(lib=None):
    _check_fd(problem(T=3, n=4, D=8, gamma=True, x_post=True, seed=1), lib)


def pin_fd_n4_plain(lib=None):
    _check_fd(problem(T=2, n=4, D=8, gamma=False, x_post=False, seed=2), lib)


def pin_fd_n6(lib=None):
    # n = 6 (the backward page's section 5 lists N = 4, 6, 8): 48 phi rows
    _check_fd(problem(T=1, n=6, D=4, gamma=True, x_post=True, seed=33), lib)


def pin_fd_sinkhorn_n6(lib=None):
    _check_fd(_sinkhorn_problem(1, 6, 4, 2, seed=34), lib)


def pin_fd_n8(lib=None):
    _check_fd(problem(T=1, n=8, D=4, gamma=True, x_post=False, seed=3), lib)


def pin_fd_n4_f16(lib=None):
    p = problem(T=2, n=4, D=8, gamma=True, x_post=True, seed=31, f16=True)
    # the inputs use fp16's extra significand bits: read as bf16 they would be other numbers
    assert np.any(p["x_bits"] & 0x7) and np.any(p["ghin_bits"] & 0x7)
    _check_fd(p, lib)


def pin_f16_grad_x_rounding(lib=None):
    # gradX is returned once rounded to fp16: numpy's float64 -> float16 conversion rounds
    # to nearest, ties to even
    p = problem(T=3, n=4, D=8, gamma=True, x_post=True, seed=32, f16=True)
    r = backward(p, lib=lib)
    want = r.grad_x.astype(np.float16).view(np.uint16)
    assert np.array_equal(r.grad_x_bits, want), "gradX's fp16 bits are not the nearest fp16"
    # and in bf16 mode the bits are within half a bf16 ulp of the value
    q = problem(T=3, n=4, D=8, gamma=True, x_post=True, seed=32)
    rq = backward(q, lib=lib)
    got = bf16_bits_to_f32(rq.grad_x_bits).astype(np.float64)
    lo = np.abs(rq.grad_x - got) <= np.abs(rq.grad_x) * 2.0 ** -8   # half an ulp: 2^-8 of the leading power of two at most
    assert np.all(lo), "gradX's bf16 bits are not within half a bf16 ulp"


def pin_forward64_matches_forward(lib=None):
    p = problem(T=5, n=4, D=16, gamma=True, seed=4)
    f = forward64(p, lib=lib)
    r = oracle.forward(p["x_bits"], p["phi"], p["alpha"], p["bias"], p["gamma"], num_iters=1)
    _close(f.inv_rms, r.inv_rms, 1e-14, what="invRms")
    _close(f.h_mix, r.h_mix, 1e-13, 1e-14, what="hMix")
    _close(f.h_pre, r.h_pre, 1e-14, what="hPre")
    _close(f.h_post, r.h_post, 1e-14, what="hPost")
    _close(f.h_in, r.h_in, 1e-13, 1e-14, what="hIn")
    n = 4
    want = (np.float64(p["alpha"][2]) * f.h_mix[:, 2 * n:] * f.inv_rms[:, None]
            + p["bias"][2 * n:].astype(np.float64)).reshape(-1, n, n)
    _close(f.h_res, want, 1e-15, 1e-15, what="hRes = alpha2 pRes + bias")


def pin_alpha_zero(lib=None):
    p = problem(T=4, n=4, D=8, gamma=True, x_post=True, seed=5)
    p["alpha"] = np.zeros(3, np.float32)
    f = forward64(p, lib=lib)
    r = backward(p, fwd=f, lib=lib)
    assert np.all(r.grad_phi == 0.0) and np.all(r.grad_gamma == 0.0), "no gradient reaches hMix"
    want = p["ghin"][:, None, :] * f.h_pre.astype(np.float32).astype(np.float64)[:, :, None] + p["gxp"]
    assert np.array_equal(r.grad_x, want), "gradX = gradHIn * hPre + gradXPost"
    # alpha gradients: sum of g2 * w over the branch (w = hMix * invRms)
    inv = f.inv_rms.astype(np.float32).astype(np.float64)
    hm = f.h_mix.astype(np.float32).astype(np.float64)
    w = hm * inv[:, None]
    hp = f.h_pre.astype(np.float32).astype(np.float64) - EPS
    ghp = np.einsum("td,tid->ti", p["ghin"], p["x"])
    g2pre = ghp * hp * (1 - hp)
    hq = f.h_post.astype(np.float32).astype(np.float64)
    g2post = p["ghpost"].astype(np.float64) * hq * (1 - hq / 2)
    _close(r.grad_alpha, [np.sum(g2pre * w[:, :4]), np.sum(g2post * w[:, 4:8]),
                          np.sum(p["ghres"].reshape(-1, 16) * w[:, 8:])], 1e-12, 1e-14, what="gradAlpha")
    _close(r.grad_bias, np.concatenate([g2pre.sum(0), g2post.sum(0), p["ghres"].astype(np.float64).reshape(-1, 16).sum(0)]),
           1e-12, 1e-14, what="gradBias")


def pin_page_example(lib=None):
    # MhcPreBackward guide, section 7: T = 1024, N = 4, D = 512, every input 1.0
    # (x, phi, alpha, gradHIn, gradHPost, gradHRes, invRms, hMix, hPre, hPost, gamma),
    # gradXPost 0. By hand: s = 1 - eps, g2pre = D s (1 - s) per pre entry; g2post =
    # 1 * 1 * (1 - 1/2) = 1/2; the res entries pass gradHRes = 1. With alpha = invRms =
    # hMix = phi = gamma = 1, gHMix = gW = (g2pre x4, 1/2 x4, 1 x16) and
    # G = sum gW = 4 g2pre + 2 + 16 is both the invRms gradient and (gHMix . phi)[k].
    # gradX = gradHIn hPre + G gamma - G invRms^3 x / (n D) = 1 + G - G / 2048;
    # gradPhi[m][k] = T gW[m]; gradGamma[k] = T G; gradAlpha = T (4 g2pre, 4 / 2, 16);
    # gradBias = T gW.
    T, n, D = 1024, 4, 512
    M, K = 24, 2048
    one = np.ones
    x_bits = f32_to_bf16_bits(one((T, n, D), np.float32))
    r = oracle.backward(x_bits, one((M, K), np.float32), one(3, np.float32),
                        f32_to_bf16_bits(one((T, D), np.float32)), one((T, n), np.float32),
                        one((T, n, n), np.float32), one(T, np.float32), one((T, M), np.float32),
                        one((T, n), np.float32), one((T, n), np.float32), one((n, D), np.float32),
                        f32_to_bf16_bits(np.zeros((T, n, D), np.float32)), tokens=[0, 511, 1023],
                        lib=lib)
    s = 1.0 - EPS
    g2pre = D * s * (1 - s)
    gw = np.array([g2pre] * 4 + [0.5] * 4 + [1.0] * 16)
    G = gw.sum()
    _close(r.grad_x, np.full((3, n, D), 1.0 + G - G / K), 1e-13, what="gradX")
    _close(r.grad_phi, np.repeat(T * gw[:, None], K, axis=1), 1e-13, what="gradPhi")
    _close(r.grad_gamma, np.full((n, D), T * G), 1e-13, what="gradGamma")
    _close(r.grad_alpha, [T * 4 * g2pre, T * 2.0, T * 16.0], 1e-12, what="gradAlpha")
    _close(r.grad_bias, T * gw, 1e-12, what="gradBias")


def pin_abs_sums(lib=None):
    p = problem(T=6, n=4, D=8, gamma=True, x_post=True, seed=6)
    r = backward(p, lib=lib)
    for v, a, what in ((r.grad_x, r.grad_x_abs, "gradX"), (r.grad_phi, r.grad_phi_abs, "gradPhi"),
                       (r.grad_alpha, r.grad_alpha_abs, "gradAlpha"),
                       (r.grad_bias, r.grad_bias_abs, "gradBias"),
                       (r.grad_gamma, r.grad_gamma_abs, "gradGamma")):
        assert np.all(a >= np.abs(v) * (1 - 1e-15)), f"{what}: |sum| <= sum |terms|"
    # all terms non-negative: x > 0, gradients of hMix > 0 (alpha > 0, only gradHRes > 0)
    q = problem(T=3, n=4, D=8, gamma=False, x_post=False, seed=7)
    q["x_bits"], q["x"] = _bf16(np.abs(q["x"]) + 0.25)
    q["ghin_bits"], q["ghin"] = _bf16(np.zeros_like(q["ghin"]))
    q["ghpost"] = np.zeros_like(q["ghpost"])
    q["ghres"] = np.abs(q["ghres"]) + 0.1
    r = backward(q, lib=lib)
    _close(r.grad_phi_abs, r.grad_phi, 1e-15, what="gradPhi with non-negative terms")


def pin_token_subset(lib=None):
    p = problem(T=7, n=4, D=8, gamma=True, x_post=True, seed=8)
    f = forward64(p, lib=lib)
    full = backward(p, fwd=f, lib=lib)
    sub = backward(p, fwd=f, lib=lib, tokens=[6, 0, 3])
    assert np.array_equal(sub.grad_x, full.grad_x[[6, 0, 3]]), "gradX rows follow the token list"
    assert np.array_equal(sub.grad_phi, full.grad_phi), "gradPhi sums over all tokens"


def _sinkhorn_problem(T, n, D, it, seed, gamma=True):
    p = problem(T=T, n=n, D=D, gamma=gamma, x_post=False, seed=seed)
    p["num_iters"] = it
    return p


def pin_fd_sinkhorn_n4(lib=None):
    _check_fd(_sinkhorn_problem(2, 4, 8, 3, seed=21), lib)


def pin_fd_sinkhorn_n4_20_iters(lib=None):
    _check_fd(_sinkhorn_problem(1, 4, 8, 20, seed=22, gamma=False), lib)


def pin_fd_sinkhorn_n8(lib=None):
    _check_fd(_sinkhorn_problem(1, 8, 4, 2, seed=23), lib)


def pin_fd_sinkhorn_one_iter(lib=None):
    _check_fd(_sinkhorn_problem(2, 4, 8, 1, seed=24), lib)


def pin_sinkhorn_forward64_matches_forward(lib=None):
    p = _sinkhorn_problem(5, 4, 16, 4, seed=25)
    f = forward64(p, lib=lib)
    r = oracle.forward(p["x_bits"], p["phi"], p["alpha"], p["bias"], p["gamma"], num_iters=4)
    _close(f.h_res, r.h_res, 1e-13, 1e-15, what="hRes (Sinkhorn)")
    _close(f.sum_out, r.sum_out, 1e-13, 1e-15, what="sumOut")
    _close(f.norm_out, r.norm_out, 1e-13, 1e-15, what="normOut")


def pin_sinkhorn_logit_gradient_row_sums(lib=None):
    # one token, no other gradient reaching the res logits: gradBias[2n:] is the logit
    # gradient, and a constant added to a row of logits leaves every plane unchanged
    p = _sinkhorn_problem(1, 4, 8, 5, seed=26)
    r = backward(p, lib=lib)
    g = r.grad_bias[8:].reshape(4, 4)
    scale = float(np.max(np.abs(g)))
    assert scale > 1e-3, "the test needs a non-trivial logit gradient"
    _close(g.sum(axis=1), np.zeros(4), 0.0, 1e-6 * scale, what="row sums of the logit gradient")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
