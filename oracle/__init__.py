"""fp64 CPU oracle of the mHC pre-mapping forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product library never does, and this
package imports nothing from the product package.

The arithmetic lives in ``mhc_oracle.c`` (plain C, fp64, one token at a time,
OpenMP over tokens). This module only builds it with gcc and marshals numpy
arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mhc_oracle.c")
_SRC_BWD = os.path.join(_HERE, "mhc_oracle_bwd.c")
_SRC_POST = os.path.join(_HERE, "mhc_oracle_post.c")
_LIB = os.path.join(_HERE, "libmhc_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP). Returns the .so path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, _SRC_BWD, _SRC_POST, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("n", ctypes.c_int32), ("D", ctypes.c_int32),
                ("n_alpha", ctypes.c_int32), ("num_iters", ctypes.c_int32),
                ("norm_eps", ctypes.c_double), ("hc_eps", ctypes.c_double),
                ("x_f16", ctypes.c_int32)]


class _Out(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("inv_rms", "h_mix", "h_pre", "h_post", "h_res", "sum_out",
                 "norm_out", "h_in", "h_in_bf16")]


class _BwdIn(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("n", ctypes.c_int32), ("D", ctypes.c_int32),
                ("hc_eps", ctypes.c_double)] + [
        (name, ctypes.c_void_p) for name in
        ("x", "phi", "alpha", "grad_h_in", "grad_h_post", "grad_h_res", "inv_rms",
         "h_mix", "h_pre", "h_post", "gamma", "grad_x_post")] + [
        ("num_iters", ctypes.c_int32), ("sum_out", ctypes.c_void_p), ("norm_out", ctypes.c_void_p),
        ("x_f16", ctypes.c_int32)]


class _BwdOut(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("grad_x", "grad_x_bits", "grad_x_abs", "grad_phi", "grad_phi_abs",
                 "grad_alpha", "grad_alpha_abs", "grad_bias", "grad_bias_abs",
                 "grad_gamma", "grad_gamma_abs", "g_mix")]


def _bind(lib):
    lib.oracle_pre_forward.restype = ctypes.c_int
    lib.oracle_pre_forward.argtypes = [
        ctypes.POINTER(_Cfg), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.POINTER(_Out), ctypes.c_int]
    lib.oracle_bf16_from_double.restype = ctypes.c_uint16
    lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
    if hasattr(lib, "oracle_f16_from_double"):
        lib.oracle_f16_from_double.restype = ctypes.c_uint16
        lib.oracle_f16_from_double.argtypes = [ctypes.c_double]
        lib.oracle_f16_to_double.restype = ctypes.c_double
        lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_max_threads.restype = ctypes.c_int
    dp = ctypes.c_void_p
    lib.oracle_mhcpre_forward_f64.restype = ctypes.c_int
    lib.oracle_mhcpre_forward_f64.argtypes = [
        ctypes.c_int64, ctypes.c_int, ctypes.c_int, dp, dp, dp, dp, dp,
        ctypes.c_double, ctypes.c_double, ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp]
    if hasattr(lib, "oracle_mhc_post"):   # builds of altered copies may leave it out
        lib.oracle_mhc_post.restype = ctypes.c_int
        lib.oracle_mhc_post.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, dp, dp, dp, dp,
                                        dp, dp, dp]
    if hasattr(lib, "oracle_mhc_post_fmt"):
        lib.oracle_mhc_post_fmt.restype = ctypes.c_int
        lib.oracle_mhc_post_fmt.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, dp, dp, dp, dp,
                                            dp, dp, dp, ctypes.c_int]
    if hasattr(lib, "oracle_pre_sinkhorn"):
        lib.oracle_inv_rms.restype = ctypes.c_int
        lib.oracle_inv_rms.argtypes = [ctypes.POINTER(_Cfg), dp, dp, ctypes.c_int]
        lib.oracle_pre_sinkhorn.restype = ctypes.c_int
        lib.oracle_pre_sinkhorn.argtypes = [ctypes.POINTER(_Cfg), dp, dp, dp, dp, dp, dp,
                                            ctypes.POINTER(_Out), ctypes.c_int]
    lib.oracle_pre_backward.restype = ctypes.c_int
    lib.oracle_pre_backward.argtypes = [ctypes.POINTER(_BwdIn), dp, ctypes.c_int64,
                                        ctypes.POINTER(_BwdOut), ctypes.c_int]
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def load_library(path: str):
    """Bind another build of mhc_oracle.c (the mutation tests compile altered copies)."""
    return _bind(ctypes.CDLL(os.path.abspath(path)))


def bf16_from_double(v: float, lib=None) -> int:
    """Nearest bf16 (ties to even) of a double, as 16 raw bits."""
    return int((lib or _load()).oracle_bf16_from_double(float(v)))


def f16_from_double(v: float, lib=None) -> int:
    """Nearest binary16 (ties to even) of a double, as 16 raw bits."""
    return int((lib or _load()).oracle_f16_from_double(float(v)))


def f16_to_double(bits: int, lib=None) -> float:
    return float((lib or _load()).oracle_f16_to_double(int(bits) & 0xFFFF))


def bf16_to_double(bits: int, lib=None) -> float:
    return float((lib or _load()).oracle_bf16_to_double(int(bits) & 0xFFFF))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data


@dataclass
class OracleResult:
    inv_rms: np.ndarray
    h_mix: np.ndarray
    h_pre: np.ndarray
    h_post: np.ndarray
    h_res: np.ndarray
    sum_out: np.ndarray | None
    norm_out: np.ndarray | None
    h_in: np.ndarray
    h_in_bf16: np.ndarray


def forward(x_bits, phi, alpha, bias, gamma=None, pre_mix=None, *, num_iters=20,
            norm_eps=1e-6, hc_eps=1e-6, tokens=None, want_h_in=True,
            want_sinkhorn_steps=True, nthreads=0, x_f16=False, lib=None) -> OracleResult:
    """Run the oracle.

    x_bits: uint16 bf16 bit patterns, shape [T, n, D]. phi: float32 [M, n*D].
    alpha: float32 [3] or [2]. bias: float32 [M]. gamma: float32 [n, D] or None.
    pre_mix: float32 [T, n] or None. tokens: optional int64 list of token indices;
    results are returned for those tokens, in that order. All results are float64
    (h_in_bf16 is uint16 bits), Sinkhorn planes step-major [2*it, ntok, ...].
    """
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 3:
        raise ValueError("x must be [T, n, D]")
    T, n, D = x_bits.shape
    alpha = np.ascontiguousarray(alpha, dtype=np.float32).reshape(-1)
    n_alpha = int(alpha.shape[0])
    M = n * n + 2 * n if n_alpha == 3 else 2 * n
    phi = np.ascontiguousarray(phi, dtype=np.float32)
    bias = np.ascontiguousarray(bias, dtype=np.float32).reshape(-1)
    if phi.shape != (M, n * D) or bias.shape != (M,):
        raise ValueError(f"phi must be [{M}, {n * D}] and bias [{M}]")
    if gamma is not None:
        gamma = np.ascontiguousarray(gamma, dtype=np.float32).reshape(n, D)
    if pre_mix is not None:
        pre_mix = np.ascontiguousarray(pre_mix, dtype=np.float32).reshape(T, n)
    if tokens is None:
        tok = None
        ntok = T
    else:
        tok = np.ascontiguousarray(tokens, dtype=np.int64).reshape(-1)
        ntok = int(tok.shape[0])

    steps = 2 * num_iters if n_alpha == 3 else 0
    res = OracleResult(
        inv_rms=np.empty(ntok), h_mix=np.empty((ntok, M)), h_pre=np.empty((ntok, n)),
        h_post=np.empty((ntok, n)), h_res=np.empty((ntok, n, n)),
        sum_out=np.empty((steps, ntok, n)) if (steps and want_sinkhorn_steps) else None,
        norm_out=np.empty((steps, ntok, n, n)) if (steps and want_sinkhorn_steps) else None,
        h_in=np.empty((ntok, D)) if want_h_in else None,
        h_in_bf16=np.empty((ntok, D), dtype=np.uint16) if want_h_in else None)
    out = _Out(*[_ptr(getattr(res, f)) for f, _ in _Out._fields_])
    cfg = _Cfg(T, n, D, n_alpha, int(num_iters), float(norm_eps), float(hc_eps), int(bool(x_f16)))
    rc = (lib or _load()).oracle_pre_forward(
        ctypes.byref(cfg), _ptr(x_bits), _ptr(phi), _ptr(alpha), _ptr(bias), _ptr(gamma),
        _ptr(pre_mix), _ptr(tok), ntok, ctypes.byref(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem description")
    return res


def inv_rms(x_bits, *, norm_eps=1e-6, nthreads=0, x_f16=False, lib=None) -> np.ndarray:
    """invRms alone: x_bits uint16 bf16 bits [T, n, D] -> float64 [T]."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 3:
        raise ValueError("x must be [T, n, D]")
    T, n, D = x_bits.shape
    out = np.empty(T)
    cfg = _Cfg(T, n, D, 3, 1, float(norm_eps), 0.0, int(bool(x_f16)))
    if (lib or _load()).oracle_inv_rms(ctypes.byref(cfg), _ptr(x_bits), _ptr(out), int(nthreads)) != 0:
        raise ValueError("oracle rejected the problem description")
    return out


def pre_sinkhorn(x_bits, h_mix, inv_rms_in, alpha, bias, pre_mix=None, *, num_iters=20,
                 hc_eps=1e-6, want_sinkhorn_steps=True, nthreads=0, x_f16=False, lib=None) -> OracleResult:
    """The Sinkhorn stage alone: from given mixes h_mix [T, M] and invRms [T] (converted
    to float64 exactly) and x [T, n, D] to hPre, hPost, hRes, the Sinkhorn planes and hIn.
    The result's inv_rms and h_mix fields echo the inputs."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 3:
        raise ValueError("x must be [T, n, D]")
    T, n, D = x_bits.shape
    alpha = np.ascontiguousarray(alpha, dtype=np.float32).reshape(-1)
    n_alpha = int(alpha.shape[0])
    M = n * n + 2 * n if n_alpha == 3 else 2 * n
    bias = np.ascontiguousarray(bias, dtype=np.float32).reshape(-1)
    h_mix = np.ascontiguousarray(h_mix, dtype=np.float64).reshape(T, M)
    inv_in = np.ascontiguousarray(inv_rms_in, dtype=np.float64).reshape(T)
    if bias.shape != (M,):
        raise ValueError(f"bias must be [{M}]")
    if pre_mix is not None:
        pre_mix = np.ascontiguousarray(pre_mix, dtype=np.float32).reshape(T, n)
    steps = 2 * num_iters if n_alpha == 3 else 0
    res = OracleResult(
        inv_rms=inv_in.copy(), h_mix=h_mix.copy(), h_pre=np.empty((T, n)),
        h_post=np.empty((T, n)), h_res=np.empty((T, n, n)),
        sum_out=np.empty((steps, T, n)) if (steps and want_sinkhorn_steps) else None,
        norm_out=np.empty((steps, T, n, n)) if (steps and want_sinkhorn_steps) else None,
        h_in=np.empty((T, D)), h_in_bf16=np.empty((T, D), dtype=np.uint16))
    ptrs = {f: _ptr(getattr(res, f)) for f, _ in _Out._fields_}
    ptrs["inv_rms"] = ptrs["h_mix"] = None
    out = _Out(*[ptrs[f] for f, _ in _Out._fields_])
    cfg = _Cfg(T, n, D, n_alpha, int(num_iters), 1e-6, float(hc_eps), int(bool(x_f16)))
    rc = (lib or _load()).oracle_pre_sinkhorn(
        ctypes.byref(cfg), _ptr(x_bits), _ptr(h_mix), _ptr(inv_in), _ptr(alpha), _ptr(bias),
        _ptr(pre_mix), ctypes.byref(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem description")
    return res


@dataclass
class MhcPreF64:
    inv_rms: np.ndarray
    h_mix: np.ndarray
    h_pre: np.ndarray
    h_post: np.ndarray
    h_res: np.ndarray
    h_in: np.ndarray
    sum_out: np.ndarray | None = None
    norm_out: np.ndarray | None = None


def mhcpre_forward_f64(x, phi, alpha, bias, gamma=None, *, norm_eps=1e-6, hc_eps=1e-6,
                       num_iters=0, lib=None) -> MhcPreF64:
    """The forward on float64 inputs: the function whose gradient ``backward`` returns.
    num_iters == 0: MhcPre (affine hRes); >= 1: MhcPreSinkhorn (hRes the Sinkhorn of it,
    with the sum_out / norm_out planes). x: [T, n, D]; phi: [n*n + 2n, n*D]; alpha: [3];
    bias: [n*n + 2n]; gamma: [n, D] or None. All results float64, hIn unrounded."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    T, n, D = x.shape
    M = n * n + 2 * n
    phi = np.ascontiguousarray(phi, dtype=np.float64).reshape(M, n * D)
    alpha = np.ascontiguousarray(alpha, dtype=np.float64).reshape(3)
    bias = np.ascontiguousarray(bias, dtype=np.float64).reshape(M)
    if gamma is not None:
        gamma = np.ascontiguousarray(gamma, dtype=np.float64).reshape(n, D)
    steps = 2 * int(num_iters)
    r = MhcPreF64(np.empty(T), np.empty((T, M)), np.empty((T, n)), np.empty((T, n)),
                  np.empty((T, n, n)), np.empty((T, D)),
                  np.empty((steps, T, n)) if steps else None,
                  np.empty((steps, T, n, n)) if steps else None)
    rc = (lib or _load()).oracle_mhcpre_forward_f64(
        T, n, D, _ptr(x), _ptr(phi), _ptr(alpha), _ptr(bias), _ptr(gamma),
        float(norm_eps), float(hc_eps), int(num_iters), _ptr(r.inv_rms), _ptr(r.h_mix),
        _ptr(r.h_pre), _ptr(r.h_post), _ptr(r.h_res), _ptr(r.h_in), _ptr(r.sum_out),
        _ptr(r.norm_out))
    if rc != 0:
        raise ValueError("oracle rejected the problem description")
    return r


@dataclass
class BackwardResult:
    grad_x: np.ndarray        # [ntok, n, D] float64, unrounded
    grad_x_bits: np.ndarray   # [ntok, n, D] bits of x's format (bf16, or fp16 with x_f16)
    grad_x_abs: np.ndarray    # sum of |terms| per gradX element
    grad_phi: np.ndarray      # [M, n*D]
    grad_phi_abs: np.ndarray
    grad_alpha: np.ndarray    # [3]
    grad_alpha_abs: np.ndarray
    grad_bias: np.ndarray     # [M]
    grad_bias_abs: np.ndarray
    grad_gamma: np.ndarray | None
    grad_gamma_abs: np.ndarray | None
    g_mix: np.ndarray         # [T, M]: gradient with respect to hMix


def backward(x_bits, phi, alpha, grad_h_in_bits, grad_h_post, grad_h_res, inv_rms, h_mix,
             h_pre, h_post, gamma=None, grad_x_post_bits=None, *, hc_eps=1e-6, tokens=None,
             num_iters=0, sum_out=None, norm_out=None, nthreads=0, x_f16=False, lib=None) -> BackwardResult:
    """The MhcPre backward in fp64 from the inputs the GPU receives: x, gradHIn and
    gradXPost as bf16 bits (fp16 bits with x_f16: gradX then rounds to fp16, the
    MhcPreBackward guide's section 8.2 giving gradX gradHIn's type); phi [n*n + 2n, n*D], alpha [3], gradHPost [T, n],
    gradHRes [T, n, n], invRms [T], hMix [T, M], hPre [T, n], hPost [T, n], gamma [n, D]
    as float32. gradX rows are returned for ``tokens`` (default: all); every other
    gradient sums over all tokens. num_iters >= 1: the MhcPreSinkhorn backward, reading
    the forward's saved planes sum_out [2it, T, n] and norm_out [2it, T, n, n] (float32)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, n, D = x_bits.shape
    M = n * n + 2 * n
    K = n * D
    f32 = lambda a, shape: np.ascontiguousarray(a, dtype=np.float32).reshape(shape)
    phi = f32(phi, (M, K))
    alpha = f32(alpha, (3,))
    ghin = np.ascontiguousarray(grad_h_in_bits, dtype=np.uint16).reshape(T, D)
    ghpost = f32(grad_h_post, (T, n))
    ghres = f32(grad_h_res, (T, n, n))
    inv_rms = f32(inv_rms, (T,))
    h_mix = f32(h_mix, (T, M))
    h_pre = f32(h_pre, (T, n))
    h_post = f32(h_post, (T, n))
    if gamma is not None:
        gamma = f32(gamma, (n, D))
    if grad_x_post_bits is not None:
        grad_x_post_bits = np.ascontiguousarray(grad_x_post_bits, dtype=np.uint16).reshape(T, n, D)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64).reshape(-1)
    ntok = T if tok is None else int(tok.shape[0])
    g = gamma is not None
    r = BackwardResult(
        np.empty((ntok, n, D)), np.empty((ntok, n, D), dtype=np.uint16), np.empty((ntok, n, D)),
        np.empty((M, K)), np.empty((M, K)), np.empty(3), np.empty(3), np.empty(M), np.empty(M),
        np.empty((n, D)) if g else None, np.empty((n, D)) if g else None, np.empty((T, M)))
    if num_iters:
        sum_out = f32(sum_out, (2 * num_iters, T, n))
        norm_out = f32(norm_out, (2 * num_iters, T, n, n))
    bin_ = _BwdIn(T, n, D, float(hc_eps), *[_ptr(a) for a in (
        x_bits, phi, alpha, ghin, ghpost, ghres, inv_rms, h_mix, h_pre, h_post, gamma,
        grad_x_post_bits)], int(num_iters), _ptr(sum_out) if num_iters else None,
        _ptr(norm_out) if num_iters else None, int(bool(x_f16)))
    bout = _BwdOut(*[_ptr(getattr(r, f)) for f, _ in _BwdOut._fields_])
    rc = (lib or _load()).oracle_pre_backward(ctypes.byref(bin_), _ptr(tok), ntok,
                                              ctypes.byref(bout), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem description")
    return r


@dataclass
class PostResult:
    out_bf16: np.ndarray   # uint16 [T, n, D]
    out: np.ndarray        # float64 [T, n, D], before rounding
    out_abs: np.ndarray    # float64 [T, n, D], sum of |terms|


def post(x_bits, residual_bits, post_w, comb, lib=None, x_f16=False) -> PostResult:
    """hc_post: out[t, j, d] = post[t, j] x[t, d] + sum_i comb[t, i, j] residual[t, i, d]
    (x [T, D] and residual [T, n, D] as bf16 bits, post [T, n], comb [T, n, n] float32):
    the HcPre guide's printed expression on its 4-D comb_frag, where the summed index is
    comb's first one."""
    lib = lib or _load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    residual_bits = np.ascontiguousarray(residual_bits, dtype=np.uint16)
    post_w = np.ascontiguousarray(post_w, dtype=np.float32)
    comb = np.ascontiguousarray(comb, dtype=np.float32)
    T, n, D = residual_bits.shape
    assert x_bits.shape == (T, D) and post_w.shape == (T, n) and comb.shape == (T, n, n)
    ob = np.zeros((T, n, D), dtype=np.uint16)
    o = np.zeros((T, n, D), dtype=np.float64)
    oa = np.zeros((T, n, D), dtype=np.float64)
    if x_f16:   # binary16 x, residual and out
        st = lib.oracle_mhc_post_fmt(T, n, D, _ptr(x_bits), _ptr(residual_bits), _ptr(post_w), _ptr(comb),
                                     _ptr(ob), _ptr(o), _ptr(oa), 1)
    else:
        st = lib.oracle_mhc_post(T, n, D, _ptr(x_bits), _ptr(residual_bits), _ptr(post_w), _ptr(comb),
                                 _ptr(ob), _ptr(o), _ptr(oa))
    if st != 0:
        raise ValueError(f"oracle_mhc_post status {st}")
    return PostResult(ob, o, oa)
