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
_LIB = os.path.join(_HERE, "libmhc_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP). Returns the .so path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("n", ctypes.c_int32), ("D", ctypes.c_int32),
                ("n_alpha", ctypes.c_int32), ("num_iters", ctypes.c_int32),
                ("norm_eps", ctypes.c_double), ("hc_eps", ctypes.c_double)]


class _Out(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("inv_rms", "h_mix", "h_pre", "h_post", "h_res", "sum_out",
                 "norm_out", "h_in", "h_in_bf16")]


def _bind(lib):
    lib.oracle_pre_forward.restype = ctypes.c_int
    lib.oracle_pre_forward.argtypes = [
        ctypes.POINTER(_Cfg), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.POINTER(_Out), ctypes.c_int]
    lib.oracle_bf16_from_double.restype = ctypes.c_uint16
    lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_max_threads.restype = ctypes.c_int
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
            want_sinkhorn_steps=True, nthreads=0, lib=None) -> OracleResult:
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
    cfg = _Cfg(T, n, D, n_alpha, int(num_iters), float(norm_eps), float(hc_eps))
    rc = (lib or _load()).oracle_pre_forward(
        ctypes.byref(cfg), _ptr(x_bits), _ptr(phi), _ptr(alpha), _ptr(bias), _ptr(gamma),
        _ptr(pre_mix), _ptr(tok), ntok, ctypes.byref(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem description")
    return res
