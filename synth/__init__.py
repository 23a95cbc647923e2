"""Seeded synthetic inputs for the mHC pre-mapping forward.

Shared by the tests, the smoke check and the benchmark, and by both sides of
every comparison (the HIP library and the CPU oracle). It holds no step of the
method itself: only random draws and the float32 -> bf16 conversion that turns
drawn activations into the bf16 tensor the operator consumes.

Recipe (per workload, NumPy PCG64 seeded with ``seed``), tensors drawn in this
order, each in C order:
  x       [T, n, D]  float32 N(0, 1), then rounded to bf16 (nearest, ties to even), or
                     to binary16 for an fp16 workload (NumPy's float16 conversion);
                     drawn in chunks of ``X_CHUNK`` values (the stream is identical
                     to a single draw, the chunking only bounds host memory)
  phi     [M, n*D]   float32 N(0, 1) / sqrt(n*D)   (std 1/sqrt(n*D): mixes stay O(1))
  gamma   [n, D]     float32 U(0.5, 1.5)            (only when the workload has gamma)
  alpha   [3] or [2] float32 U(0.5, 1.5)
  bias    [M]        float32 N(0, 0.1)               (0.1 is the standard deviation)
  pre_mix [T, n]     float32 U(0, 1)                 (only when the workload has pre_mix)
with M = n*n + 2n for a 3-entry alpha and 2n for a 2-entry alpha.

MhcPre backward inputs (``backward_inputs``; M = n*n + 2n), drawn in this order:
  x            [T, n, D]  N(0, 1) -> bf16 (chunked as above)
  phi          [M, n*D]   N(0, 1) / sqrt(n*D)
  alpha        [3]        U(0.5, 1.5)
  grad_h_in    [T, D]     N(0, 1) -> bf16
  grad_h_post  [T, n]     N(0, 1)
  grad_h_res   [T, n, n]  N(0, 1)
  inv_rms      [T]        U(0.5, 1.5)
  h_mix        [T, M]     N(0, 1)
  h_pre        [T, n]     U(0, 1) + 1e-6   (the range of sigmoid + hcEps)
  h_post       [T, n]     U(0, 2)          (the range of 2 sigmoid)
  gamma        [n, D]     U(0.5, 1.5)      (when asked for)
  grad_x_post  [T, n, D]  N(0, 1) -> bf16  (when asked for)
  (x_f16: x, grad_h_in and grad_x_post rounded to binary16 instead, as for the forward)
  sum_out      [2 it, T, n]     U(0.9, 1.1)    (when Sinkhorn planes are asked for)
  norm_out     [2 it, T, n, n]  U(0.05, 0.45)
hc_post inputs (``post_inputs``), drawn in this order:
  x         [T, D]     N(0, 1) -> bf16   (the layer output)
  residual  [T, n, D]  N(0, 1) -> bf16   (the n streams; chunked as above)
  post      [T, n]     U(0, 2)           (the range of 2 sigmoid)
  comb      [T, n, n]  U(0.05, 0.45)     (the range of the Sinkhorn matrix entries at n = 4)
Standalone-stage inputs (``stage_inputs``: invRms alone and the Sinkhorn stage from given
mixes), drawn in this order:
  x         [T, n, D]  N(0, 1) -> bf16 (chunked as above)
  alpha     [3] or [2] U(0.5, 1.5)
  bias      [M]        N(0, 0.1)
  h_mix     [T, M]     N(0, 1)         (mixes of O(1), as phi's scaling gives the forward)
  inv_rms   [T]        U(0.5, 1.5)     (x ~ N(0, 1) gives invRms near 1)
  pre_mix   [T, n]     U(0, 1)         (when asked for)
The saved forward values are drawn independently, in the ranges the forward produces:
the backward is a function of all of them, whatever forward they came from. (Parity
tests of the Sinkhorn backward take the planes from the oracle's forward instead, so
that they are consistent; the benchmark only needs their ranges.)
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

X_CHUNK = 1 << 24


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    NaN stays NaN (quiet); values that round past the largest bf16 become inf.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    name: str
    T: int
    n: int
    D: int
    n_alpha: int = 3
    gamma: bool = False
    pre_mix: bool = False
    need_backward: bool = False
    num_iters: int = 20
    norm_eps: float = 1e-6
    hc_eps: float = 1e-6
    seed: int = 0
    note: str = ""
    x_f16: bool = False     # x (and hIn) in binary16 instead of bf16

    @property
    def M(self) -> int:
        return self.n * self.n + 2 * self.n if self.n_alpha == 3 else 2 * self.n

    @property
    def K(self) -> int:
        return self.n * self.D


# The five measured workloads: a tiny prefill, a mid-size prefill with gamma, a large
# training prefill with the backward intermediates, decode-size T, and a wide n = 8
# stream set with alpha[2] and an external pre_mix (seeds 1001..1005).
WORKLOADS = {
    "tiny": Workload("tiny", T=128, n=4, D=256, seed=1001,
                     note="T=128, n=4, D=256, no gamma, needBackward=false"),
    "mid_prefill": Workload("mid_prefill", T=4096, n=4, D=4096, gamma=True, seed=1002,
                            note="T=4096 (b=1, s=4096), n=4, D=4096, gamma [4, 4096]"),
    "large_prefill_bwd": Workload("large_prefill_bwd", T=16384, n=4, D=7168,
                                  need_backward=True, seed=1003,
                                  note="T=16384 (b=4, s=4096), n=4, D=7168, needBackward=true"),
    "decode": Workload("decode", T=64, n=4, D=7168, seed=1004,
                       note="T=64, n=4, D=7168, 1000 back-to-back launches"),
    "wide_premix": Workload("wide_premix", T=32768, n=8, D=2048, n_alpha=2, pre_mix=True,
                            seed=1005,
                            note="T=32768, n=8, D=2048, alpha[2], external pre_mix [T, 8]"),
}


@dataclass
class Inputs:
    wl: Workload
    x: np.ndarray            # uint16 bf16 bits [T, n, D]
    phi: np.ndarray          # float32 [M, n*D]
    alpha: np.ndarray        # float32 [n_alpha]
    bias: np.ndarray         # float32 [M]
    gamma: np.ndarray | None = None    # float32 [n, D]
    pre_mix: np.ndarray | None = None  # float32 [T, n]
    extra: dict = field(default_factory=dict)


def generate(wl: Workload, seed: int | None = None) -> Inputs:
    """Draw one workload's inputs with the recipe in the module docstring."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    total = wl.T * wl.n * wl.D
    x = np.empty(total, dtype=np.uint16)
    for start in range(0, total, X_CHUNK):
        stop = min(total, start + X_CHUNK)
        v = rng.standard_normal(stop - start, dtype=np.float32)
        x[start:stop] = v.astype(np.float16).view(np.uint16) if wl.x_f16 else f32_to_bf16_bits(v)
    x = x.reshape(wl.T, wl.n, wl.D)
    K = wl.K
    phi = (rng.standard_normal((wl.M, K), dtype=np.float32) / np.float32(np.sqrt(K))).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, size=(wl.n, wl.D)).astype(np.float32) if wl.gamma else None
    alpha = rng.uniform(0.5, 1.5, size=(wl.n_alpha,)).astype(np.float32)
    bias = (rng.standard_normal(wl.M) * 0.1).astype(np.float32)
    pre_mix = rng.uniform(0.0, 1.0, size=(wl.T, wl.n)).astype(np.float32) if wl.pre_mix else None
    return Inputs(wl, x, phi, alpha, bias, gamma, pre_mix)


def custom(T: int, n: int, D: int, *, n_alpha: int = 3, gamma: bool = False,
           pre_mix: bool = False, need_backward: bool = False, num_iters: int = 20,
           seed: int = 7, name: str = "custom", x_f16: bool = False) -> Inputs:
    """Same distributions at any shape (test sizes: tails, page example shapes)."""
    wl = Workload(name, T=T, n=n, D=D, n_alpha=n_alpha, gamma=gamma, pre_mix=pre_mix,
                  need_backward=need_backward, num_iters=num_iters, seed=seed, x_f16=x_f16)
    return generate(wl)


def _x16_normal(rng, count: int, f16: bool = False) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16)
    for start in range(0, count, X_CHUNK):
        stop = min(count, start + X_CHUNK)
        v = rng.standard_normal(stop - start, dtype=np.float32)
        out[start:stop] = v.astype(np.float16).view(np.uint16) if f16 else f32_to_bf16_bits(v)
    return out


@dataclass
class BwdInputs:
    T: int
    n: int
    D: int
    x: np.ndarray              # uint16 bf16 bits [T, n, D]
    phi: np.ndarray            # float32 [M, n*D]
    alpha: np.ndarray          # float32 [3]
    grad_h_in: np.ndarray      # uint16 bf16 bits [T, D]
    grad_h_post: np.ndarray    # float32 [T, n]
    grad_h_res: np.ndarray     # float32 [T, n, n]
    inv_rms: np.ndarray        # float32 [T]
    h_mix: np.ndarray          # float32 [T, M]
    h_pre: np.ndarray          # float32 [T, n]
    h_post: np.ndarray         # float32 [T, n]
    gamma: np.ndarray | None = None        # float32 [n, D]
    grad_x_post: np.ndarray | None = None  # uint16 bf16 bits [T, n, D]
    hc_eps: float = 1e-6
    num_iters: int = 0                     # >= 1: Sinkhorn planes below
    sum_out: np.ndarray | None = None      # float32 [2 it, T, n]
    norm_out: np.ndarray | None = None     # float32 [2 it, T, n, n]
    x_f16: bool = False                    # x, grad_h_in, grad_x_post as binary16 bits

    @property
    def M(self) -> int:
        return self.n * self.n + 2 * self.n


def backward_inputs(T: int, n: int, D: int, *, gamma: bool = False, x_post: bool = False,
                    sinkhorn_iters: int = 0, seed: int = 11, x_f16: bool = False) -> BwdInputs:
    """Inputs of the MhcPre backward with the recipe in the module docstring."""
    rng = np.random.default_rng(seed)
    M, K = n * n + 2 * n, n * D
    x = _x16_normal(rng, T * K, x_f16).reshape(T, n, D)
    phi = (rng.standard_normal((M, K), dtype=np.float32) / np.float32(np.sqrt(K))).astype(np.float32)
    alpha = rng.uniform(0.5, 1.5, size=3).astype(np.float32)
    ghin = _x16_normal(rng, T * D, x_f16).reshape(T, D)
    ghpost = rng.standard_normal((T, n), dtype=np.float32)
    ghres = rng.standard_normal((T, n, n), dtype=np.float32)
    inv = rng.uniform(0.5, 1.5, size=T).astype(np.float32)
    hmix = rng.standard_normal((T, M), dtype=np.float32)
    hpre = (rng.uniform(0.0, 1.0, size=(T, n)) + 1e-6).astype(np.float32)
    hpost = rng.uniform(0.0, 2.0, size=(T, n)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, size=(n, D)).astype(np.float32) if gamma else None
    gxp = _x16_normal(rng, T * K, x_f16).reshape(T, n, D) if x_post else None
    bi = BwdInputs(T, n, D, x, phi, alpha, ghin, ghpost, ghres, inv, hmix, hpre, hpost, g, gxp,
                   x_f16=x_f16)
    if sinkhorn_iters:
        bi.num_iters = sinkhorn_iters
        bi.sum_out = rng.uniform(0.9, 1.1, size=(2 * sinkhorn_iters, T, n)).astype(np.float32)
        bi.norm_out = rng.uniform(0.05, 0.45, size=(2 * sinkhorn_iters, T, n, n)).astype(np.float32)
    return bi


@dataclass
class PostInputs:
    T: int
    n: int
    D: int
    x: np.ndarray          # uint16 [T, D] bf16 bits
    residual: np.ndarray   # uint16 [T, n, D] bf16 bits
    post: np.ndarray       # float32 [T, n]
    comb: np.ndarray       # float32 [T, n, n]


def post_inputs(T: int, n: int, D: int, *, seed: int = 21) -> PostInputs:
    """Inputs of hc_post with the recipe in the module docstring."""
    rng = np.random.default_rng(seed)
    x = _x16_normal(rng, T * D).reshape(T, D)
    residual = _x16_normal(rng, T * n * D).reshape(T, n, D)
    post = rng.uniform(0.0, 2.0, size=(T, n)).astype(np.float32)
    comb = rng.uniform(0.05, 0.45, size=(T, n, n)).astype(np.float32)
    return PostInputs(T, n, D, x, residual, post, comb)


@dataclass
class StageInputs:
    T: int
    n: int
    D: int
    n_alpha: int
    x: np.ndarray          # uint16 [T, n, D] bf16 bits
    alpha: np.ndarray      # float32 [n_alpha]
    bias: np.ndarray       # float32 [M]
    h_mix: np.ndarray      # float32 [T, M]
    inv_rms: np.ndarray    # float32 [T]
    pre_mix: np.ndarray | None = None   # float32 [T, n]

    @property
    def M(self) -> int:
        return self.n * self.n + 2 * self.n if self.n_alpha == 3 else 2 * self.n


def stage_inputs(T: int, n: int, D: int, *, n_alpha: int = 3, pre_mix: bool = False,
                 seed: int = 31, x_f16: bool = False) -> StageInputs:
    """Inputs of the standalone stages with the recipe in the module docstring (x_f16: x
    rounded to binary16 instead of bf16)."""
    rng = np.random.default_rng(seed)
    M = n * n + 2 * n if n_alpha == 3 else 2 * n
    if x_f16:
        x = rng.standard_normal(T * n * D, dtype=np.float32).astype(np.float16).view(np.uint16).reshape(T, n, D)
    else:
        x = _x16_normal(rng, T * n * D).reshape(T, n, D)
    alpha = rng.uniform(0.5, 1.5, size=n_alpha).astype(np.float32)
    bias = (0.1 * rng.standard_normal(M)).astype(np.float32)
    hmix = rng.standard_normal((T, M), dtype=np.float32)
    inv = rng.uniform(0.5, 1.5, size=T).astype(np.float32)
    pm = rng.uniform(0.0, 1.0, size=(T, n)).astype(np.float32) if pre_mix else None
    return StageInputs(T, n, D, n_alpha, x, alpha, bias, hmix, inv, pm)
