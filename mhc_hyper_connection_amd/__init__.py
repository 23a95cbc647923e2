"""Fused mHC pre-mapping forward for AMD Instinct MI355X (gfx950).

Python face of the C-ABI library libmhc.so (include/mhc.h). Per token it computes
invRms, the projection hMix = (x * gamma) . phi^T, the sigmoid pre/post gates, a
2*numIters-step Sinkhorn of the n x n residual block and the collapse
hIn = sum_i weight_i * x_i (aclnnMhcPreV2 guide, kwkr.cn/news/422178, section 3;
aclnnMhcPreSinkhorn guide, m.mzlw.cn/news/197063, section 3.2; HcPre guide,
mhpn.cn/news/2282827, function prototype for pre_mix).

PyTorch is used for device memory and the current HIP stream only; the work runs in
the library's kernels, and nothing here falls back to another implementation.
"""
from __future__ import annotations

import math

from ._binding import (FORWARD_EVENTS, MHC_ERR_NULLPTR, MHC_ERR_PARAM_INVALID,
                       MHC_ERR_RUNTIME, MHC_OK, STAGES, MhcError, Params, bwd_workspace_size,
                       forward_path, raw_inv_rms, raw_post, raw_sinkhorn,
                       load, make_bwd_params, make_params, packed_size, raw_backward,
                       raw_forward, raw_forward_noalloc, raw_forward_timed, raw_prepack, raw_wait_status,
                       status_string,
                       version, workspace_size)

__all__ = ["PreForward", "PreBackward", "mhc_pre", "mhc_pre_backward", "mhc_post", "mhc_pre_inv_rms",
           "mhc_pre_sinkhorn", "prepack", "version",
           "status_string", "MhcError", "FORWARD_EVENTS", "STAGES",
           "make_params", "packed_size", "workspace_size", "load",
           "MHC_OK", "MHC_ERR_NULLPTR", "MHC_ERR_PARAM_INVALID", "MHC_ERR_RUNTIME"]


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    # torch's current stream on `device` as a raw handle (the direct getter: a fraction of
    # the cost of building a torch.cuda.Stream object on every call)
    torch = _torch()
    getter = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if getter is not None and device.index is not None:
        return ctypes_void(getter(device.index))
    return ctypes_void(torch.cuda.current_stream(device).cuda_stream)


def ctypes_void(handle):
    import ctypes
    return ctypes.c_void_p(handle) if handle else None


def _check(t, name, dtype, shape, device):
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.shape != shape:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.get_device() != (device.index if device.type == "cuda" else -1):
        raise ValueError(f"{name} is on {t.device}, expected {device}")


class PreForward:
    """Launcher for one problem size. Owns the workspace the library needs.

    Calls issued through one instance must not overlap (they share the workspace);
    calls on one stream are ordered by the stream and are safe.
    """

    def __init__(self, T, n, D, n_alpha=3, *, num_iters=20, norm_eps=1e-6, hc_eps=1e-6,
                 need_backward=False, device="cuda", x_f16=False):
        torch = _torch()
        load()
        self.T, self.n, self.D, self.n_alpha = int(T), int(n), int(D), int(n_alpha)
        self.num_iters = int(num_iters)
        self.need_backward = bool(need_backward)
        self.M = n * n + 2 * n if n_alpha == 3 else 2 * n
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.x_f16 = bool(x_f16)
        self.xdt = torch.float16 if self.x_f16 else torch.bfloat16   # x and hIn
        self.params = make_params(T, n, D, n_alpha, num_iters, norm_eps, hc_eps, need_backward, self.x_f16)
        self.ws_bytes = workspace_size(self.params)
        self.packed_bytes = packed_size(self.params)
        # zero-filled once: its first bytes hold the call counter the library keeps
        self.workspace = torch.zeros(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)

    def path(self, has_pre_mix=False):
        """2 when calls take the one-launch kernel on this device, 1 the single-read kernel,
        0 the classic path."""
        return forward_path(self.params, has_pre_mix)

    def wait_status(self):
        """mhc_pre_wait_status on this launcher's workspace: 1 if a wait of the single-read
        or one-launch kernel gave up since the last query (its tokens then hold NaN), else 0. Synchronises the current
        stream; clears the flag."""
        return raw_wait_status(_ptr(self.workspace), self.workspace.numel(), _stream(self.device))

    # -- outputs -----------------------------------------------------------------------
    def alloc_outputs(self, *, intermediates=None):
        """torch.empty outputs. intermediates: None (what need_backward requires),
        True (all of them) or False (only hIn, hPost, hRes)."""
        torch = _torch()
        T, n, D, M, dev = self.T, self.n, self.D, self.M, self.device
        f32 = dict(dtype=torch.float32, device=dev)
        want = self.need_backward if intermediates is None else bool(intermediates)
        out = {"h_in": torch.empty((T, D), dtype=self.xdt, device=dev),
               "h_post": torch.empty((T, n), **f32),
               "h_res": torch.empty((T, n, n), **f32)}
        if want:
            out["inv_rms"] = torch.empty((T,), **f32)
            out["h_mix"] = torch.empty((T, M), **f32)
            out["h_pre"] = torch.empty((T, n), **f32)
            if self.n_alpha == 3:
                out["sum_out"] = torch.empty((2 * self.num_iters, T, n), **f32)
                out["norm_out"] = torch.empty((2 * self.num_iters, T, n, n), **f32)
        return out

    def _check_out(self, out):
        # every tensor the library writes: known name, dtype, shape, device, contiguous
        torch = _torch()
        T, n, D, M = self.T, self.n, self.D, self.M
        it = self.num_iters
        want = {"h_in": (self.xdt, (T, D)), "h_post": (torch.float32, (T, n)),
                "h_res": (torch.float32, (T, n, n)), "inv_rms": (torch.float32, (T,)),
                "h_mix": (torch.float32, (T, M)), "h_pre": (torch.float32, (T, n)),
                "sum_out": (torch.float32, (2 * it, T, n)), "norm_out": (torch.float32, (2 * it, T, n, n))}
        unknown = set(out) - set(want)
        if unknown:
            raise ValueError(f"out: unknown outputs {sorted(unknown)}")
        for k in ("h_in", "h_post", "h_res"):
            if out.get(k) is None:
                raise ValueError(f"out[{k!r}] is required")
        for k, v in out.items():
            _check(v, k, *want[k], self.device)

    # -- weights -----------------------------------------------------------------------
    def prepack(self, phi, gamma=None, out=None):
        torch = _torch()
        _check(phi, "phi", torch.float32, (self.M, self.n * self.D), self.device)
        _check(gamma, "gamma", torch.float32, (self.n, self.D), self.device)
        if out is None:
            out = torch.empty(self.packed_bytes, dtype=torch.uint8, device=self.device)
        st = raw_prepack(self.params, _ptr(phi), _ptr(gamma), _ptr(out), out.numel(),
                         _stream(self.device))
        if st != MHC_OK:
            raise MhcError(st, "mhc_pre_prepack")
        return out

    # -- forward -----------------------------------------------------------------------
    def __call__(self, x, phi, alpha, bias, gamma=None, pre_mix=None, *, phi_packed=None,
                 out=None, events=None, noalloc=False):
        """events: optional list of FORWARD_EVENTS torch.cuda.Event(enable_timing=True) or
        None, each event recorded at least once before (so that its HIP event exists); the
        call then records them around its kernels (STAGES order) and skips the None
        entries, see mhc_pre_forward_timed. noalloc: call mhc_pre_forward_noalloc instead
        (the library's per-GPU scratch array as workspace; no events)."""
        torch = _torch()
        T, n, D, M, dev = self.T, self.n, self.D, self.M, self.device
        _check(x, "x", self.xdt, (T, n, D), dev)
        if phi_packed is None:
            _check(phi, "phi", torch.float32, (M, n * D), dev)
        _check(alpha, "alpha", torch.float32, (self.n_alpha,), dev)
        _check(bias, "bias", torch.float32, (M,), dev)
        _check(gamma, "gamma", torch.float32, (n, D), dev)
        _check(pre_mix, "pre_mix", torch.float32, (T, n), dev)
        if phi_packed is not None:
            if phi_packed.dtype != torch.uint8 or phi_packed.numel() < self.packed_bytes:
                raise ValueError(f"phi_packed: uint8 of at least {self.packed_bytes} bytes expected "
                                 "(mhc_pre_prepack's output)")
            _check(phi_packed, "phi_packed", torch.uint8, tuple(phi_packed.shape), dev)
        if out is None:
            out = self.alloc_outputs()
        else:
            self._check_out(out)
        ptrs = {"x": _ptr(x), "phi": _ptr(phi), "alpha": _ptr(alpha), "bias": _ptr(bias),
                "gamma": _ptr(gamma), "pre_mix": _ptr(pre_mix), "phi_packed": _ptr(phi_packed)}
        for k, v in out.items():
            ptrs[k] = _ptr(v)
        if noalloc:
            st = raw_forward_noalloc(self.params, ptrs, _stream(dev))
            if st != MHC_OK:
                raise MhcError(st, "mhc_pre_forward_noalloc")
        elif events is None:
            st = raw_forward(self.params, ptrs, _ptr(self.workspace), self.ws_bytes,
                             _stream(dev))
            if st != MHC_OK:
                raise MhcError(st, "mhc_pre_forward")
        else:
            st = raw_forward_timed(self.params, ptrs, _ptr(self.workspace), self.ws_bytes,
                                   _stream(dev),
                                   [None if e is None else (e.cuda_event or None) for e in events])
            if st != MHC_OK:
                raise MhcError(st, "mhc_pre_forward_timed")
        return out


_RUNNERS: dict = {}


def _runner(T, n, D, n_alpha, num_iters, norm_eps, hc_eps, need_backward, device, x_f16=False):
    key = (T, n, D, n_alpha, num_iters, norm_eps, hc_eps, need_backward, str(device), x_f16)
    r = _RUNNERS.get(key)
    if r is None:
        r = PreForward(T, n, D, n_alpha, num_iters=num_iters, norm_eps=norm_eps, hc_eps=hc_eps,
                       need_backward=need_backward, device=device, x_f16=x_f16)
        _RUNNERS[key] = r
    return r


def prepack(phi, gamma=None, *, n, n_alpha=3):
    """Pack static weights once; pass the result as phi_packed to mhc_pre."""
    D = phi.shape[1] // n
    return _runner(1, n, D, n_alpha, 20, 1e-6, 1e-6, False, phi.device).prepack(phi, gamma)


def mhc_pre(x, phi, alpha, bias, gamma=None, pre_mix=None, *, num_iters=20, norm_eps=1e-6,
            hc_eps=1e-6, need_backward=False, phi_packed=None):
    """Fused pre-mapping forward. x: bf16 or fp16 [T, n, D] or [B, S, n, D]; hIn takes x's dtype.

    Returns (h_in, h_post, h_res, extras); extras holds inv_rms, h_mix, h_pre, sum_out
    and norm_out when need_backward is set. Shapes follow x's leading dimensions.
    """
    lead = tuple(x.shape[:-2])
    n, D = int(x.shape[-2]), int(x.shape[-1])
    T = math.prod(lead) if lead else 1
    n_alpha = int(alpha.shape[0])
    r = _runner(T, n, D, n_alpha, num_iters, norm_eps, hc_eps, need_backward, x.device,
                x.dtype == _torch().float16)
    xf = x.reshape(T, n, D)
    pm = None if pre_mix is None else pre_mix.reshape(T, n)
    out = r(xf, phi, alpha, bias, gamma, pm, phi_packed=phi_packed)
    h_in = out.pop("h_in").reshape(*lead, D)
    h_post = out.pop("h_post").reshape(*lead, n)
    h_res = out.pop("h_res").reshape(*lead, n, n)
    extras = {}
    for k, v in out.items():
        if k in ("sum_out", "norm_out"):
            extras[k] = v.reshape(v.shape[0], *lead, *v.shape[2:])
        elif k == "inv_rms":
            extras[k] = v.reshape(*lead)
        else:
            extras[k] = v.reshape(*lead, v.shape[-1])
    return h_in, h_post, h_res, extras


class PreBackward:
    """Launcher of the MhcPre backward for one problem size (MhcPreBackward guide,
    0539edu.com/news/4871844, section 3); with num_iters >= 1 the MhcPreSinkhorn backward
    (the forward's Sinkhorn planes are then inputs). x_f16: x, grad_h_in, grad_x_post
    and grad_x in float16 (else bfloat16). Owns its workspace; calls through one
    instance must not overlap."""

    def __init__(self, T, n, D, *, hc_eps=1e-6, num_iters=0, x_f16=False, device="cuda"):
        torch = _torch()
        load()
        self.T, self.n, self.D = int(T), int(n), int(D)
        self.M = n * n + 2 * n
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.num_iters = int(num_iters)
        self.x_f16 = bool(x_f16)
        self.params = make_bwd_params(T, n, D, hc_eps, num_iters, self.x_f16)
        self.ws_bytes = bwd_workspace_size(self.params)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)

    def alloc_outputs(self, gamma=False):
        torch = _torch()
        T, n, D, M, dev = self.T, self.n, self.D, self.M, self.device
        f32 = dict(dtype=torch.float32, device=dev)
        x16 = torch.float16 if self.x_f16 else torch.bfloat16
        out = {"grad_x": torch.empty((T, n, D), dtype=x16, device=dev),
               "grad_phi": torch.empty((M, n * D), **f32), "grad_alpha": torch.empty((3,), **f32),
               "grad_bias": torch.empty((M,), **f32)}
        if gamma:
            out["grad_gamma"] = torch.empty((n, D), **f32)
        return out

    def __call__(self, x, phi, alpha, grad_h_in, grad_h_post, grad_h_res, inv_rms, h_mix, h_pre,
                 h_post, gamma=None, grad_x_post=None, *, sum_out=None, norm_out=None, out=None):
        torch = _torch()
        T, n, D, M, dev = self.T, self.n, self.D, self.M, self.device
        bf = torch.float16 if self.x_f16 else torch.bfloat16
        f32 = torch.float32
        for t, name, dt, shape in ((x, "x", bf, (T, n, D)), (phi, "phi", f32, (M, n * D)),
                                   (alpha, "alpha", f32, (3,)), (grad_h_in, "grad_h_in", bf, (T, D)),
                                   (grad_h_post, "grad_h_post", f32, (T, n)),
                                   (grad_h_res, "grad_h_res", f32, (T, n, n)),
                                   (inv_rms, "inv_rms", f32, (T,)), (h_mix, "h_mix", f32, (T, M)),
                                   (h_pre, "h_pre", f32, (T, n)), (h_post, "h_post", f32, (T, n)),
                                   (gamma, "gamma", f32, (n, D)),
                                   (grad_x_post, "grad_x_post", bf, (T, n, D))):
            _check(t, name, dt, shape, dev)
        it = self.num_iters
        if it:
            if sum_out is None or norm_out is None:
                raise ValueError("num_iters >= 1 needs the forward's sum_out and norm_out")
            _check(sum_out, "sum_out", f32, (2 * it, T, n), dev)
            _check(norm_out, "norm_out", f32, (2 * it, T, n, n), dev)
        if out is None:
            out = self.alloc_outputs(gamma is not None)
        else:
            want = {"grad_x": (bf, (T, n, D)), "grad_phi": (f32, (M, n * D)), "grad_alpha": (f32, (3,)),
                    "grad_bias": (f32, (M,))}
            if gamma is not None:
                want["grad_gamma"] = (f32, (n, D))
            if set(out) != set(want):
                raise ValueError(f"out must hold exactly {sorted(want)}")
            for k, (dt, shape) in want.items():
                _check(out[k], k, dt, shape, dev)
        ptrs = {"x": _ptr(x), "phi": _ptr(phi), "alpha": _ptr(alpha), "grad_h_in": _ptr(grad_h_in),
                "grad_h_post": _ptr(grad_h_post), "grad_h_res": _ptr(grad_h_res),
                "inv_rms": _ptr(inv_rms), "h_mix": _ptr(h_mix), "h_pre": _ptr(h_pre),
                "h_post": _ptr(h_post), "gamma": _ptr(gamma), "grad_x_post": _ptr(grad_x_post),
                "sum_out": _ptr(sum_out) if it else None, "norm_out": _ptr(norm_out) if it else None}
        for k, v in out.items():
            ptrs[k] = _ptr(v)
        st = raw_backward(self.params, ptrs, _ptr(self.workspace), self.ws_bytes, _stream(dev))
        if st != MHC_OK:
            raise MhcError(st, "mhc_pre_backward")
        return out


_BWD_RUNNERS: dict = {}


def mhc_pre_backward(x, phi, alpha, grad_h_in, grad_h_post, grad_h_res, inv_rms, h_mix, h_pre,
                     h_post, gamma=None, grad_x_post=None, *, hc_eps=1e-6, num_iters=0,
                     sum_out=None, norm_out=None):
    """MhcPre backward (num_iters == 0) or MhcPreSinkhorn backward (num_iters >= 1, with
    the forward's sum_out [2it, ..., n] and norm_out [2it, ..., n, n]). x: bf16 or fp16
    [T, n, D] or [B, S, n, D] (grad_h_in, grad_x_post and the returned grad_x in the same
    format); the other per-token tensors follow x's leading dimensions. Returns dict
    grad_x, grad_phi, grad_alpha, grad_bias (and grad_gamma when gamma is given)."""
    lead = tuple(x.shape[:-2])
    n, D = int(x.shape[-2]), int(x.shape[-1])
    T = math.prod(lead) if lead else 1
    f16 = x.dtype == _torch().float16
    key = (T, n, D, hc_eps, num_iters, f16, str(x.device))
    r = _BWD_RUNNERS.get(key)
    if r is None:
        r = _BWD_RUNNERS[key] = PreBackward(T, n, D, hc_eps=hc_eps, num_iters=num_iters,
                                            x_f16=f16, device=x.device)
    M = n * n + 2 * n
    rs = lambda t, *shape: None if t is None else t.reshape(*shape)
    out = r(x.reshape(T, n, D), phi, alpha, rs(grad_h_in, T, D), rs(grad_h_post, T, n),
            rs(grad_h_res, T, n, n), rs(inv_rms, T), rs(h_mix, T, M), rs(h_pre, T, n),
            rs(h_post, T, n), gamma, rs(grad_x_post, T, n, D),
            sum_out=rs(sum_out, 2 * num_iters, T, n), norm_out=rs(norm_out, 2 * num_iters, T, n, n))
    out["grad_x"] = out["grad_x"].reshape(*lead, n, D)
    return out


def mhc_post(x, residual, post, comb, *, out=None):
    """hc_post: out[t, j, d] = post[t, j] x[t, d] + sum_i comb[t, i, j] residual[t, i, d]
    (the HcPre guide's broadcast expression on its 4-D comb: the sum is over comb's first index).
    x [T, D] and residual [T, n, D] both bf16 or both fp16, post f32 [T, n], comb f32
    [T, n, n] on one device; returns (or fills) [T, n, D] in x's dtype. The stream is
    torch's current stream."""
    torch = _torch()
    T, n, D = residual.shape
    dev = residual.device
    xdt = torch.float16 if residual.dtype == torch.float16 else torch.bfloat16
    _check(x, "x", xdt, (T, D), dev)
    _check(residual, "residual", xdt, (T, n, D), dev)
    _check(post, "post", torch.float32, (T, n), dev)
    _check(comb, "comb", torch.float32, (T, n, n), dev)
    if out is None:
        out = torch.empty((T, n, D), dtype=xdt, device=dev)
    _check(out, "out", xdt, (T, n, D), dev)
    st = raw_post(T, n, D, _ptr(x), _ptr(residual), _ptr(post), _ptr(comb), _ptr(out), _stream(dev),
                  xdt == torch.float16)
    if st != MHC_OK:
        raise MhcError(st, "mhc_post")
    return out


def mhc_pre_inv_rms(x, *, norm_eps=1e-6):
    """invRms alone: x bf16 or fp16 [T, n, D] -> f32 [T] on x's device and torch's current stream."""
    torch = _torch()
    T, n, D = x.shape
    f16 = x.dtype == torch.float16
    _check(x, "x", torch.float16 if f16 else torch.bfloat16, (T, n, D), x.device)
    out = torch.empty((T,), dtype=torch.float32, device=x.device)
    params = make_params(T, n, D, norm_eps=norm_eps, x_f16=f16)
    st = raw_inv_rms(params, _ptr(x), _ptr(out), _stream(x.device))
    if st != MHC_OK:
        raise MhcError(st, "mhc_pre_inv_rms")
    return out


def mhc_pre_sinkhorn(x, h_mix, inv_rms, alpha, bias, pre_mix=None, *, num_iters=20, hc_eps=1e-6,
                     need_backward=False):
    """The Sinkhorn stage alone, from given mixes h_mix f32 [T, M] and inv_rms f32 [T]
    with x bf16 or fp16 [T, n, D] (hIn in the same dtype). Returns (h_in, h_pre, h_post, h_res, extras); extras holds
    sum_out and norm_out when need_backward is set and alpha has 3 entries."""
    torch = _torch()
    T, n, D = x.shape
    dev = x.device
    n_alpha = int(alpha.shape[0])
    M = n * n + 2 * n if n_alpha == 3 else 2 * n
    xdt = torch.float16 if x.dtype == torch.float16 else torch.bfloat16
    _check(x, "x", xdt, (T, n, D), dev)
    _check(h_mix, "h_mix", torch.float32, (T, M), dev)
    _check(inv_rms, "inv_rms", torch.float32, (T,), dev)
    _check(alpha, "alpha", torch.float32, (n_alpha,), dev)
    _check(bias, "bias", torch.float32, (M,), dev)
    if pre_mix is not None:
        _check(pre_mix, "pre_mix", torch.float32, (T, n), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"h_in": torch.empty((T, D), dtype=xdt, device=dev),
           "h_pre": torch.empty((T, n), **f32), "h_post": torch.empty((T, n), **f32),
           "h_res": torch.empty((T, n, n), **f32)}
    extras = {}
    if need_backward and n_alpha == 3:
        extras["sum_out"] = torch.empty((2 * num_iters, T, n), **f32)
        extras["norm_out"] = torch.empty((2 * num_iters, T, n, n), **f32)
    params = make_params(T, n, D, n_alpha=n_alpha, num_iters=num_iters, hc_eps=hc_eps,
                         need_backward=need_backward, x_f16=xdt == torch.float16)
    ptrs = {"x": _ptr(x), "h_mix": _ptr(h_mix), "inv_rms": _ptr(inv_rms), "alpha": _ptr(alpha),
            "bias": _ptr(bias), "pre_mix": None if pre_mix is None else _ptr(pre_mix)}
    ptrs.update({k: _ptr(v) for k, v in out.items()})
    ptrs.update({k: _ptr(v) for k, v in extras.items()})
    st = raw_sinkhorn(params, ptrs, _stream(dev))
    if st != MHC_OK:
        raise MhcError(st, "mhc_pre_sinkhorn")
    return out["h_in"], out["h_pre"], out["h_post"], out["h_res"], extras
