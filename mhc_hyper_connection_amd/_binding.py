"""ctypes binding of libmhc.so (include/mhc.h). Argument marshalling only.

PyTorch supplies device memory (torch.empty / torch.zeros) and the HIP stream
(torch.cuda.current_stream); every step of the computation runs in the library's
HIP kernels. There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmhc.so")

MHC_OK = 0
MHC_ERR_NULLPTR = 161001
MHC_ERR_PARAM_INVALID = 161002
MHC_ERR_RUNTIME = 361001


class MhcError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class Params(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("n", ctypes.c_int32), ("D", ctypes.c_int32),
                ("n_alpha", ctypes.c_int32), ("num_iters", ctypes.c_int32),
                ("norm_eps", ctypes.c_double), ("hc_eps", ctypes.c_double),
                ("need_backward", ctypes.c_int32), ("x_dtype", ctypes.c_int32)]


TENSOR_FIELDS = ("x", "phi", "alpha", "bias", "gamma", "pre_mix", "phi_packed", "h_in",
                 "h_post", "h_res", "inv_rms", "h_mix", "h_pre", "sum_out", "norm_out")


class Tensors(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in TENSOR_FIELDS]


class BwdParams(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("n", ctypes.c_int32), ("D", ctypes.c_int32),
                ("hc_eps", ctypes.c_double), ("num_iters", ctypes.c_int32),
                ("x_f16", ctypes.c_int32)]


BWD_TENSOR_FIELDS = ("x", "phi", "alpha", "grad_h_in", "grad_h_post", "grad_h_res", "inv_rms",
                     "h_mix", "h_pre", "h_post", "gamma", "grad_x_post", "grad_x", "grad_phi",
                     "grad_alpha", "grad_bias", "grad_gamma", "sum_out", "norm_out")


class BwdTensors(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in BWD_TENSOR_FIELDS]


EXPORTS = ("mhc_version", "mhc_status_string", "mhc_pre_packed_size",
           "mhc_pre_workspace_size", "mhc_pre_prepack", "mhc_pre_forward",
           "mhc_pre_forward_timed", "mhc_pre_forward_path", "mhc_pre_backward_workspace_size",
           "mhc_pre_backward", "mhc_post", "mhc_pre_inv_rms", "mhc_pre_sinkhorn",
           "mhc_pre_wait_status", "mhc_pre_forward_noalloc")

# MHC_FORWARD_EVENTS: events of mhc_pre_forward_timed (before the first kernel, then one
# after each of pack, projection, epilogue, hIn)
FORWARD_EVENTS = 5
STAGES = ("pack", "projection", "epilogue", "hin")

_lib = None


class PostParams(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("n", ctypes.c_int32), ("D", ctypes.c_int32),
                ("x_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class PostTensors(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in ("x", "residual", "post", "comb", "out")]


SINKHORN_TENSOR_FIELDS = ("x", "h_mix", "inv_rms", "alpha", "bias", "pre_mix", "h_in", "h_pre",
                          "h_post", "h_res", "sum_out", "norm_out")


class SinkhornTensors(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in SINKHORN_TENSOR_FIELDS]


def load(path: str | None = None):
    """Load and bind libmhc.so. Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m mhc_hyper_connection_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(p)
    lib.mhc_version.restype = ctypes.c_int
    lib.mhc_version.argtypes = []
    lib.mhc_status_string.restype = ctypes.c_char_p
    lib.mhc_status_string.argtypes = [ctypes.c_int32]
    lib.mhc_pre_packed_size.restype = ctypes.c_int32
    lib.mhc_pre_packed_size.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(ctypes.c_size_t)]
    lib.mhc_pre_workspace_size.restype = ctypes.c_int32
    lib.mhc_pre_workspace_size.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(ctypes.c_size_t)]
    lib.mhc_pre_prepack.restype = ctypes.c_int32
    lib.mhc_pre_prepack.argtypes = [ctypes.POINTER(Params), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mhc_pre_forward.restype = ctypes.c_int32
    lib.mhc_pre_forward.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(Tensors),
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mhc_pre_forward_timed.restype = ctypes.c_int32
    lib.mhc_pre_forward_timed.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(Tensors),
                                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]
    lib.mhc_pre_backward_workspace_size.restype = ctypes.c_int32
    lib.mhc_pre_backward_workspace_size.argtypes = [ctypes.POINTER(BwdParams), ctypes.POINTER(ctypes.c_size_t)]
    lib.mhc_pre_backward.restype = ctypes.c_int32
    lib.mhc_post.restype = ctypes.c_int32
    lib.mhc_post.argtypes = [ctypes.POINTER(PostParams), ctypes.POINTER(PostTensors), ctypes.c_void_p]
    lib.mhc_pre_inv_rms.restype = ctypes.c_int32
    lib.mhc_pre_inv_rms.argtypes = [ctypes.POINTER(Params), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.mhc_pre_sinkhorn.restype = ctypes.c_int32
    lib.mhc_pre_sinkhorn.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(SinkhornTensors), ctypes.c_void_p]
    lib.mhc_pre_forward_path.restype = ctypes.c_int32
    lib.mhc_pre_forward_path.argtypes = [ctypes.POINTER(Params), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.mhc_pre_forward_noalloc.restype = ctypes.c_int32
    lib.mhc_pre_forward_noalloc.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(Tensors), ctypes.c_void_p]
    lib.mhc_pre_wait_status.restype = ctypes.c_int32
    lib.mhc_pre_wait_status.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.POINTER(ctypes.c_int32)]
    lib.mhc_pre_backward.argtypes = [ctypes.POINTER(BwdParams), ctypes.POINTER(BwdTensors),
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    if path is None:
        _lib = lib
    return lib


def version() -> int:
    return int(load().mhc_version())


def status_string(status: int) -> str:
    return load().mhc_status_string(int(status)).decode()


DTYPE_BF16, DTYPE_F16 = 0, 1


def make_params(T, n, D, n_alpha=3, num_iters=20, norm_eps=1e-6, hc_eps=1e-6,
                need_backward=False, x_f16=False) -> Params:
    return Params(int(T), int(n), int(D), int(n_alpha), int(num_iters), float(norm_eps),
                  float(hc_eps), int(bool(need_backward)), DTYPE_F16 if x_f16 else DTYPE_BF16)


def packed_size(params: Params) -> int:
    out = ctypes.c_size_t(0)
    st = load().mhc_pre_packed_size(ctypes.byref(params), ctypes.byref(out))
    if st != MHC_OK:
        raise MhcError(st, "mhc_pre_packed_size")
    return int(out.value)


def workspace_size(params: Params) -> int:
    out = ctypes.c_size_t(0)
    st = load().mhc_pre_workspace_size(ctypes.byref(params), ctypes.byref(out))
    if st != MHC_OK:
        raise MhcError(st, "mhc_pre_workspace_size")
    return int(out.value)


def forward_path(params: Params, has_pre_mix: bool) -> int:
    """mhc_pre_forward's path on the current device: 2 the one-launch kernel, 1 the
    single-read kernel, 0 the classic path."""
    out = ctypes.c_int32(0)
    st = load().mhc_pre_forward_path(ctypes.byref(params), int(bool(has_pre_mix)), ctypes.byref(out))
    if st != MHC_OK:
        raise MhcError(st, "mhc_pre_forward_path")
    return int(out.value)


def raw_prepack(params: Params, phi_ptr, gamma_ptr, packed_ptr, packed_bytes, stream) -> int:
    return int(load().mhc_pre_prepack(ctypes.byref(params), phi_ptr, gamma_ptr, packed_ptr,
                                      packed_bytes, stream))


def raw_forward(params: Params, ptrs: dict, ws_ptr, ws_bytes, stream) -> int:
    t = Tensors(*[ptrs.get(f) for f in TENSOR_FIELDS])
    return int(load().mhc_pre_forward(ctypes.byref(params), ctypes.byref(t), ws_ptr, ws_bytes, stream))


def raw_forward_timed(params: Params, ptrs: dict, ws_ptr, ws_bytes, stream, events) -> int:
    """events: sequence of raw hipEvent_t handles (ints or None)."""
    t = Tensors(*[ptrs.get(f) for f in TENSOR_FIELDS])
    arr = (ctypes.c_void_p * max(len(events), 1))(*events)
    return int(load().mhc_pre_forward_timed(ctypes.byref(params), ctypes.byref(t), ws_ptr, ws_bytes,
                                            stream, arr, len(events)))


def make_bwd_params(T, n, D, hc_eps=1e-6, num_iters=0, x_f16=False) -> BwdParams:
    return BwdParams(int(T), int(n), int(D), float(hc_eps), int(num_iters), int(bool(x_f16)))


def bwd_workspace_size(params: BwdParams) -> int:
    out = ctypes.c_size_t(0)
    st = load().mhc_pre_backward_workspace_size(ctypes.byref(params), ctypes.byref(out))
    if st != MHC_OK:
        raise MhcError(st, "mhc_pre_backward_workspace_size")
    return int(out.value)


def raw_backward(params: BwdParams, ptrs: dict, ws_ptr, ws_bytes, stream) -> int:
    t = BwdTensors(*[ptrs.get(f) for f in BWD_TENSOR_FIELDS])
    return int(load().mhc_pre_backward(ctypes.byref(params), ctypes.byref(t), ws_ptr, ws_bytes, stream))


def raw_post(T, n, D, x_ptr, residual_ptr, post_ptr, comb_ptr, out_ptr, stream, x_f16=False) -> int:
    p = PostParams(int(T), int(n), int(D), 1 if x_f16 else 0, 0)
    t = PostTensors(x_ptr, residual_ptr, post_ptr, comb_ptr, out_ptr)
    return int(load().mhc_post(ctypes.byref(p), ctypes.byref(t), stream))


def raw_inv_rms(params: Params, x_ptr, inv_rms_ptr, stream) -> int:
    return int(load().mhc_pre_inv_rms(ctypes.byref(params), x_ptr, inv_rms_ptr, stream))


def raw_sinkhorn(params: Params, ptrs: dict, stream) -> int:
    t = SinkhornTensors(*[ptrs.get(f) for f in SINKHORN_TENSOR_FIELDS])
    return int(load().mhc_pre_sinkhorn(ctypes.byref(params), ctypes.byref(t), stream))


def raw_wait_status(ws_ptr, ws_bytes, stream) -> int:
    """mhc_pre_wait_status: 1 if a single-read wait gave up since the last query (clears it)."""
    out = ctypes.c_int32(0)
    st = load().mhc_pre_wait_status(ctypes.c_void_p(ws_ptr), ctypes.c_size_t(ws_bytes), stream,
                                    ctypes.byref(out))
    if st != MHC_OK:
        raise MhcError(st, "mhc_pre_wait_status")
    return int(out.value)


def raw_forward_noalloc(params: Params, ptrs: dict, stream) -> int:
    """mhc_pre_forward_noalloc: the forward with the library's per-GPU scratch array as workspace."""
    t = Tensors(*[ptrs.get(f) for f in TENSOR_FIELDS])
    return int(load().mhc_pre_forward_noalloc(ctypes.byref(params), ctypes.byref(t), stream))
