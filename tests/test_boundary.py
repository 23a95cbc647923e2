"""The C-ABI library on a host without a GPU: it loads, exports every declared
symbol, and its validation runs before any HIP call (no compute is launched here).

Error classes follow the aclnnMhcPreSinkhorn guide (m.mzlw.cn/news/197063), section 6:
161001 for a NULL required pointer, 161002 for invalid parameters, 361001 runtime.
"""
import ctypes
import os
import re

import pytest

from mhc_hyper_connection_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc.h")

FAKE = 0x10000            # 256-byte aligned, never dereferenced: every case returns first
WS_BIG = 1 << 40


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = B.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert B.version() == 10000


def test_status_strings():
    for st in (B.MHC_OK, B.MHC_ERR_NULLPTR, B.MHC_ERR_PARAM_INVALID, B.MHC_ERR_RUNTIME):
        assert B.status_string(st).startswith("MHC_")
    assert B.status_string(12345) == "unknown mhc_status"


def _p(**kw):
    base = dict(T=128, n=4, D=256, n_alpha=3, num_iters=20, norm_eps=1e-6, hc_eps=1e-6,
                need_backward=False)
    base.update(kw)
    return B.make_params(**base)


def _ptrs(**over):
    p = {f: FAKE for f in ("x", "phi", "alpha", "bias", "h_in", "h_post", "h_res")}
    p.update(over)
    return p


def fwd(params, ptrs=None, ws=FAKE, ws_bytes=WS_BIG):
    return B.raw_forward(params, _ptrs() if ptrs is None else ptrs, ws, ws_bytes, None)


def test_sizes():
    p = _p(T=16384, D=7168)
    packed = B.packed_size(p)
    # (224 d-blocks x 4 streams + 32 zero K-steps) x 4 octet rows x 80 columns x 16 bytes
    assert packed == (896 + 32) * 4 * 80 * 16
    ws = B.workspace_size(p)
    # packed weights, hIn weights, and 32 slices of partial records (8 + 20 floats per
    # token) for each of the 256 tiles
    assert ws >= packed + 16384 * 4 * 4 + 32 * 16384 * 28 * 4
    assert B.workspace_size(_p(T=0, D=7168)) >= packed


@pytest.mark.parametrize("field", ["x", "alpha", "bias", "h_in", "h_post", "h_res"])
def test_null_required_pointer(field):
    assert fwd(_p(), _ptrs(**{field: None})) == B.MHC_ERR_NULLPTR


def test_null_params_workspace_and_weights():
    lib = B.load()
    t = B.Tensors(*[_ptrs().get(f) for f in B.TENSOR_FIELDS])
    assert lib.mhc_pre_forward(None, ctypes.byref(t), FAKE, WS_BIG, None) == B.MHC_ERR_NULLPTR
    assert fwd(_p(), ws=None) == B.MHC_ERR_NULLPTR
    assert fwd(_p(), _ptrs(phi=None)) == B.MHC_ERR_NULLPTR
    # phi may be NULL when packed weights are given
    assert fwd(_p(T=0), _ptrs(phi=None, phi_packed=FAKE)) == B.MHC_OK
    # hRes may be NULL without the res branch
    assert fwd(_p(T=0, n_alpha=2), _ptrs(h_res=None)) == B.MHC_OK


@pytest.mark.parametrize("kw", [dict(n=5), dict(n=7), dict(n=2), dict(n=16), dict(D=0), dict(D=-8), dict(D=12),
                                dict(D=16392), dict(n=8, D=8200),
                                dict(n_alpha=4), dict(n_alpha=1), dict(num_iters=0),
                                dict(norm_eps=0.0), dict(norm_eps=float("nan")),
                                dict(hc_eps=-1e-6), dict(T=-1)])
def test_invalid_attributes(kw):
    assert fwd(_p(**kw)) == B.MHC_ERR_PARAM_INVALID


def test_x_dtype_and_need_backward_values():
    for bad in (2, -1, 7):
        p = _p()
        p.x_dtype = bad
        assert fwd(p) == B.MHC_ERR_PARAM_INVALID
    p = _p(T=0)
    p.x_dtype = B.DTYPE_F16
    assert fwd(p) == B.MHC_OK
    # fp16 never takes the single-read kernel
    path = ctypes.c_int32(-1)
    p = _p(T=1 << 16, D=7168)
    p.x_dtype = B.DTYPE_F16
    assert B.load().mhc_pre_forward_path(ctypes.byref(p), 0, ctypes.byref(path)) == B.MHC_OK
    assert path.value == 0
    p = _p()
    p.need_backward = 2
    assert fwd(p) == B.MHC_ERR_PARAM_INVALID


def test_need_backward_requires_intermediates():
    p = _p(need_backward=True)
    assert fwd(p) == B.MHC_ERR_PARAM_INVALID
    full = _ptrs(inv_rms=FAKE, h_mix=FAKE, h_pre=FAKE, sum_out=FAKE, norm_out=FAKE)
    assert fwd(_p(T=0, need_backward=True), full) == B.MHC_OK
    partial = dict(full)
    partial.pop("norm_out")
    assert fwd(p, partial) == B.MHC_ERR_PARAM_INVALID
    # without the res branch there are no Sinkhorn planes to ask for
    p2 = _p(T=0, n_alpha=2, need_backward=True)
    assert fwd(p2, _ptrs(inv_rms=FAKE, h_mix=FAKE, h_pre=FAKE)) == B.MHC_OK
    assert fwd(p2, _ptrs(inv_rms=FAKE, h_mix=FAKE, h_pre=FAKE, sum_out=FAKE)) == B.MHC_ERR_PARAM_INVALID


def test_optional_outputs_are_independent():
    # unlike an all-or-none group, any subset of the optional outputs is accepted
    assert fwd(_p(T=0), _ptrs(h_pre=FAKE)) == B.MHC_OK
    assert fwd(_p(T=0), _ptrs(inv_rms=FAKE, norm_out=FAKE)) == B.MHC_OK


def test_workspace_too_small_and_alignment():
    p = _p()
    need = B.workspace_size(p)
    assert fwd(p, ws_bytes=need - 1) == B.MHC_ERR_PARAM_INVALID
    assert fwd(p, _ptrs(x=FAKE + 8)) == B.MHC_ERR_PARAM_INVALID
    assert fwd(p, _ptrs(h_in=FAKE + 2)) == B.MHC_ERR_PARAM_INVALID
    assert fwd(p, ws=FAKE + 64) == B.MHC_ERR_PARAM_INVALID
    assert fwd(p, _ptrs(alpha=FAKE + 2)) == B.MHC_ERR_PARAM_INVALID


def test_empty_input_succeeds_without_launch():
    assert fwd(_p(T=0)) == B.MHC_OK


def test_prepack_validation():
    p = _p()
    need = B.packed_size(p)
    assert B.raw_prepack(p, None, None, FAKE, need, None) == B.MHC_ERR_NULLPTR
    assert B.raw_prepack(p, FAKE, None, None, need, None) == B.MHC_ERR_NULLPTR
    assert B.raw_prepack(p, FAKE, None, FAKE, need - 16, None) == B.MHC_ERR_PARAM_INVALID
    assert B.raw_prepack(_p(n=5), FAKE, None, FAKE, need, None) == B.MHC_ERR_PARAM_INVALID
    assert B.raw_prepack(p, FAKE, None, FAKE + 4, need, None) == B.MHC_ERR_PARAM_INVALID


def test_timed_forward_validates_events_first():
    lib = B.load()
    t = B.Tensors(*[_ptrs().get(f) for f in B.TENSOR_FIELDS])
    five = (ctypes.c_void_p * 5)(*([FAKE] * 5))
    # NULL array: NULLPTR; wrong count: PARAM_INVALID (NULL entries are boundaries the
    # caller does not want recorded)
    assert lib.mhc_pre_forward_timed(ctypes.byref(_p()), ctypes.byref(t), FAKE, WS_BIG, None,
                                     None, 5) == B.MHC_ERR_NULLPTR
    holes = (ctypes.c_void_p * 5)(FAKE, FAKE, None, FAKE, FAKE)
    assert lib.mhc_pre_forward_timed(ctypes.byref(_p()), ctypes.byref(t), FAKE, WS_BIG, None,
                                     holes, 4) == B.MHC_ERR_PARAM_INVALID
    assert lib.mhc_pre_forward_timed(ctypes.byref(_p()), ctypes.byref(t), FAKE, WS_BIG, None,
                                     five, 4) == B.MHC_ERR_PARAM_INVALID
    # then the forward's own validation, before any HIP call
    assert B.raw_forward_timed(_p(n=5), _ptrs(), FAKE, WS_BIG, None, [FAKE] * 5) == B.MHC_ERR_PARAM_INVALID
    assert B.raw_forward_timed(_p(), _ptrs(x=None), FAKE, WS_BIG, None, [FAKE] * 5) == B.MHC_ERR_NULLPTR


def test_wait_status_validation():
    # mhc_pre_wait_status rejects before any HIP call: NULL workspace or output, a workspace
    # smaller than its 256-byte head, a misaligned one
    lib = B.load()
    out = ctypes.c_int32(7)
    assert lib.mhc_pre_wait_status(None, 1 << 20, None, ctypes.byref(out)) == B.MHC_ERR_NULLPTR
    assert lib.mhc_pre_wait_status(ctypes.c_void_p(FAKE), 1 << 20, None, None) == B.MHC_ERR_NULLPTR
    assert lib.mhc_pre_wait_status(ctypes.c_void_p(FAKE), 255, None, ctypes.byref(out)) == B.MHC_ERR_PARAM_INVALID
    assert lib.mhc_pre_wait_status(ctypes.c_void_p(FAKE + 64), 1 << 20, None, ctypes.byref(out)) == B.MHC_ERR_PARAM_INVALID
    assert out.value == 7   # untouched on error


def test_noalloc_validation():
    # mhc_pre_forward_noalloc: NULL arguments, and a problem whose workspace exceeds the
    # library's 64 MiB array, are refused before any HIP call
    lib = B.load()
    assert lib.mhc_pre_forward_noalloc(None, None, None) == B.MHC_ERR_NULLPTR
    big = _p(T=65536, D=7168, need_backward=True)
    assert B.workspace_size(big) > (64 << 20)
    assert B.raw_forward_noalloc(big, _ptrs(), None) == B.MHC_ERR_PARAM_INVALID
    assert B.raw_forward_noalloc(_p(n=5), _ptrs(), None) == B.MHC_ERR_PARAM_INVALID
