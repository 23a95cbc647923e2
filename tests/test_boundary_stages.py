"""Host-side validation of the two standalone stages, mhc_pre_inv_rms and mhc_pre_sinkhorn
(no GPU needed: every case below is refused, or succeeds with T == 0, before any HIP call)."""
import ctypes

import pytest

from mhc_hyper_connection_amd import _binding as B

FIELDS = B.SINKHORN_TENSOR_FIELDS
GOOD = {"x": 16, "h_mix": 16, "inv_rms": 16, "alpha": 16, "bias": 16, "pre_mix": None, "h_in": 16,
        "h_pre": 16, "h_post": 16, "h_res": 16, "sum_out": None, "norm_out": None}


def inv_rms(params, x=16, out=16):
    return B.load().mhc_pre_inv_rms(ctypes.byref(params) if params else None,
                                     ctypes.c_void_p(x) if x else None,
                                     ctypes.c_void_p(out) if out else None, None)


def sinkhorn(params, **over):
    p = dict(GOOD, **over)
    t = B.SinkhornTensors(*[ctypes.c_void_p(p[f]) if p[f] else None for f in FIELDS])
    return B.load().mhc_pre_sinkhorn(ctypes.byref(params) if params else None, ctypes.byref(t), None)


def test_inv_rms_validation():
    assert inv_rms(None) == B.MHC_ERR_NULLPTR
    assert inv_rms(B.make_params(4, 4, 64), x=0) == B.MHC_ERR_NULLPTR
    assert inv_rms(B.make_params(4, 4, 64), out=0) == B.MHC_ERR_NULLPTR
    assert inv_rms(B.make_params(4, 4, 64), x=8) == B.MHC_ERR_PARAM_INVALID        # x not 16-byte aligned
    assert inv_rms(B.make_params(4, 4, 64), out=18) == B.MHC_ERR_PARAM_INVALID     # out not 4-byte aligned
    assert inv_rms(B.make_params(4, 5, 64)) == B.MHC_ERR_PARAM_INVALID
    assert inv_rms(B.make_params(4, 4, 60)) == B.MHC_ERR_PARAM_INVALID
    assert inv_rms(B.make_params(4, 4, 64, norm_eps=0.0)) == B.MHC_ERR_PARAM_INVALID
    assert inv_rms(B.make_params(-1, 4, 64)) == B.MHC_ERR_PARAM_INVALID
    assert inv_rms(B.make_params(0, 4, 64), x=0, out=0) == B.MHC_OK


@pytest.mark.parametrize("field", ["x", "h_mix", "inv_rms", "alpha", "bias", "h_in", "h_pre", "h_post", "h_res"])
def test_sinkhorn_required_pointers(field):
    assert sinkhorn(B.make_params(4, 4, 64), **{field: 0}) == B.MHC_ERR_NULLPTR


def test_sinkhorn_rules():
    assert B.load().mhc_pre_sinkhorn(None, None, None) == B.MHC_ERR_NULLPTR
    # without the res branch hRes may be NULL, and there are no Sinkhorn planes
    assert sinkhorn(B.make_params(0, 4, 64, n_alpha=2), h_res=0) == B.MHC_OK
    assert sinkhorn(B.make_params(4, 4, 64, n_alpha=2), sum_out=16) == B.MHC_ERR_PARAM_INVALID
    # needBackward with the res branch needs both planes
    assert sinkhorn(B.make_params(4, 4, 64, need_backward=True)) == B.MHC_ERR_PARAM_INVALID
    assert sinkhorn(B.make_params(4, 4, 64, need_backward=True), sum_out=16) == B.MHC_ERR_PARAM_INVALID
    # alignment
    assert sinkhorn(B.make_params(4, 4, 64), x=8) == B.MHC_ERR_PARAM_INVALID
    assert sinkhorn(B.make_params(4, 4, 64), h_in=8) == B.MHC_ERR_PARAM_INVALID
    assert sinkhorn(B.make_params(4, 4, 64), h_mix=18) == B.MHC_ERR_PARAM_INVALID
    assert sinkhorn(B.make_params(4, 4, 64), pre_mix=18) == B.MHC_ERR_PARAM_INVALID
    # attributes
    assert sinkhorn(B.make_params(4, 4, 64, num_iters=0)) == B.MHC_ERR_PARAM_INVALID
    assert sinkhorn(B.make_params(4, 4, 64, hc_eps=-1.0)) == B.MHC_ERR_PARAM_INVALID
    assert sinkhorn(B.make_params(-1, 4, 64)) == B.MHC_ERR_PARAM_INVALID
    # empty input: success with no pointers at all
    empty = {f: 0 for f in FIELDS}
    assert sinkhorn(B.make_params(0, 4, 64), **empty) == B.MHC_OK
