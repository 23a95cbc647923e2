"""hc_post's C-ABI validation on the host (no GPU needed: every case below is refused
before any HIP call)."""
import ctypes

import pytest

from mhc_hyper_connection_amd import _binding as B


def call(T, n, D, ptrs=(16, 16, 16, 16, 16), x_dtype=0, reserved=0):
    p = B.PostParams(T, n, D, x_dtype, reserved)
    t = B.PostTensors(*[ctypes.c_void_p(v) if v else None for v in ptrs])
    return B.load().mhc_post(ctypes.byref(p), ctypes.byref(t), None)


@pytest.mark.parametrize("T,n,D,want", [(-1, 4, 64, B.MHC_ERR_PARAM_INVALID), (4, 5, 64, B.MHC_ERR_PARAM_INVALID), (4, 7, 64, B.MHC_ERR_PARAM_INVALID),
                                        (4, 4, 60, B.MHC_ERR_PARAM_INVALID), (4, 4, 0, B.MHC_ERR_PARAM_INVALID),
                                        (4, 4, 16392, B.MHC_ERR_PARAM_INVALID), (0, 4, 64, B.MHC_OK)])
def test_sizes(T, n, D, want):
    assert call(T, n, D) == want


def test_null_and_alignment():
    assert B.load().mhc_post(None, None, None) == B.MHC_ERR_NULLPTR
    assert call(4, 4, 64, (16, 0, 16, 16, 16)) == B.MHC_ERR_NULLPTR
    assert call(4, 4, 64, (16, 16, 16, 16, 8)) == B.MHC_ERR_PARAM_INVALID    # out not 16-byte aligned
    assert call(4, 4, 64, (16, 16, 18, 16, 16)) == B.MHC_ERR_PARAM_INVALID   # post not 4-byte aligned


def test_format_fields():
    assert call(4, 4, 64, x_dtype=2) == B.MHC_ERR_PARAM_INVALID
    assert call(4, 4, 64, reserved=1) == B.MHC_ERR_PARAM_INVALID
    assert call(0, 4, 64, x_dtype=1) == B.MHC_OK
