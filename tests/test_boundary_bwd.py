"""The MhcPre backward's C-ABI validation on a host without a GPU: every error path
returns before any HIP call (no compute is launched here).

Error classes as for the forward (aclnnMhcPreSinkhorn guide, section 6): 161001 for a
NULL required pointer, 161002 for invalid parameters.
"""
import pytest

from mhc_hyper_connection_amd import _binding as B

FAKE = 0x10000            # 256-byte aligned, never dereferenced: every case returns first
WS_BIG = 1 << 40
REQUIRED = ("x", "phi", "alpha", "grad_h_in", "grad_h_post", "grad_h_res", "inv_rms", "h_mix",
            "h_pre", "h_post", "grad_x", "grad_phi", "grad_alpha", "grad_bias")


def _ptrs(**over):
    p = {f: FAKE for f in REQUIRED}
    p.update(over)
    return p


def bwd(params, ptrs=None, ws=FAKE, ws_bytes=WS_BIG):
    return B.raw_backward(params, _ptrs() if ptrs is None else ptrs, ws, ws_bytes, None)


def test_workspace_size_large_workload():
    T, n, D = 16384, 4, 7168
    ws = B.bwd_workspace_size(B.make_bwd_params(T, n, D))
    M, K = 24, n * D
    # packed phi (224 d-blocks x 4 streams x 2 halves x 3 terms x 1 KiB), per-token gMix
    # (32 floats), c3, fp64 terms (27), and the per-group partials of gradPhi and gradGamma
    assert ws >= 224 * 4 * 2 * 3 * 1024 + T * 32 * 4 + T * 4 + T * 27 * 8 + (M + 1) * K * 4
    assert B.bwd_workspace_size(B.make_bwd_params(0, n, D)) >= 224 * 4 * 2 * 3 * 1024


@pytest.mark.parametrize("field", REQUIRED)
def test_null_required_pointer(field):
    assert bwd(B.make_bwd_params(128, 4, 256), _ptrs(**{field: None})) == B.MHC_ERR_NULLPTR


def test_null_params_and_workspace():
    lib = B.load()
    t = B.BwdTensors(*[_ptrs().get(f) for f in B.BWD_TENSOR_FIELDS])
    assert lib.mhc_pre_backward(None, t, FAKE, WS_BIG, None) == B.MHC_ERR_NULLPTR
    assert bwd(B.make_bwd_params(128, 4, 256), ws=None) == B.MHC_ERR_NULLPTR
    # gamma without grad_gamma
    assert bwd(B.make_bwd_params(128, 4, 256), _ptrs(gamma=FAKE)) == B.MHC_ERR_NULLPTR


@pytest.mark.parametrize("kw", [dict(n=5), dict(n=2), dict(n=16), dict(D=0), dict(D=12), dict(D=16392),
                                dict(T=-1), dict(hc_eps=-1.0), dict(hc_eps=float("nan"))])
def test_invalid_attributes(kw):
    base = dict(T=128, n=4, D=256, hc_eps=1e-6)
    base.update(kw)
    p = B.make_bwd_params(**base)
    assert bwd(p) == B.MHC_ERR_PARAM_INVALID
    with pytest.raises(B.MhcError):
        B.bwd_workspace_size(p)


def test_format_flag_and_iterations():
    for v in (-1, 2):
        p = B.make_bwd_params(128, 4, 256)
        p.x_f16 = v
        assert bwd(p) == B.MHC_ERR_PARAM_INVALID, v
    # fp16 needs the same workspace as bf16
    assert B.bwd_workspace_size(B.make_bwd_params(128, 4, 256, x_f16=True)) == \
        B.bwd_workspace_size(B.make_bwd_params(128, 4, 256))
    for it in (-1, 1001):
        p = B.make_bwd_params(128, 4, 256, num_iters=it)
        assert bwd(p) == B.MHC_ERR_PARAM_INVALID, it


def test_sinkhorn_backward_needs_the_planes():
    p = B.make_bwd_params(128, 4, 256, num_iters=20)
    assert bwd(p) == B.MHC_ERR_NULLPTR
    assert bwd(p, _ptrs(sum_out=FAKE)) == B.MHC_ERR_NULLPTR
    assert bwd(p, _ptrs(norm_out=FAKE)) == B.MHC_ERR_NULLPTR
    # the same workspace size as the MhcPre backward
    assert B.bwd_workspace_size(p) == B.bwd_workspace_size(B.make_bwd_params(128, 4, 256))


def test_workspace_too_small_and_alignment():
    p = B.make_bwd_params(128, 4, 256)
    need = B.bwd_workspace_size(p)
    assert bwd(p, ws_bytes=need - 1) == B.MHC_ERR_PARAM_INVALID
    assert bwd(p, ws=FAKE + 16) == B.MHC_ERR_PARAM_INVALID
    for f in ("x", "grad_h_in", "grad_x"):
        assert bwd(p, _ptrs(**{f: FAKE + 2})) == B.MHC_ERR_PARAM_INVALID, f
    assert bwd(p, _ptrs(grad_x_post=FAKE + 8)) == B.MHC_ERR_PARAM_INVALID


def test_empty_tokens_need_only_the_weight_gradients():
    # T == 0: per-token tensors may be NULL; the weights and their gradients may not
    p = B.make_bwd_params(0, 4, 256)
    ptrs = {f: None for f in B.BWD_TENSOR_FIELDS}
    for f in ("phi", "alpha", "grad_phi", "grad_alpha", "grad_bias"):
        missing = {k: FAKE for k in ("phi", "alpha", "grad_phi", "grad_alpha", "grad_bias") if k != f}
        assert bwd(p, {**ptrs, **missing}) == B.MHC_ERR_NULLPTR, f
