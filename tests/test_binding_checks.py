"""The Python launchers' argument checks, on the host: every case raises ValueError before
any call into the library (CPU tensors, a launcher built for the CPU device), so a
tensor of the wrong format, shape or size never reaches a kernel as a raw pointer."""
import pytest

torch = pytest.importorskip("torch")

import mhc_hyper_connection_amd as mhc

CPU = "cpu"
T, N, D = 4, 4, 64
M = N * N + 2 * N


def _fwd(x_f16=False, need_backward=True):
    return mhc.PreForward(T, N, D, 3, num_iters=2, need_backward=need_backward, device=CPU, x_f16=x_f16)


def _fwd_inputs(x_dtype=torch.bfloat16):
    return (torch.zeros((T, N, D), dtype=x_dtype), torch.zeros((M, N * D)), torch.zeros(3),
            torch.zeros(M))


def test_forward_rejects_wrong_x_format_and_shape():
    r = _fwd()
    x, phi, alpha, bias = _fwd_inputs(torch.float16)
    with pytest.raises(ValueError, match="x: dtype"):
        r(x, phi, alpha, bias)
    r16 = _fwd(x_f16=True)
    with pytest.raises(ValueError, match="x: dtype"):
        r16(*_fwd_inputs(torch.bfloat16))
    with pytest.raises(ValueError, match="x: shape"):
        r(torch.zeros((T, N, D + 8), dtype=torch.bfloat16), phi, alpha, bias)
    with pytest.raises(ValueError, match="contiguous"):
        r(torch.zeros((T, D, N), dtype=torch.bfloat16).transpose(1, 2), phi, alpha, bias)


@pytest.mark.parametrize("case", ["missing_h_in", "unknown", "h_in_format", "h_pre_shape", "norm_out_steps"])
def test_forward_checks_the_outputs_it_writes(case):
    r = _fwd()
    out = r.alloc_outputs()
    if case == "missing_h_in":
        del out["h_in"]
        err = "required"
    elif case == "unknown":
        out["h_other"] = torch.zeros(1)
        err = "unknown"
    elif case == "h_in_format":
        out["h_in"] = torch.zeros((T, D), dtype=torch.float16)
        err = "h_in: dtype"
    elif case == "h_pre_shape":
        out["h_pre"] = torch.zeros((T, N + 1))
        err = "h_pre: shape"
    else:
        out["norm_out"] = torch.zeros((2, T, N, N))      # 2 iterations need 4 planes
        err = "norm_out: shape"
    with pytest.raises(ValueError, match=err):
        r(*_fwd_inputs(), out=out)


def test_forward_checks_packed_weights():
    r = _fwd()
    x, phi, alpha, bias = _fwd_inputs()
    with pytest.raises(ValueError, match="phi_packed"):
        r(x, None, alpha, bias, phi_packed=torch.zeros(r.packed_bytes - 16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="phi_packed"):
        r(x, None, alpha, bias, phi_packed=torch.zeros(r.packed_bytes // 4, dtype=torch.float32))


def _bwd(x_f16=False):
    return mhc.PreBackward(T, N, D, device=CPU, x_f16=x_f16)


def _bwd_inputs(x_dtype=torch.bfloat16):
    z = torch.zeros
    return (z((T, N, D), dtype=x_dtype), z((M, N * D)), z(3), z((T, D), dtype=x_dtype), z((T, N)),
            z((T, N, N)), z(T), z((T, M)), z((T, N)), z((T, N)))


def test_backward_takes_one_16_bit_format():
    with pytest.raises(ValueError, match="x: dtype"):
        _bwd()(*_bwd_inputs(torch.float16))
    with pytest.raises(ValueError, match="x: dtype"):
        _bwd(x_f16=True)(*_bwd_inputs(torch.bfloat16))
    args = list(_bwd_inputs(torch.float16))
    args[3] = torch.zeros((T, D), dtype=torch.bfloat16)       # gradHIn in the other format
    with pytest.raises(ValueError, match="grad_h_in: dtype"):
        _bwd(x_f16=True)(*args)
    assert _bwd(x_f16=True).alloc_outputs()["grad_x"].dtype == torch.float16


@pytest.mark.parametrize("case", ["missing", "extra", "grad_x_format", "grad_phi_shape", "gamma_needs_grad_gamma"])
def test_backward_checks_the_outputs_it_writes(case):
    r = _bwd()
    gamma = None
    out = r.alloc_outputs()
    if case == "missing":
        del out["grad_bias"]
        err = "exactly"
    elif case == "extra":
        out["grad_gamma"] = torch.zeros((N, D))               # no gamma given
        err = "exactly"
    elif case == "grad_x_format":
        out["grad_x"] = torch.zeros((T, N, D), dtype=torch.float16)
        err = "grad_x: dtype"
    elif case == "grad_phi_shape":
        out["grad_phi"] = torch.zeros((M, N * D + 1))
        err = "grad_phi: shape"
    else:
        gamma = torch.ones((N, D))
        err = "exactly"
    with pytest.raises(ValueError, match=err):
        r(*_bwd_inputs(), gamma, out=out)
