"""The fp64 oracle against closed forms, invariants and independent routines."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(None)


def test_token_subset_matches_full_run():
    import numpy as np

    import oracle
    from synth import custom

    inp = custom(9, 4, 16, gamma=True, seed=3)
    full = oracle.forward(inp.x, inp.phi, inp.alpha, inp.bias, inp.gamma)
    sub = oracle.forward(inp.x, inp.phi, inp.alpha, inp.bias, inp.gamma, tokens=[7, 0, 4])
    for name in ("inv_rms", "h_mix", "h_pre", "h_post", "h_res", "h_in", "h_in_bf16"):
        assert np.array_equal(getattr(sub, name), getattr(full, name)[[7, 0, 4]]), name
    assert np.array_equal(sub.norm_out, full.norm_out[:, [7, 0, 4]])
    assert np.array_equal(sub.sum_out, full.sum_out[:, [7, 0, 4]])
