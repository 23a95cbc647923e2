"""binary16 (fp16) x and hIn in the oracle: the conversions against the IEEE 754 binary16
definition and NumPy's float16 (a library routine), and the forward in fp16 mode against
closed forms and against its bf16 mode on values both formats hold exactly. Then planted
mistakes, each caught by a pin."""
import math
import os
import subprocess

import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "mhc_oracle.c")
BWD = os.path.join(HERE, "mhc_oracle_bwd.c")
POST = os.path.join(HERE, "mhc_oracle_post.c")

# binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits
F16_CASES = [
    (1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF), (65520.0, 0x7C00),   # tie above the largest -> inf
    (65519.0, 0x7BFF), (2.0 ** -14, 0x0400), (2.0 ** -24, 0x0001),
    (2.0 ** -25, 0x0000),                              # tie between 0 and the smallest -> even (0)
    (1.5 * 2.0 ** -25, 0x0001), (3 * 2.0 ** -25, 0x0002),   # 1.5 ulp -> 2 (even)
    (1.0 + 2.0 ** -11, 0x3C00), (1.0 + 3 * 2.0 ** -11, 0x3C02), (1.0 + 2.0 ** -11 + 2.0 ** -40, 0x3C01),
    (0.1, 0x2E66), (-0.0, 0x8000), (float("inf"), 0x7C00), (2.0 ** -14 - 2.0 ** -24, 0x03FF),
]


def pin_f16_table(lib=None):
    for v, bits in F16_CASES:
        got = oracle.f16_from_double(v, lib=lib)
        assert got == bits, f"f16({v!r}) = {got:#06x}, want {bits:#06x}"
    for bits in (0x3C00, 0xC000, 0x7BFF, 0x0001, 0x03FF, 0x0400, 0x2E66, 0x8001):
        assert oracle.f16_from_double(oracle.f16_to_double(bits, lib=lib), lib=lib) == bits


def pin_f16_numpy(lib=None):
    rng = np.random.default_rng(70)
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-9, 5, 3000),
                        rng.uniform(-1, 1, 500) * 2.0 ** -24 * 3])
    with np.errstate(over="ignore"):   # values past 65520 round to infinity on both sides
        want = v.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f16_from_double(float(a), lib=lib) for a in v], np.uint16)
    assert np.array_equal(got, want), f"{int((got != want).sum())} roundings differ from NumPy"
    bits = rng.integers(0, 0x7C00, 2000).astype(np.uint16)
    back = np.array([oracle.f16_to_double(int(b), lib=lib) for b in bits])
    assert np.array_equal(back, bits.view(np.float16).astype(np.float64)), "widening differs"


def _zeros(n, D):
    M = n * n + 2 * n
    return np.zeros((M, n * D), np.float32), np.ones(3, np.float32), np.zeros(M, np.float32)


def pin_forward_f16_closed(lib=None):
    n, D = 4, 8
    phi, alpha, bias = _zeros(n, D)
    c = 1.0 + 2.0 ** -10          # exact in binary16, not in bf16
    x = np.full((2, n, D), oracle.f16_from_double(c, lib=lib), np.uint16)
    r = oracle.forward(x, phi, alpha, bias, x_f16=True, lib=lib)
    want = 1.0 / math.sqrt(c * c + 1e-6)
    assert np.all(np.abs(r.inv_rms - want) <= 1e-15 * want), "invRms of a constant fp16 x"
    # one-hot pre_mix: hIn is the picked stream, bit for bit, in fp16
    rng = np.random.default_rng(71)
    xv = (rng.standard_normal((3, n, D)) * 3).astype(np.float16).view(np.uint16)
    pm = np.zeros((3, n), np.float32)
    pm[[0, 1, 2], [1, 3, 0]] = 1.0
    r = oracle.forward(xv, phi, alpha, bias, pre_mix=pm, x_f16=True, lib=lib)
    for t, i in zip(range(3), [1, 3, 0]):
        assert np.array_equal(r.h_in_bf16[t], xv[t, i]), f"one-hot pre_mix fp16, token {t}"


def pin_forward_f16_matches_bf16(lib=None):
    # x values that both formats hold exactly: every double result is the same, and hIn
    # is that same double rounded to each format
    n, D, T = 4, 16, 5
    M = n * n + 2 * n
    rng = np.random.default_rng(72)
    xf = np.round(rng.standard_normal((T, n, D)) * 32) / 32
    xb = f32_to_bf16_bits(xf.astype(np.float32))
    xh = xf.astype(np.float16).view(np.uint16)
    assert np.array_equal(xf.astype(np.float16).astype(np.float64), xf)
    phi = (rng.standard_normal((M, n * D)) / 8).astype(np.float32)
    alpha = rng.uniform(0.5, 1.5, 3).astype(np.float32)
    bias = rng.uniform(-0.2, 0.2, M).astype(np.float32)
    rb = oracle.forward(xb, phi, alpha, bias, num_iters=3, lib=lib)
    rh = oracle.forward(xh, phi, alpha, bias, num_iters=3, x_f16=True, lib=lib)
    for f in ("inv_rms", "h_mix", "h_pre", "h_post", "h_res", "sum_out", "norm_out", "h_in"):
        assert np.array_equal(getattr(rb, f), getattr(rh, f)), f
    want = np.array([oracle.f16_from_double(float(v), lib=lib) for v in rh.h_in.ravel()], np.uint16)
    assert np.array_equal(rh.h_in_bf16.ravel(), want)
    assert np.array_equal(oracle.inv_rms(xh, x_f16=True, lib=lib), rh.inv_rms)


PINS = [pin_f16_table, pin_f16_numpy, pin_forward_f16_closed, pin_forward_f16_matches_bf16]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(None)


MUTANTS = {
    "f16_ties_away": ("(fmod(lo, 2.0) == 0.0 ? lo : lo + 1.0)", "(lo + 1.0)"),
    "f16_flush_subnormals": ("if (e < -14) e = -14;", "if (e < -14) return sgn;"),
    "f16_exponent_bias_16": ("const int ex = re2 - 1 + 15;", "const int ex = re2 - 1 + 16;"),
    "f16_widen_subnormal_scale": ("mag = ldexp((double)fr, -24);", "mag = ldexp((double)fr, -25);"),
    "x_always_bf16": ("return c->x_f16 ? oracle_f16_to_double(bits) : oracle_bf16_to_double(bits);",
                      "return oracle_bf16_to_double(bits);"),
    "hin_always_bf16": ("return c->x_f16 ? oracle_f16_from_double(v) : oracle_bf16_from_double(v);",
                        "return oracle_bf16_from_double(v);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(so_path),
                    str(c_path), BWD, POST, "-lm"], check=True)
    lib = oracle.load_library(str(so_path))
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
