"""The fp64 hc_post oracle (oracle/mhc_oracle_post.c) against what pins it, and the pins
against planted mistakes.

The HcPre guide (mhpn.cn/news/2282827, section "mHC 架构与 HcPre 的定位") prints hc_post
as torch broadcasting over comb_frag, whose shape its section "返回值说明" gives as
[b, s, hc_mult, hc_mult]. On that 4-D layout the sum over dim 2 runs over comb's first
index: out[j] = post[j] x + sum_i comb[i][j] residual[i].

Pins:
  page expression  the printed expression evaluated by NumPy broadcasting on 4-D arrays
               ([b, s, n, n] comb, [b, s, n, d] residual, [b, s, n] post, [b, s, d] x)
               equals the oracle's TND call on the same values (T = b s) to 1e-12.
  permutation  comb[t] a permutation matrix that is not symmetric (a 4-cycle, and its
               8-stream analogue) and post = 0: output stream perm(i) is exactly residual
               stream i (bf16 passes through unchanged). Catches a transposed comb, a
               residual indexed by the output stream, a dropped or doubled residual term.
  column sums  every residual stream equal (r) and post = 0: out[j] = r * (column sum j of
               comb), with the row sums all different from the column sums, so the
               orientation shows; rounded by this file's own float64 -> bf16 rounding.
  post only    residual = 0: out = bf16(post[j] * x[d]), rounded the same way.
  einsum       random inputs: the unrounded output equals NumPy's float64 einsum of the
               same two terms to 1e-12 relative (a library routine as the second
               implementation), and the bf16 output is its nearest bf16.
Mutants: textual changes to the oracle source, each compiled and run through the pins.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "mhc_oracle_post.c")
FWD = os.path.join(HERE, "mhc_oracle.c")
BWD = os.path.join(HERE, "mhc_oracle_bwd.c")


def _bf16_round(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, nearest with ties to even, via exact float64 arithmetic."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    for idx, val in np.ndenumerate(v):
        if val == 0.0:
            out[idx] = 0x8000 if np.signbit(val) else 0
            continue
        m, e = np.frexp(abs(val))                  # val = m 2^e, m in [0.5, 1)
        q = np.ldexp(m, 8)                         # 8 significant bits
        lo = np.floor(q)
        r = q - lo
        q = lo + (1.0 if (r > 0.5 or (r == 0.5 and int(lo) % 2 == 1)) else 0.0)
        f = np.float32(np.ldexp(q, e - 8) * (1 if val > 0 else -1))
        out[idx] = np.frombuffer(np.float32(f).tobytes(), dtype=np.uint32)[0] >> 16
    return out


def pin_page_expression_4d(lib):
    # the guide's expression, term by term, as NumPy broadcasting on the 4-D shapes
    # the guide documents (b, s leading), against the oracle on the flattened tokens
    b, s_len, n, D = 2, 3, 4, 16
    inp = synth.post_inputs(b * s_len, n, D, seed=31)
    r = oracle.post(inp.x, inp.residual, inp.post, inp.comb, lib=lib)
    x4 = synth.bf16_bits_to_f32(inp.x).astype(np.float64).reshape(b, s_len, D)
    res4 = synth.bf16_bits_to_f32(inp.residual).astype(np.float64).reshape(b, s_len, n, D)
    post4 = inp.post.astype(np.float64).reshape(b, s_len, n)
    comb4 = inp.comb.astype(np.float64).reshape(b, s_len, n, n)
    # out = post.unsqueeze(-1) * x.unsqueeze(-2) + torch.sum(comb.unsqueeze(-1) * residual.unsqueeze(-2), dim=2)
    page = post4[..., :, None] * x4[..., None, :] + np.sum(comb4[..., :, :, None] * res4[..., :, None, :], axis=2)
    assert page.shape == (b, s_len, n, D)
    assert np.allclose(r.out, page.reshape(b * s_len, n, D), rtol=1e-12, atol=1e-12)


def pin_permutation(lib):
    for n in (4, 8):
        T, D = 3, 24
        inp = synth.post_inputs(T, n, D, seed=5 + n)
        perm = [(i + 1) % n for i in range(n)]          # a cycle: not its own transpose
        comb = np.zeros((T, n, n), dtype=np.float32)
        for i in range(n):
            comb[:, i, perm[i]] = 1.0                   # column perm[i] holds its 1 in row i
        r = oracle.post(inp.x, inp.residual, np.zeros((T, n), np.float32), comb, lib=lib)
        for i in range(n):
            assert np.array_equal(r.out_bf16[:, perm[i], :], inp.residual[:, i, :]), (n, i)


def pin_column_sums(lib):
    # equal residual streams: out[j] = r * sum_i comb[i][j]; comb's row sums (1, 2, 3, 4
    # times 1/4) and column sums (0.625 each) differ, and the products are exact
    T, n, D = 2, 4, 16
    inp = synth.post_inputs(T, n, D, seed=17)
    res = np.repeat(inp.residual[:, :1, :], n, axis=1)
    comb = np.zeros((T, n, n), dtype=np.float32)
    for i in range(n):
        comb[:, i, :] = 0.0625 * (i + 1)               # row i constant: row sums differ
    comb[:, 0, 0] += 0.25                               # and one column sum differs
    r = oracle.post(inp.x, res, np.zeros((T, n), np.float32), comb, lib=lib)
    cs = comb.astype(np.float64).sum(axis=1)            # [T, n] column sums
    rf = synth.bf16_bits_to_f32(res[:, 0, :]).astype(np.float64)
    want = _bf16_round(cs[:, :, None] * rf[:, None, :])
    assert np.array_equal(r.out_bf16, want)


def pin_post_only(lib):
    T, n, D = 4, 4, 16
    inp = synth.post_inputs(T, n, D, seed=9)
    zeros = np.zeros_like(inp.residual)
    r = oracle.post(inp.x, zeros, inp.post, inp.comb, lib=lib)
    xf = synth.bf16_bits_to_f32(inp.x).astype(np.float64)
    want = _bf16_round(inp.post.astype(np.float64)[:, :, None] * xf[:, None, :])
    assert np.array_equal(r.out_bf16, want)


def pin_einsum(lib):
    T, n, D = 5, 4, 40
    inp = synth.post_inputs(T, n, D, seed=13)
    r = oracle.post(inp.x, inp.residual, inp.post, inp.comb, lib=lib)
    xf = synth.bf16_bits_to_f32(inp.x).astype(np.float64)
    rf = synth.bf16_bits_to_f32(inp.residual).astype(np.float64)
    want = (np.einsum("tj,td->tjd", inp.post.astype(np.float64), xf)
            + np.einsum("tij,tid->tjd", inp.comb.astype(np.float64), rf))
    assert np.allclose(r.out, want, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r.out_bf16, _bf16_round(r.out))
    assert np.all(r.out_abs >= np.abs(r.out) - 1e-12)


def pin_f16_permutation_and_einsum(lib=None):
    # binary16 storage: a permutation comb with post = 0 returns the picked residual rows
    # bit for bit, and the unrounded output equals NumPy's float64 einsum, rounded to fp16
    T, n, D = 3, 4, 24
    rng = np.random.default_rng(77)
    x = (rng.standard_normal((T, D)) * 2).astype(np.float16).view(np.uint16)
    res = (rng.standard_normal((T, n, D)) * 2).astype(np.float16).view(np.uint16)
    perm = [1, 2, 3, 0]
    comb = np.zeros((T, n, n), np.float32)
    comb[:, np.arange(n), perm] = 1.0                  # output stream perm[i] takes stream i
    r = oracle.post(x, res, np.zeros((T, n), np.float32), comb, lib=lib, x_f16=True)
    assert np.array_equal(r.out_bf16[:, perm, :], res), "fp16 permutation"
    post_w = rng.uniform(0, 2, (T, n)).astype(np.float32)
    comb = rng.uniform(0.05, 0.45, (T, n, n)).astype(np.float32)
    r = oracle.post(x, res, post_w, comb, lib=lib, x_f16=True)
    xf, rf = x.view(np.float16).astype(np.float64), res.view(np.float16).astype(np.float64)
    want = post_w[:, :, None] * xf[:, None, :] + np.einsum("tij,tid->tjd", comb.astype(np.float64), rf)
    assert np.allclose(r.out, want, rtol=1e-12, atol=0), "fp16 einsum"
    assert np.array_equal(r.out_bf16, want.astype(np.float16).view(np.uint16)), "fp16 rounding"


PINS = [pin_page_expression_4d, pin_permutation, pin_column_sums, pin_post_only, pin_einsum,
        pin_f16_permutation_and_einsum]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(None)


MUTANTS = {
    # the row-major product comb residual (comb's second index summed)
    "comb_transposed": ("comb[(t * n + i) * n + j]", "comb[(t * n + j) * n + i]"),
    "residual_by_output_stream": ("residual[(t * n + i) * (int64_t)D + d]", "residual[(t * n + j) * (int64_t)D + d]"),
    "post_term_dropped": ("double acc = p * xv;", "double acc = 0.0;"),
    "post_from_next_stream": ("const double p = (double)post[t * n + j];", "const double p = (double)post[t * n + (j + 1) % n];"),
    "residual_term_dropped": ("acc += c * r;", "(void)r;"),
    "f16_residual_read_as_bf16": ("const double r = x_f16 ? oracle_f16_to_double(rb) : oracle_bf16_to_double(rb);",
                                  "const double r = oracle_bf16_to_double(rb);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    c_path = tmp_path / "mutant_post.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(so_path),
                    FWD, BWD, str(c_path), "-lm"], check=True)
    lib = oracle.load_library(str(so_path))
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
