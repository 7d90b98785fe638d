"""The rounding model of the kernels (tests/kernel_rounding.py) against the
oracle: which tolerances the kernels' bf16 roundings alone require.

The GPU parity tests hold O, dQ, dK, dV to max-abs 2e-2 and mean-abs 2e-3
against the exact result. That fixed absolute bound assumes outputs of order
one. Three kinds of GPU test use a bound derived here instead:
  * softmax scales other than 1/sqrt(d) (gradients, and O on launches of
    more than one workgroup per CU), and dBias: bf16 roundings of P, dS
    and of the outputs give errors proportional to the output magnitude
    M = max|ref|, and the tests use 2e-2 * max(1, M/2) (2e-3 * max(1, M/2)
    for the mean). The model's own errors must stay within three quarters
    of that bound, and for scale 2.5 they must exceed the plain 2e-2 (the widening
    is needed);
  * rows with logsumexp far below zero: every key shares a large component
    along -q, so dQ = scale * sum_j dS_ij K_j cancels a large common part,
    and the bf16 rounding of dS leaves a dQ mean error above 2e-3. The GPU
    test gives the backward the exact O rounded to bf16 and holds each
    gradient to 1.5 times the model's error (or the magnitude-scaled bound
    where that is larger); here the model's dQ mean error must exceed 2e-3.
"""

import math

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests import kernel_rounding as kr

MAX_TOL, MEAN_TOL = 2e-2, 2e-3
# The model's error may use at most this share of a derived bound; the rest
# is headroom for what the model leaves out (fp32 accumulation order, the
# running maximum's lag moving rounding boundaries).
HEADROOM = 0.75


def ref_backward(x, causal, scale, bias=None):
    if bias is None:
        rq, rk, rv, ro, rl, _ = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], causal, scale)
        return {"dq": rq, "dk": rk, "dv": rv, "o": ro, "lse": rl}
    rq, rk, rv, rdb, ro, rl, _ = oracle.attention_backward_bias(x["q"], x["k"], x["v"], bias, x["do"], causal, scale)
    return {"dq": rq, "dk": rk, "dv": rv, "dbias": rdb, "o": ro, "lse": rl}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
def test_model_without_rounding_is_the_oracle(causal, with_bias):
    B, N, H, d = 2, 37, 2, 16
    bits = si.draw(B, N, H, d, 4321 + int(causal), backward=True)
    x = {n: si.bf16_bits_to_f64(bits[n]) for n in bits}
    bias = si.bf16_bits_to_f64(si.draw_bias_with_holes(B, H, N, 4322)) if with_bias else None
    ref = ref_backward(x, causal, 0.3, bias)
    got = kr.emulate(x["q"], x["k"], x["v"], x["do"], causal, 0.3, bias=bias, rounding=False)
    for n in ref:
        finite = np.isfinite(ref[n])
        assert np.array_equal(finite, np.isfinite(got[n])), n
        assert np.allclose(got[n][finite], ref[n][finite], rtol=1e-12, atol=1e-12), n


def test_model_rounds_where_the_kernels_do():
    """The modelled outputs are bf16 values, and the model's error is of the
    size bf16 rounding gives (non-zero, well below the plain bound, for
    ordinary inputs at the default scale)."""
    B, N, H, d = 1, 150, 2, 64
    bits = si.draw(B, N, H, d, 77 + d, backward=True)
    x = {n: si.bf16_bits_to_f64(bits[n]) for n in bits}
    got = kr.emulate(x["q"], x["k"], x["v"], x["do"], True, d ** -0.5)
    ref = ref_backward(x, True, d ** -0.5)
    for n in ("o", "dq", "dk", "dv"):
        assert np.array_equal(kr.bf16(got[n]), got[n]), n
        mx, mn = kr.error(got[n], ref[n])
        assert 0 < mx <= MAX_TOL / 2 and mn <= MEAN_TOL / 2, (n, mx, mn)


@pytest.mark.parametrize("d", [64, 128])
def test_scaled_bound_admits_the_roundings_at_other_scales(d):
    """The inputs of the GPU test of other scales (N = 150, H = 2, seed
    77 + d): the model's gradient errors lie within three quarters of
    2e-2 * max(1, M/2), and at scale 2.5 some exceed the plain 2e-2."""
    bits = si.draw(1, 150, 2, d, 77 + d, backward=True)
    x = {n: si.bf16_bits_to_f64(bits[n]) for n in bits}
    beyond_plain = False
    for scale in (-0.2, 0.0, 0.9, 2.5):
        for causal in (False, True):
            got = kr.emulate(x["q"], x["k"], x["v"], x["do"], causal, scale)
            ref = ref_backward(x, causal, scale)
            for n in ("dq", "dk", "dv"):
                mx, mn = kr.error(got[n], ref[n])
                m = max(1.0, float(np.abs(ref[n]).max()) / 2.0)
                assert mx <= HEADROOM * MAX_TOL * m and mn <= HEADROOM * MEAN_TOL * m, (scale, causal, n, mx, mn, m)
                beyond_plain |= mx > MAX_TOL
    assert beyond_plain, "the plain bound would have sufficed: the widening is not needed"


def test_scaled_bound_admits_the_roundings_of_o_at_other_scales():
    """O at other scales, on the inputs of the GPU tests that hold it to the
    magnitude-scaled bound (N = 150, H = 2, seed 77 + d; and B = 1, N = 700,
    H = 50, d = 128, seed 3100): within three quarters of the bound. At
    large scales the softmax is nearly one-hot and |O| reaches V's largest
    entries, where one bf16 rounding is up to |O| 2^-9."""
    cases = [(si.draw(1, 150, 2, d, 77 + d, backward=True), (-0.2, 0.0, 0.9, 2.5)) for d in (64, 128)]
    cases.append((si.draw(1, 700, 50, 128, 3100, backward=True), (-0.2, 0.0, 0.9, 2.5)))
    for bits, scales in cases:
        x = {n: si.bf16_bits_to_f64(bits[n]) for n in bits}
        for scale in scales:
            for causal in (False, True):
                got = kr.emulate(x["q"], x["k"], x["v"], x["do"], causal, scale)
                ref = ref_backward(x, causal, scale)
                mx, mn = kr.error(got["o"], ref["o"])
                m = max(1.0, float(np.abs(ref["o"]).max()) / 2.0)
                assert mx <= HEADROOM * MAX_TOL * m and mn <= HEADROOM * MEAN_TOL * m, (scale, causal, mx, mn, m)


def test_scaled_bound_admits_the_roundings_of_dbias():
    """The biased cases of the GPU tests whose dBias reaches |dS| of several
    units on short causal rows: the model's dBias error lies within three
    quarters of 2e-2 * max(1, M/2) on every small shape the GPU test runs."""
    for B, N, H, d in [(1, 17, 2, 64), (2, 64, 2, 128), (1, 129, 3, 64), (1, 200, 2, 128), (2, 256, 1, 128)]:
        for causal in (False, True):
            seed = 9100 + N + d + int(causal)
            bits = si.draw(B, N, H, d, seed, backward=True)
            x = {n: si.bf16_bits_to_f64(bits[n]) for n in bits}
            bias = si.bf16_bits_to_f64(si.draw_bias_with_holes(B, H, N, seed + 1, holes=N > 1))
            scale = 1.0 / math.sqrt(d)
            got = kr.emulate(x["q"], x["k"], x["v"], x["do"], causal, scale, bias=bias)
            ref = ref_backward(x, causal, scale, bias)
            mx, mn = kr.error(got["dbias"], ref["dbias"])
            m = max(1.0, float(np.abs(ref["dbias"]).max()) / 2.0)
            assert mx <= HEADROOM * MAX_TOL * m and mn <= HEADROOM * MEAN_TOL * m, ((B, N, H, d, causal), mx, mn, m)


@pytest.mark.parametrize("d", [64, 128])
def test_negative_logsumexp_rows_need_a_derived_bound(d):
    """The inputs of the GPU test with logsumexp below -88 (N = 100, H = 2,
    scale 1/8, seed 5 + d), with the backward given the exact O rounded to
    bf16 (as that test does): bf16 rounding of dS alone puts dQ's mean error
    above the plain 2e-3, for both masks."""
    bits = si.draw_negative_logsumexp(1, 100, 2, d, 5 + d)
    x = {n: si.bf16_bits_to_f64(bits[n]) for n in bits}
    for causal in (False, True):
        ref = ref_backward(x, causal, 1.0 / 8.0)
        got = kr.emulate(x["q"], x["k"], x["v"], x["do"], causal, 1.0 / 8.0, o_in=kr.bf16(ref["o"]))
        assert ref["lse"].max() < -88.0
        _, mn = kr.error(got["dq"], ref["dq"])
        assert mn > MEAN_TOL, (causal, mn)
