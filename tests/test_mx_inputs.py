"""CPU checks of the microscaled FP8 input generator (no GPU needed).

The generator follows the OCP Microscaling rule for e4m3 elements: a block's
shared scale is 2^X with X = floor(log2(max |x|)) - 8, so the block's largest
magnitude lands in [2^8, 2^9) before rounding, and values above 448 (e4m3's
largest) saturate. These tests hold every element to that rule.
"""

import numpy as np
import pytest

import oracle
import seeded_inputs as si


def _check_block_rule(x, vals, scales, axis_blocks):
    """x: float64 values grouped as [..., blocks, 32]; vals: their decoded
    values; scales: E8M0 codes [..., blocks]."""
    amax = np.abs(x).max(axis=-1)
    X = scales.astype(np.float64) - 127.0
    nz = amax > 0
    assert np.all(np.floor(np.log2(amax[nz])) - 8 == X[nz]), "scale exponent differs from the MX rule"
    step = np.exp2(X)[..., None]
    y = x / step                          # the value the e4m3 rounding sees
    sat = np.abs(y) > 448.0
    err = np.abs(vals - x) / step         # error in units of the block scale
    # e4m3 rounding to nearest: half a unit in the last place (2^-4 relative
    # in the normal range, 2^-10 absolute below 2^-6); saturated values hold +-448
    ok = np.where(sat, np.abs(vals / step) == 448.0, err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + 1e-12)
    assert np.all(ok), f"{np.count_nonzero(~ok)} elements break the e4m3 rounding rule"


@pytest.mark.parametrize("N", [1, 31, 32, 33, 100])
def test_row_blocks(N):
    rng = np.random.default_rng(N)
    x = (rng.standard_normal((2, N, 3, 64)) * np.exp2(rng.integers(-20, 20, (2, N, 3, 1)))).astype(np.float32)
    codes, sc = si.quantize_mx_rows(x)
    assert codes.shape == x.shape and sc.shape == (2, N, 3, 2) and sc.dtype == np.uint8
    vals = oracle.dequantize_mx_rows(codes, sc)
    _check_block_rule(x.astype(np.float64).reshape(2, N, 3, 2, 32), vals.reshape(2, N, 3, 2, 32), sc, 3)


@pytest.mark.parametrize("N", [1, 31, 32, 33, 100])
def test_column_blocks(N):
    rng = np.random.default_rng(100 + N)
    x = (rng.standard_normal((2, N, 3, 64)) * np.exp2(rng.integers(-20, 20, (2, 1, 3, 64)))).astype(np.float32)
    codes, sc = si.quantize_mx_cols(x)
    nb = (N + 31) // 32
    assert codes.shape == x.shape and sc.shape == (2, nb, 3, 64)
    vals = oracle.dequantize_mx_cols(codes, sc)
    pad = lambda a: np.concatenate([a, np.zeros((2, nb * 32 - N, 3, 64))], axis=1)
    xb = pad(x.astype(np.float64)).reshape(2, nb, 32, 3, 64).transpose(0, 1, 3, 4, 2)
    vb = pad(vals).reshape(2, nb, 32, 3, 64).transpose(0, 1, 3, 4, 2)
    _check_block_rule(xb, vb, sc, 1)


def test_zero_block_and_extremes():
    x = np.zeros((1, 2, 1, 64), np.float32)
    x[0, 1, 0, 32:] = 3.0e38                       # largest exponents: scale code 254 at most
    codes, sc = si.quantize_mx_rows(x)
    assert sc[0, 0, 0, 0] == 0 and sc[0, 0, 0, 1] == 0 and np.all(codes[0, 0] == 0)
    assert sc[0, 1, 0, 1] == 127 + int(np.floor(np.log2(3.0e38))) - 8
    assert np.all(np.isfinite(oracle.dequantize_mx_rows(codes, sc)))


def test_draw_is_deterministic():
    a, b = si.draw_mxfp8(1, 40, 2, 128, 9), si.draw_mxfp8(1, 40, 2, 128, 9)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    assert a["q_scale"].shape == (1, 40, 2, 4) and a["v_scale"].shape == (1, 2, 2, 128)
