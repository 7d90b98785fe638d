"""CPU self-check of the FP8 forward's per-element error bound: an exact
result and a result with e4m3-rounded probabilities lie inside it, while
plausible kernel mistakes (planted here, in fp64 on the CPU) fall outside."""

import numpy as np

import oracle
import seeded_inputs as si
from tests.fp8_bound import head_bound


def _e4m3_round(x):
    return oracle.e4m3_decode(si.f64_to_e4m3_bits(x))


def _inputs(N, seed, causal):
    b8 = si.draw_fp8(1, N, 1, 128, seed)
    q, k, v = (oracle.dequantize_fp8(b8[n], b8[n + "_descale"])[0, :, 0] for n in ("q", "k", "v"))
    return q, k, v, b8["v_descale"][0, 0]


def _emulate(q, k, v, causal, scale, c_log2=4.0, vrows=None, vscale=1.0, score_scale=None):
    """The kernel's arithmetic in fp64: P = 2^c * exp2(t - m) rounded to e4m3,
    O = (P v) / sum(unrounded P)."""
    N = k.shape[0]
    s = (scale if score_scale is None else score_scale) * (q @ k.T)
    if causal:
        s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    p = np.exp2((s - m) / np.log(2.0) + c_log2)
    pr = _e4m3_round(p)
    vv = v if vrows is None else v[vrows]
    return (pr @ vv) * vscale / p.sum(axis=1, keepdims=True)


def _ratio(o, q, k, v, causal, scale):
    ro, rl, bd = head_bound(q, k, v, causal, scale)
    return float((np.abs(o - ro) / bd).max())


def test_exact_and_rounded_results_are_inside():
    for causal in (False, True):
        q, k, v, _ = _inputs(300, 20, causal)
        ro, _, _ = head_bound(q, k, v, causal, 0.088)
        assert _ratio(ro, q, k, v, causal, 0.088) < 1e-3
        # every scale the lagging running max allows: P = 2^c exp2(s - max)
        # from c = 4 (running max at the row maximum) up to a largest value
        # of 448, the largest e4m3 number (c = log2(448))
        for c in (4.0, 6.0, 8.0, float(np.log2(448.0))):
            assert _ratio(_emulate(q, k, v, causal, 0.088, c), q, k, v, causal, 0.088) <= 1.0


def test_planted_kernel_mistakes_are_outside():
    q, k, v, vd = _inputs(300, 21, True)
    N = k.shape[0]
    perm = np.arange(N)
    swapped = (perm & ~12) | ((perm & 4) << 1) | ((perm & 8) >> 1)     # V rows left in LDS key order
    assert _ratio(_emulate(q, k, v, True, 0.088, vrows=swapped), q, k, v, True, 0.088) > 1.0
    assert _ratio(_emulate(q, k, v, True, 0.088, vscale=1.0 / vd), q, k, v, True, 0.088) > 1.0  # V descale dropped
    assert _ratio(_emulate(q, k, v, True, 0.088, score_scale=1.0), q, k, v, True, 0.088) > 1.0  # unscaled scores
    shift = np.roll(np.arange(N), 1)                                   # off-by-one key
    assert _ratio(_emulate(q, k, v, True, 0.088, vrows=shift), q, k, v, True, 0.088) > 1.0


def _mx_inputs(d, seed):
    """Microscaled inputs with block scales far apart (as the GPU test that
    checks the scales reach the right blocks)."""
    b8 = si.draw_mxfp8(1, 300, 1, d, seed)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    b8["q_scale"] = (b8["q_scale"].astype(np.int64) + np.array([-6, 3, 0, -2])[: d // 32]).astype(np.uint8)
    b8["k_scale"] = (b8["k_scale"].astype(np.int64) + np.array([4, -3, 1, 0])[: d // 32]).astype(np.uint8)
    vs = b8["v_scale"].astype(np.int64)
    vs += 5 * (np.arange(vs.shape[1]) % 2)[None, :, None, None] + 3 * (np.arange(d) % 3 == 0)[None, None, None, :]
    vs += rng.integers(-2, 3, vs.shape)
    b8["v_scale"] = vs.astype(np.uint8)
    return b8


def _mx_values(b8, qs=None, ks=None, vs=None):
    q = oracle.dequantize_mx_rows(b8["q"], b8["q_scale"] if qs is None else qs)[0, :, 0]
    k = oracle.dequantize_mx_rows(b8["k"], b8["k_scale"] if ks is None else ks)[0, :, 0]
    v = oracle.dequantize_mx_cols(b8["v"], b8["v_scale"] if vs is None else vs)[0, :, 0]
    return q, k, v


def test_mx_scale_mistakes_are_outside():
    """For the microscaled form, the mistakes a kernel could make with the
    block scales — Q's or K's scales applied to the other lane half's blocks
    or to the neighbouring 32-element block, K's scales taken
    from the neighbouring key row, V's scales from the neighbouring key block
    or column — move the result outside the bound that the correct
    arithmetic (with e4m3-rounded P) stays inside, at d = 64 and 128."""
    scale = 0.09
    for d in (64, 128):
        b8 = _mx_inputs(d, 21 + d)
        q, k, v = _mx_values(b8)
        assert _ratio(_emulate(q, k, v, True, scale), q, k, v, True, scale) <= 1.0
        nb = d // 32
        halves = np.arange(nb) ^ (nb // 2)                               # the two lane halves' blocks swapped
        steps = np.arange(nb) ^ 1                                        # neighbouring d-blocks swapped
        wrong = [
            _mx_values(b8, qs=b8["q_scale"][..., halves]),
            _mx_values(b8, ks=b8["k_scale"][..., halves]),
            _mx_values(b8, qs=b8["q_scale"][..., steps]),
            _mx_values(b8, ks=b8["k_scale"][..., steps]),
            _mx_values(b8, ks=np.roll(b8["k_scale"], 1, axis=1)),        # neighbouring key row
            _mx_values(b8, vs=np.roll(b8["v_scale"], 1, axis=1)),        # neighbouring key block
            _mx_values(b8, vs=np.roll(b8["v_scale"], 1, axis=3)),        # neighbouring column
        ]
        for qw, kw, vw in wrong:
            assert _ratio(_emulate(qw, kw, vw, True, scale), q, k, v, True, scale) > 1.0
