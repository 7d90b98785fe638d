"""CPU check of the padded-key arithmetic of the backward's dQ product.

Keys past the end of a sequence are read as zero rows. With no mask, such a
key's recomputed probability is exp2(0 * c2 - L * log2 e), which overflows
float32 for a row whose logsumexp L is below about -88.7. Its dS term is then
inf * (0 - D), and the dQ product multiplies it by the zero K row: 0 * inf is
NaN. This test emulates exactly that float32 arithmetic on an input whose
oracle logsumexp is far below -88 (a valid input with a finite exact result),
and shows that masking the key (probability 0) keeps the term at 0.
"""

import numpy as np

import oracle
import seeded_inputs as si


def test_padded_key_term_overflows_unless_masked():
    B, N, H, d = 1, 100, 2, 64
    scale = 1.0 / 8.0
    bits = si.draw_negative_logsumexp(B, N, H, d, 69)
    q, k, v, do = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v", "do"))
    _, _, _, o, lse, dsum = oracle.attention_backward(q, k, v, do, False, scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert lse.max() < -88.0  # every row: exp(-L) overflows float32

    f32 = np.float32
    c2 = f32(scale) * f32(np.log2(np.e))
    l2 = lse.astype(np.float32) * f32(np.log2(np.e))   # L * log2 e per row
    d_row = dsum.astype(np.float32)
    s_pad = f32(0.0)                                    # zero K row: score 0
    dp_pad = f32(0.0)                                   # zero V row: dP 0
    k_pad = f32(0.0)                                    # the K element dQ multiplies by
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp2(s_pad * c2 - l2)                    # unmasked recomputed probability
        ds = p * (dp_pad - d_row)
        term = k_pad * ds
    assert np.all(np.isinf(p))
    assert np.all(np.isnan(term[d_row != 0]))           # the row's dQ would turn NaN

    p_masked = np.where(True, f32(0.0), p)              # the kernel's mask: key >= N -> 0
    term_masked = k_pad * (p_masked * (dp_pad - d_row))
    assert np.all(term_masked == 0.0)
