"""Per-element error bound of the FP8 forward (shared by the GPU parity test
and its CPU self-check).

The probabilities are rounded to e4m3 for the P V product: a probability
p' = exp(s - max) is held as P = c p' with 2^4 <= c <= 2^8 and rounded to
nearest, an error of at most 2^-4 P in the normal range and 2^-10 below
2^-6; divided by the row sum, output element (i, d) moves by at most
sum_j max(2^-4 p'_ij, 2^-14) |v_jd| / sum_j p'_ij, plus the bf16 rounding of
the output (2^-9 |O|, taken as 2^-8 |O|).
"""

import numpy as np


def head_bound(q, k, v, causal, scale, rows=None):
    """Reference rows of one head (fp64 dequantized q, k, v [N, d]) and the
    per-element error bound. Returns (O_ref [R, d], L_ref [R], bound [R, d])."""
    N = k.shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    s = scale * (q[rows] @ k.T)
    if causal:
        s = np.where(np.arange(N)[None, :] > rows[:, None], -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v) / l
    w = np.where(p > 0, np.maximum(p * 2.0 ** -4, 2.0 ** -14), 0.0)
    bound = (w @ np.abs(v)) / l + 2.0 ** -8 * np.abs(o) + 1e-6
    return o, (m + np.log(l))[:, 0], bound
