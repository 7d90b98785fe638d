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


def head_bound(q, k, v, causal, scale, rows=None, chunk=2048):
    """Reference rows of one head (fp64 dequantized q, k, v [N, d]) and the
    per-element error bound, in chunks of `chunk` query rows (each holds
    whole rows of scores). Returns (O_ref [R, d], L_ref [R], bound [R, d])."""
    N = k.shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    o = np.empty((rows.size, v.shape[1]))
    lse = np.empty(rows.size)
    bound = np.empty((rows.size, v.shape[1]))
    av = np.abs(v)
    for c0 in range(0, rows.size, chunk):
        rr = rows[c0 : c0 + chunk]
        s = scale * (q[rr] @ k.T)
        if causal:
            s = np.where(np.arange(N)[None, :] > rr[:, None], -np.inf, s)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        oc = (p @ v) / l
        w = np.where(p > 0, np.maximum(p * 2.0 ** -4, 2.0 ** -14), 0.0)
        o[c0 : c0 + chunk] = oc
        lse[c0 : c0 + chunk] = (m + np.log(l))[:, 0]
        bound[c0 : c0 + chunk] = (w @ av) / l + 2.0 ** -8 * np.abs(oc) + 1e-6
    return o, lse, bound
