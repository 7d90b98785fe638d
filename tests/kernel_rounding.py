"""An fp64 model of the roundings the HIP kernels make, for deriving test
tolerances (test infrastructure; the parity reference is always oracle/).

The oracle computes attention exactly. The kernels compute the same thing
with these roundings, and only these, at the bf16 level (fp32 accumulation
and fp32 exponentials are orders of magnitude finer and are not modelled):

  forward   P~ = exp(S - m) is rounded to bf16 for the P V product; the row
            sum uses the unrounded values; O = bf16(sum_j bf16(P~_ij) V_j /
            sum_j P~_ij). (The kernel's running maximum may lag the row
            maximum by a factor; that moves where rounding boundaries fall,
            not their size.)
  backward  D = rowsum(dO * O) from the forward's bf16 O;
            P = exp(S - L) and dS = P * (dP - D), each rounded to bf16 as
            MFMA operands: dV = bf16(bf16(P)^T dO), dK = bf16(scale *
            bf16(dS)^T Q), dQ = bf16(scale * bf16(dS) K); with a bias,
            dBias = bf16(dS).

With rounding switched off the model is the plain definition, and equals
the oracle (checked in tests/test_rounding_bounds.py). The model serves
tests whose inputs make the bf16 roundings themselves exceed the fixed
absolute tolerances: a tolerance is then derived from the model's own error
against the oracle.
"""

from __future__ import annotations

import numpy as np

import seeded_inputs as si


def bf16(x):
    """Round to bfloat16 (nearest, ties to even), returned as float64."""
    return si.bf16_bits_to_f64(si.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def _ident(x):
    return np.asarray(x, dtype=np.float64)


def emulate(q, k, v, do, causal: bool, scale: float, bias=None, rounding: bool = True, o_in=None):
    """Forward and backward of one problem, with the kernels' roundings.

    q, k, v, do: float64 [B, N, H, d]; bias: float64 [B, H, N, N] or None.
    o_in: the O the backward is given (float64 [B, N, H, d], e.g. bf16
    values); None takes the modelled forward's O.
    Returns a dict with o, lse, dq, dk, dv (and dbias with a bias)."""
    r = bf16 if rounding else _ident
    B, N, H, d = q.shape
    out = {n: np.zeros_like(q) for n in ("o", "dq", "dk", "dv")}
    out["lse"] = np.zeros((B, H, N))
    if bias is not None:
        out["dbias"] = np.zeros((B, H, N, N))
    hide = np.arange(N)[None, :] > np.arange(N)[:, None]
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h]
            s = scale * (qh @ kh.T)
            if bias is not None:
                s = s + bias[b, h]
            if causal:
                s = np.where(hide, -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            pt = np.exp(s - m)
            ell = pt.sum(axis=1, keepdims=True)
            seen = ell[:, 0] > 0
            with np.errstate(divide="ignore", invalid="ignore"):
                o = np.where(seen[:, None], (r(pt) @ vh) / np.where(seen, ell[:, 0], 1.0)[:, None], 0.0)
                lse = np.where(seen, m[:, 0] + np.log(np.where(seen, ell[:, 0], 1.0)), -np.inf)
            o = r(o)
            p = np.where(seen[:, None], np.exp(s - np.where(seen, lse, 0.0)[:, None]), 0.0)
            D = (doh * (o if o_in is None else o_in[b, :, h])).sum(axis=1)
            ds = r(p * (doh @ vh.T - D[:, None]))
            out["o"][b, :, h] = o
            out["lse"][b, h] = lse
            out["dv"][b, :, h] = r(r(p).T @ doh)
            out["dk"][b, :, h] = r(scale * (ds.T @ qh))
            out["dq"][b, :, h] = r(scale * (ds @ kh))
            if bias is not None:
                out["dbias"][b, h] = ds
    return out


def error(got, ref):
    """(max-abs, mean-abs) of got - ref."""
    e = np.abs(np.asarray(got) - np.asarray(ref))
    return float(e.max()), float(e.mean())
