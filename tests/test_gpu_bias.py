"""GPU parity of attention with an additive bias (fa_fwd_bias, fa_bwd_bias)
against the fp64 oracle, through the C ABI.

Same tolerances as the core path for O, dQ, dK, dV and the logsumexp. dBias
(= dS, rounded to bf16) can reach magnitudes M of several units on short
rows where the bias concentrates the probability mass; its bf16 rounding
alone is then up to M * 2^-9, so it is held to the core bounds scaled by
max(1, M / 2) (M = max |dBias| of the reference), the same rule as for
outputs at non-default softmax scales. Bias
entries of -inf remove keys; a row that loses every key must come back as
o = 0, lse = -inf and contribute no gradient.
"""

import math
import sys

import numpy as np
import pytest

import exact_tiled_attention_37_amd as fa
import oracle
import seeded_inputs as si
from tests import parity_log

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL, LSE_TOL = 2e-2, 2e-3, 1e-3
NEG_INF_BF16 = 0xFF80


def announce(msg):
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def report(msg):
    """A whole-workload parity figure: printed now and in the session summary."""
    announce(msg)
    parity_log.record(msg)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")
    fa.load_library()


def dev(bits):
    return si.bits_to_torch(bits, "cuda")


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, got, ref, max_tol=MAX_TOL, mean_tol=MEAN_TOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    assert mx <= max_tol and mn <= mean_tol, (
        f"{name}: max-abs {mx:.3e} (tol {max_tol}), mean-abs {mn:.3e} (tol {mean_tol}), "
        f"at {np.unravel_index(int(err.argmax()), err.shape)}"
    )


def check_scaled(name, got, ref):
    m = max(1.0, float(np.max(np.abs(ref))) / 2.0)
    check(name, got, ref, MAX_TOL * m, MEAN_TOL * m)


def bias_device(bits):
    """bf16 bias bits [Bb, Hb, N, N] into a padded device view (rows of a
    multiple of 8 elements), the row padding filled with NaN so that a read
    of it would show."""
    import torch

    Bb, Hb, N, _ = bits.shape
    t = fa.padded_bias(Bb, Hb, N, "cuda")
    t.as_strided((Bb, Hb, N, t.stride(2)), t.stride()).fill_(float("nan"))
    t.copy_(si.bits_to_torch(bits, "cuda"))
    return t


def run_case(bits, bias_bits, causal, scale, with_bwd=True):
    import torch

    q, k, v, do = (dev(bits[n]) for n in ("q", "k", "v", "do"))
    bias = bias_device(bias_bits)
    o, lse = fa.fa_fwd_bias(q, k, v, bias, causal, scale)
    out = {"o": o, "lse": lse}
    if with_bwd:
        dq, dk, dv, db = fa.fa_bwd_bias(q, k, v, bias, o, lse, do, causal, scale)
        out.update(dq=dq, dk=dk, dv=dv, dbias=db)
    torch.cuda.synchronize()
    return out


def compare(out, ref):
    rq, rk, rv, rdb, ro, rl, _ = ref
    empty = np.isneginf(rl)
    lse = f64(out["lse"])
    assert np.array_equal(np.isneginf(lse), empty), "rows without a visible key differ"
    check("O", f64(out["o"]), ro)
    check("LSE", lse[~empty], rl[~empty], LSE_TOL, LSE_TOL)
    if "dq" in out:
        check("dQ", f64(out["dq"]), rq)
        check("dK", f64(out["dk"]), rk)
        check("dV", f64(out["dv"]), rv)
        check_scaled("dBias", f64(out["dbias"]), rdb)


def random_bias(B, H, N, seed, holes=True):
    return si.draw_bias_with_holes(B, H, N, seed, holes)


SMALL = [(1, 1, 1, 64), (1, 17, 2, 64), (2, 64, 2, 128), (1, 129, 3, 64), (1, 200, 2, 128), (2, 256, 1, 128),
         (1, 700, 2, 64), (1, 1000, 1, 128)]  # (the last two: many tiles, a ragged end)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dN%dH%dd%d" % s)
def test_bias_small(shape, causal):
    B, N, H, d = shape
    seed = 9100 + N + d + int(causal)
    scale = 1.0 / math.sqrt(d)
    announce(f"bias fwd+bwd shape={shape} causal={causal} seed={seed}")
    bits = si.draw(B, N, H, d, seed, backward=True)
    bias_bits = random_bias(B, H, N, seed + 1, holes=N > 1)
    ref = oracle.attention_backward_bias(*(si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v")),
                                         si.bf16_bits_to_f64(bias_bits), si.bf16_bits_to_f64(bits["do"]),
                                         causal, scale)
    compare(run_case(bits, bias_bits, causal, scale), ref)


@pytest.mark.parametrize("bcast", ["batch", "head", "both"])
def test_bias_broadcast(bcast):
    """One bias matrix shared across batches and/or heads: the forward uses
    it for every (batch, head); dBias comes back per (batch, head)."""
    B, N, H, d = 2, 100, 3, 64
    announce(f"bias broadcast over {bcast}")
    bits = si.draw(B, N, H, d, 9300, backward=True)
    Bb = 1 if bcast in ("batch", "both") else B
    Hb = 1 if bcast in ("head", "both") else H
    bias_bits = random_bias(Bb, Hb, N, 9301, holes=False)
    full = np.broadcast_to(si.bf16_bits_to_f64(bias_bits), (B, H, N, N)).copy()
    ref = oracle.attention_backward_bias(*(si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v")), full,
                                         si.bf16_bits_to_f64(bits["do"]), False, 0.125)
    compare(run_case(bits, bias_bits, False, 0.125), ref)


def test_bias_triangle_is_causal():
    """A -inf strictly-upper-triangular bias without the causal flag gives
    the causal result of the plain entry points."""
    import torch

    B, N, H, d = 1, 300, 2, 128
    announce("bias triangle vs causal")
    bits = si.draw(B, N, H, d, 9400, backward=True)
    tri = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], NEG_INF_BF16, 0).astype(np.uint16)
    bias_bits = np.broadcast_to(tri, (1, 1, N, N)).copy()
    out = run_case(bits, bias_bits, False, 1 / math.sqrt(d))
    q, k, v, do = (dev(bits[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, True)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, do, True)
    torch.cuda.synchronize()
    check("O vs causal", f64(out["o"]), f64(o))
    check("LSE vs causal", f64(out["lse"]), f64(lse), LSE_TOL, LSE_TOL)
    for name, a, b in (("dQ", out["dq"], dq), ("dK", out["dk"], dk), ("dV", out["dv"], dv)):
        check(f"{name} vs causal", f64(a), f64(b))
    db = f64(out["dbias"])[0, :, np.triu_indices(N, 1)[0], np.triu_indices(N, 1)[1]]
    assert np.all(db == 0.0), "dBias must be 0 where the bias hides the key"


def test_bias_causal_zero_fill():
    """Causal dBias: keys after the query are exactly 0, including the keys
    of tiles the kernels never visit; the row padding is left untouched."""
    import torch

    B, N, H, d = 1, 333, 1, 64
    announce("bias causal dBias zero fill")
    bits = si.draw(B, N, H, d, 9500, backward=True)
    bias_bits = random_bias(B, H, N, 9501, holes=False)
    q, k, v, do = (dev(bits[n]) for n in ("q", "k", "v", "do"))
    bias = bias_device(bias_bits)
    o, lse = fa.fa_fwd_bias(q, k, v, bias, True)
    dbias = fa.padded_bias(B, H, N, "cuda")
    full = dbias.as_strided((B, H, N, dbias.stride(2)), dbias.stride())
    full.fill_(7.0)
    fa.fa_bwd_bias(q, k, v, bias, o, lse, do, True, dbias=dbias)
    torch.cuda.synchronize()
    got = f64(full)
    upper = np.triu(np.ones((N, N), dtype=bool), 1)
    assert np.all(got[0, 0, :, :N][upper] == 0.0)
    assert np.all(got[0, 0, :, N:] == 7.0), "row padding was written"


@pytest.mark.parametrize("name", list(si.BIAS_WORKLOADS))
def test_bias_workload(name):
    """The bias workload at full size (as the benchmark runs it): O, LSE,
    dQ, dK, dV and dBias of every (batch, head) against the oracle (run head
    by head in a thread pool)."""
    from tests import oracle_heads as oh

    w = si.BIAS_WORKLOADS[name]
    announce(f"bias workload {name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    bits = si.draw_with_bias(w.B, w.N, w.H, w.d, w.seed)
    out = run_case(bits, bits["bias"], w.causal, w.scale)
    got = {k: f64(v) for k, v in out.items()}
    x = {n: si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v", "do")}
    bias = si.bf16_bits_to_f64(bits["bias"])
    H = oh.head

    def one(b, h):
        rq, rk, rv, rdb, ro, rl, _ = oracle.attention_backward_bias(
            H(x["q"], b, h), H(x["k"], b, h), H(x["v"], b, h), bias[b:b + 1, h:h + 1], H(x["do"], b, h),
            w.causal, w.scale)
        # dBias [1, 1, N, N] travels as a [1, N, 1, N] slice
        return rq, rk, rv, ro, rl, rdb.transpose(0, 2, 1, 3)

    rq, rk, rv, ro, rl, rdb = oh.by_head(one, w.B, w.H, ("bnhd", "bnhd", "bnhd", "bnhd", "bhn", "bnhd"))
    rdb = rdb.transpose(0, 2, 1, 3)
    for nm, g, r in (("O", got["o"], ro), ("dQ", got["dq"], rq), ("dK", got["dk"], rk), ("dV", got["dv"], rv),
                     ("dBias", got["dbias"], rdb), ("LSE", got["lse"], rl)):
        err = np.abs(g - r)
        report(f"[parity] {name} {nm}: max-abs {err.max():.3e} mean-abs {err.mean():.3e} over {err.size} elements")
    check("O", got["o"], ro)
    check("LSE", got["lse"], rl, LSE_TOL, LSE_TOL)
    check("dQ", got["dq"], rq)
    check("dK", got["dk"], rk)
    check("dV", got["dv"], rv)
    check_scaled("dBias", got["dbias"], rdb)
