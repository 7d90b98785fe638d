"""CPU tests of the fp64 oracle against its pins (no GPU needed).

Besides running every pin against the oracle, this file plants plausible
mistakes in a copy of the oracle's source (a dropped scale, a wrong mask
index, a transposed operand, a flipped sign, ...) and requires each such
mutant to fail at least one pin, so the pins are shown to be sensitive.
"""

import contextlib
import importlib.util
import os
import types

import numpy as np
import pytest

import oracle
import oracle.attention as oracle_attention
import seeded_inputs as si
from tests import oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(oracle_attention.__file__), "attention.py")


@contextlib.contextmanager
def chunk_limit(mod, elems):
    """Force the oracle's row-chunking path with a tiny chunk bound."""
    old = mod._MAX_CHUNK_ELEMS
    mod._MAX_CHUNK_ELEMS = elems
    try:
        yield
    finally:
        mod._MAX_CHUNK_ELEMS = old


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_attention)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin_chunked(pin):
    """Same pins with query rows processed a few at a time."""
    with chunk_limit(oracle_attention, 24):
        pin(oracle_attention)


# (name, text in the oracle source, planted replacement)
MUTATIONS = [
    ("scale dropped", "s = scale * (qh @ kh.T)\n", "s = (qh @ kh.T)\n"),
    ("scale squared", "s = scale * (qh @ kh.T)\n", "s = scale * scale * (qh @ kh.T)\n"),
    ("diagonal masked", "np.where(kj > qi,", "np.where(kj >= qi,"),
    ("wrong triangle", "np.where(kj > qi,", "np.where(kj < qi,"),
    ("chunk offset lost", "qi = np.arange(row0, row0 + s.shape[0])", "qi = np.arange(0, s.shape[0])"),
    ("scores transposed", "s = scale * (qh @ kh.T)\n", "s = scale * (kh @ qh.T)\n"),
    ("max over columns", "m = s.max(axis=1, keepdims=True)", "m = s.max(axis=0, keepdims=True)"),
    ("sum over columns", "l = e.sum(axis=1, keepdims=True)", "l = e.sum(axis=0, keepdims=True)"),
    ("P transposed in PV", "o[b, r0:r1, h, :] = p @ vh\n                with np.errstate(divide=\"ignore\"):\n                    lse[b, h, r0:r1] = m + np.log(l)",
     "o[b, r0:r1, h, :] = p.T @ vh\n                with np.errstate(divide=\"ignore\"):\n                    lse[b, h, r0:r1] = m + np.log(l)"),
    ("lse without max", "lse[b, h, r0:r1] = m + np.log(l)\n    return o, lse",
     "lse[b, h, r0:r1] = np.log(l)\n    return o, lse"),
    ("lse base 2", "lse[b, h, r0:r1] = m + np.log(l)\n    return o, lse",
     "lse[b, h, r0:r1] = m + np.log2(l)\n    return o, lse"),
    ("dS sign", "ds = p * (dp - drow[:, None])", "ds = p * (dp + drow[:, None])"),
    ("D dropped", "ds = p * (dp - drow[:, None])", "ds = p * dp"),
    ("D from dP", "drow = np.sum(doh[r0:r1] * oc, axis=1)", "drow = np.sum(dp, axis=1)"),
    ("dP transposed", "dp = doh[r0:r1] @ vh.T", "dp = (vh @ doh[r0:r1].T).T[:, ::-1]"),
    ("dQ unscaled", "dq[b, r0:r1, h, :] = scale * (ds @ kh)", "dq[b, r0:r1, h, :] = (ds @ kh)"),
    ("dQ uses Q", "dq[b, r0:r1, h, :] = scale * (ds @ kh)", "dq[b, r0:r1, h, :] = scale * (ds @ qh)"),
    ("dK not transposed", "dk[b, :, h, :] += scale * (ds.T @ qh[r0:r1])",
     "dk[b, :, h, :] += scale * (ds @ qh[r0:r1])"),
    ("dK unscaled", "dk[b, :, h, :] += scale * (ds.T @ qh[r0:r1])", "dk[b, :, h, :] += (ds.T @ qh[r0:r1])"),
    ("dV not transposed", "dv[b, :, h, :] += p.T @ doh[r0:r1]", "dv[b, :, h, :] += p @ doh[r0:r1]"),
    ("dV overwritten per chunk", "dv[b, :, h, :] += p.T @ doh[r0:r1]", "dv[b, :, h, :] = p.T @ doh[r0:r1]"),
    ("sampled row offset", "s = _scores(qi, kh, int(i), causal, scale)", "s = _scores(qi, kh, 0, causal, scale)"),
    ("chunk mask includes the diagonal", "s = np.where(kpos > qpos, -np.inf, s)", "s = np.where(kpos >= qpos, -np.inf, s)"),
    ("chunk mask flipped", "s = np.where(kpos > qpos, -np.inf, s)", "s = np.where(kpos < qpos, -np.inf, s)"),
    ("chunk query offset from keys", "qpos = (q_start + np.arange(r0, r1))[:, None]",
     "qpos = (k_start + np.arange(r0, r1))[:, None]"),
    ("chunk row offset lost", "qpos = (q_start + np.arange(r0, r1))[:, None]",
     "qpos = (q_start + np.arange(0, r1 - r0))[:, None]"),
    ("chunk key offset ignored", "kpos = (k_start + np.arange(Nk))[None, :]", "kpos = np.arange(Nk)[None, :]"),
    ("chunk P transposed", "o[b, r0:r1, h, :] = p @ vh\n                with np.errstate(divide=\"ignore\"):\n                    lse[b, h, r0:r1] = np.where(",
     "o[b, r0:r1, h, :] = p[::-1] @ vh\n                with np.errstate(divide=\"ignore\"):\n                    lse[b, h, r0:r1] = np.where("),
    ("empty chunk lse zero", "lse = np.full((B, H, Nq), -np.inf)", "lse = np.zeros((B, H, Nq))"),
    ("merge lse without max", "lse = np.where(tot > 0, mx_safe + np.log(", "lse = np.where(tot > 0, np.log("),
    ("merge weights unnormalised", "frac = np.where(tot[None] > 0, w / np.where(tot > 0, tot, 1.0)[None], 0.0)",
     "frac = np.where(tot[None] > 0, w, 0.0)"),
    ("merge weights not shifted", "w = np.exp(lse_parts - mx_safe[None])", "w = np.exp(lse_parts)"),
    ("merge output layout", 'o = np.einsum("cbhn,cbnhd->bnhd", frac, o_parts)', 'o = np.einsum("cbhn,cbnhd->bnhd", frac[::-1], o_parts)'),
    ("decode top-left alignment", "return attention_forward_chunk(q, k, v, causal, scale, q_start=nk - nq, k_start=0)",
     "return attention_forward_chunk(q, k, v, causal, scale, q_start=0, k_start=0)"),
    ("decode offset off by one", "return attention_forward_chunk(q, k, v, causal, scale, q_start=nk - nq, k_start=0)",
     "return attention_forward_chunk(q, k, v, causal, scale, q_start=nk - nq - 1, k_start=0)"),
    ("bias before the scale", "s = scale * (qh @ kh.T) + bh", "s = scale * (qh @ kh.T + bh)"),
    ("bias transposed", "s = scale * (qh @ kh.T) + bh", "s = scale * (qh @ kh.T) + bh.T[: qh.shape[0], : kh.shape[0]]"),
    ("bias sign", "s = scale * (qh @ kh.T) + bh", "s = scale * (qh @ kh.T) - bh"),
    ("dBias from P", "dbias[b, h, r0:r1] = ds", "dbias[b, h, r0:r1] = p"),
    ("dBias scaled", "dbias[b, h, r0:r1] = ds", "dbias[b, h, r0:r1] = scale * ds"),
    ("bias causal mask dropped", "        s = np.where(kj > qi, -np.inf, s)\n    return s\n\n\ndef attention_forward_bias",
     "        s = s\n    return s\n\n\ndef attention_forward_bias"),
    ("bias row chunk offset", "s = _bias_scores(qh[r0:r1], kh, bias[b, h, r0:r1], r0, causal, scale)\n                p, m, l = _softmax_rows(s)\n                o[b, r0:r1, h, :] = p @ vh",
     "s = _bias_scores(qh[r0:r1], kh, bias[b, h, 0:r1 - r0], r0, causal, scale)\n                p, m, l = _softmax_rows(s)\n                o[b, r0:r1, h, :] = p @ vh"),
    ("bias dS sign", "ds = p * (dp - drow[:, None])\n                dbias[b, h, r0:r1] = ds",
     "ds = p * (dp + drow[:, None])\n                dbias[b, h, r0:r1] = ds"),
    ("bias dV not transposed", "dv[b, :, h, :] += p.T @ doh[r0:r1]\n    return dq, dk, dv, dbias",
     "dv[b, :, h, :] += p @ doh[r0:r1]\n    return dq, dk, dv, dbias"),
    ("bias dK unscaled", "dk[b, :, h, :] += scale * (ds.T @ qh[r0:r1])\n                dv[b, :, h, :] += p.T @ doh[r0:r1]\n    return dq, dk, dv, dbias",
     "dk[b, :, h, :] += (ds.T @ qh[r0:r1])\n                dv[b, :, h, :] += p.T @ doh[r0:r1]\n    return dq, dk, dv, dbias"),
    ("e4m3 exponent bias", "(1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)",
     "(1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 8.0)"),
    ("e4m3 subnormal scale", "np.where(e == 0, m * 2.0 ** -9,", "np.where(e == 0, m * 2.0 ** -10,"),
    ("e4m3 sign ignored", "sign = np.where(c & 0x80, -1.0, 1.0)", "sign = np.where(c & 0x80, 1.0, 1.0)"),
    ("fp8 Q takes the K descale", "return attention_forward(dequantize_fp8(q8, q_descale),",
     "return attention_forward(dequantize_fp8(q8, k_descale),"),
    ("fp8 V descale dropped", "dequantize_fp8(v8, v_descale), causal, scale)", "dequantize_fp8(v8, v_descale * 0 + 1), causal, scale)"),
    ("e8m0 bias 128", "np.exp2(c.astype(np.float64) - 127.0))", "np.exp2(c.astype(np.float64) - 128.0))"),
    ("e8m0 NaN code", "np.where(c == 255, np.nan,", "np.where(c == 254, np.nan,"),
    ("mx V block offset", "np.repeat(e8m0_decode(scales), 32, axis=1)[:, :n]", "np.repeat(e8m0_decode(scales), 32, axis=1)[:, 1:n + 1]"),
    ("mx row blocks interleaved", "np.repeat(e8m0_decode(scales), 32, axis=3)", "np.tile(e8m0_decode(scales), (1, 1, 1, 32))"),
    ("mx K takes the Q scales", "dequantize_mx_rows(k8, k_scale)", "dequantize_mx_rows(k8, q_scale)"),
    ("mx V scales dropped", "dequantize_mx_cols(v8, v_scale), causal, scale)", "dequantize_mx_cols(v8, v_scale * 0 + 127), causal, scale)"),
    ("head slice swapped", "sl = (slice(b, b + 1), slice(None), slice(h, h + 1), slice(None))",
     "sl = (slice(h, h + 1), slice(None), slice(b, b + 1), slice(None))"),
]


def _load_mutant(old, new):
    """The oracle with the first occurrence of `old` replaced (functions that
    repeat a line plant it in the earliest one; later copies have mutations
    of their own with longer, unique anchors)."""
    src = open(ORACLE_SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), ORACLE_SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


def _survives(mod):
    for chunk in (None, 24):
        for pin in pins.ALL_PINS:
            ctx = chunk_limit(mod, chunk) if chunk else contextlib.nullcontext()
            try:
                with ctx, np.errstate(all="ignore"):
                    pin(mod)
            except Exception:
                return False
    return True


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    assert not _survives(_load_mutant(old, new)), f"mutant '{name}' passed every pin"


def _blockwise_normalised(q, k, v, causal, scale, block):
    """The wrong computation the pages warn against: softmax each key block on
    its own, then add the block outputs."""
    B, N, H, d = q.shape
    o = np.zeros((B, N, H, d))
    for b in range(B):
        for h in range(H):
            s = scale * q[b, :, h, :] @ k[b, :, h, :].T
            if causal:
                s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
            for j0 in range(0, N, block):
                sb = s[:, j0 : j0 + block]
                m = sb.max(axis=1, keepdims=True)
                m = np.where(np.isfinite(m), m, 0.0)
                e = np.exp(sb - m)
                den = e.sum(axis=1, keepdims=True)
                p = np.where(den > 0, e / np.where(den > 0, den, 1), 0.0)
                o[b, :, h, :] += p @ v[b, j0 : j0 + block, h, :]
    return o


@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_normalisation_is_not_attention(causal):
    """Normalising each key block independently and adding the results is not
    the same calculation (IPLEX blog, 'Tiling preserves the attention
    calculation'): on the tiny workload it must miss the tolerance by far."""
    w = si.WORKLOADS["tiny"]
    bits = si.draw_workload(w)
    q, k, v = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v"))
    o, _ = oracle.attention_forward(q, k, v, causal, w.scale)
    wrong = _blockwise_normalised(q, k, v, causal, w.scale, 64)
    assert np.max(np.abs(wrong - o)) > 0.5
    assert np.mean(np.abs(wrong - o)) > 2e-2


def test_bf16_rounding_matches_torch():
    """The generator's fp32 -> bf16 rounding is round-to-nearest-even: it agrees
    bit for bit with torch's conversion, including ties."""
    import torch

    rng = np.random.Generator(np.random.PCG64(7))
    x = rng.standard_normal(1 << 16, dtype=np.float32) * np.float32(3.0)
    ties = (np.arange(1, 2049, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1e-30, 65504.0])])
    ours = si.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = si.bf16_bits_to_f64(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_generator_is_deterministic_and_ordered():
    a = si.draw(1, 5, 2, 4, seed=3, backward=True)
    b = si.draw(1, 5, 2, 4, seed=3, backward=True)
    for n in ("q", "k", "v", "do"):
        assert np.array_equal(a[n], b[n])
    c = si.draw(1, 5, 2, 4, seed=3, backward=False)
    for n in ("q", "k", "v"):
        assert np.array_equal(a[n], c[n])
    assert not np.array_equal(a["q"], a["k"])


@pytest.mark.parametrize("name", ["tiny", "train_causal"])
def test_bf16_floor_below_tolerance(name):
    """Rounding the exact outputs to bf16 alone stays well inside the parity
    tolerance, so the tolerance leaves room for the kernel's own rounding."""
    w = si.WORKLOADS[name]
    B = 1
    H = 1 if name == "train_causal" else w.H
    bits = si.draw(B, w.N, w.H, w.d, w.seed, backward=True)
    q, k, v, do = (si.bf16_bits_to_f64(bits[n][:, :, :H]) for n in ("q", "k", "v", "do"))
    dq, dk, dv, o, lse, _ = oracle.attention_backward(q, k, v, do, w.causal, w.scale)
    for t in (o, dq, dk, dv):
        floor = np.abs(si.bf16_bits_to_f64(si.f32_to_bf16_bits(t.astype(np.float32))) - t)
        assert floor.max() < 0.5 * 2e-2 and floor.mean() < 0.5 * 2e-3
