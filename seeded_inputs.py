"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no attention arithmetic. It only draws random tensors,
rounds them to bfloat16 and decodes bfloat16 bit patterns, so that the
CPU oracle and the GPU library are fed the very same bits.

Recipe (stated once, used everywhere):
  * generator  numpy.random.Generator(PCG64(seed))
  * draw order Q, K, V, then dO (only when a backward is wanted); for
               decode shapes Q has Nq rows and K, V have Nk rows; a bias
               [B, H, N, N] is drawn last
  * each draw  standard_normal((B, N, H, d), dtype=float32), C order,
               then fp32 -> bf16 round-to-nearest-even, kept as uint16 bits.

The five benchmark workloads follow the attention-kernel sweep described in
the IPLEX blog post on FlashAttention-2 work partitioning (section "Read the
reported speed-ups with their conditions"): sequence length 512 to 16k, head
dimension 64 and 128, causal masking, 16k tokens per batch.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    backward: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The tiny case the oracle finishes in well under a second, then the four
# sweep points (16k tokens each) and the forward+backward training shape.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 128, 64, False, False, 1),
    "short_noncausal": Workload("short_noncausal", 32, 16, 512, 64, False, False, 2),
    "short_causal": Workload("short_causal", 32, 16, 512, 64, True, False, 2),
    "mid_causal": Workload("mid_causal", 8, 16, 2048, 128, True, False, 3),
    "long_causal": Workload("long_causal", 1, 16, 16384, 128, True, False, 4),
    "train_causal": Workload("train_causal", 4, 16, 4096, 128, True, True, 5),
}


@dataclass(frozen=True)
class DecodeWorkload:
    """A few new query rows (the last Nq positions) against Nk keys."""

    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# Decode-shaped workloads (the post's section "Document the implementation
# difference" sets decoding apart from prefill): one new token, a
# speculative block of 16, and a d = 64 case, each against a long history.
DECODE_WORKLOADS = {
    "decode_1x8k": DecodeWorkload("decode_1x8k", 16, 16, 1, 8192, 128, True, 6),
    "decode_16x16k": DecodeWorkload("decode_16x16k", 4, 16, 16, 16384, 128, True, 7),
    "decode_4x4k_d64": DecodeWorkload("decode_4x4k_d64", 32, 16, 4, 4096, 64, True, 8),
}


# Attention with an additive bias (a variant named on the related-papers page
# for "FlashAttention on a Napkin"): a dense bias matrix per (batch, head).
BIAS_WORKLOADS = {
    "bias_2k": Workload("bias_2k", 2, 16, 2048, 128, False, True, 9),
}


# FP8 (e4m3) forward workloads: the bf16 training shape (d = 128 and 64) and
# the long sequence, with Q, K, V given as e4m3 codes and a descale factor per
# (batch, head) (a low-precision attention variant named on the
# related-papers page for "FlashAttention on a Napkin").
FP8_WORKLOADS = {
    "fp8_train_causal": Workload("fp8_train_causal", 4, 16, 4096, 128, True, False, 10),
    "fp8_long_causal": Workload("fp8_long_causal", 1, 16, 16384, 128, True, False, 11),
    "fp8_train_causal_d64": Workload("fp8_train_causal_d64", 4, 16, 4096, 64, True, False, 14),
}

# Largest |value| an input is scaled to before rounding to e4m3 (of the 448
# the format holds), leaving headroom.
FP8_INPUT_AMAX = 224.0

# Microscaled FP8 forward workloads (the same shapes): Q, K, V as e4m3 codes
# with one E8M0 scale per 32 consecutive elements along the reduction
# dimension of the product each enters (Q and K: along d; V: along tokens).
MXFP8_WORKLOADS = {
    "mxfp8_train_causal": Workload("mxfp8_train_causal", 4, 16, 4096, 128, True, False, 12),
    "mxfp8_long_causal": Workload("mxfp8_long_causal", 1, 16, 16384, 128, True, False, 13),
    "mxfp8_train_causal_d64": Workload("mxfp8_train_causal_d64", 4, 16, 4096, 64, True, False, 15),
}
# Exponent of the largest power of two an e4m3 code holds (448 = 1.75 * 2^8):
# the OCP MX rule scales a block so that its largest magnitude lands in
# [2^8, 2^9) before rounding (values above 448 saturate).
E4M3_EMAX = 8


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round to nearest, ties to even); return uint16 bits.

    Only finite inputs are expected (normal samples)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float64."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def draw(B: int, N: int, H: int, d: int, seed: int, backward: bool = False):
    """Return a dict of uint16 bf16 bit arrays q, k, v (and do) of shape [B,N,H,d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    names = ["q", "k", "v"] + (["do"] if backward else [])
    out = {}
    for name in names:
        x = rng.standard_normal((B, N, H, d), dtype=np.float32)
        out[name] = f32_to_bf16_bits(x)
    return out


def draw_workload(w: Workload):
    return draw(w.B, w.N, w.H, w.d, w.seed, backward=w.backward)


def bits_to_torch(bits: np.ndarray, device=None):
    """View uint16 bf16 bits as a torch.bfloat16 tensor (optionally moved to a device)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    if device is not None:
        t = t.to(device)
    return t


def torch_to_bits(t) -> np.ndarray:
    """Copy a torch.bfloat16 tensor back to host uint16 bits."""
    import torch

    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def draw_qkv(B: int, Nq: int, Nk: int, H: int, d: int, seed: int):
    """Q [B, Nq, H, d] and K, V [B, Nk, H, d] as bf16 bits, drawn in that
    order from one PCG64 stream (same recipe as `draw`)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, n in (("q", Nq), ("k", Nk), ("v", Nk)):
        out[name] = f32_to_bf16_bits(rng.standard_normal((B, n, H, d), dtype=np.float32))
    return out


def draw_decode(w: DecodeWorkload):
    return draw_qkv(w.B, w.Nq, w.Nk, w.H, w.d, w.seed)


def draw_with_bias(B: int, N: int, H: int, d: int, seed: int):
    """Q, K, V, dO (as `draw` with backward=True), then a bias [B, H, N, N],
    all from one PCG64 stream, as bf16 bits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name in ("q", "k", "v", "do"):
        out[name] = f32_to_bf16_bits(rng.standard_normal((B, N, H, d), dtype=np.float32))
    out["bias"] = f32_to_bf16_bits(rng.standard_normal((B, H, N, N), dtype=np.float32))
    return out




def f64_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to the OCP FP8 E4M3 format (1 sign, 4 exponent bits with bias 7,
    3 mantissa bits, subnormals, largest finite 448, no infinities) with
    round-to-nearest-even, saturating at +-448; returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    a = np.minimum(np.abs(x), 448.0)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)          # 0 .. 8 (8 is the smallest normal)
    m, e = np.frexp(a[~sub])                                           # a = m * 2^e, m in [0.5, 1)
    e = e - 1                                                          # a = (2m) * 2^e, 2m in [1, 2)
    mq = np.rint((2.0 * m - 1.0) * 8.0).astype(np.int64)
    carry = mq == 8
    e = e + carry
    mq = np.where(carry, 0, mq)
    code[~sub] = ((e + 7) << 3) | mq
    return (np.minimum(code, 0x7E).astype(np.uint8) | sign).astype(np.uint8)


def draw_fp8(B: int, N: int, H: int, d: int, seed: int):
    """Q, K, V drawn as in `draw` (float32 N(0,1), one PCG64 stream), then for
    each tensor and each (batch, head) a descale factor D = max|x| / 224
    (float32) and e4m3 codes of x / D. Returns uint8 codes q, k, v
    [B, N, H, d] and float32 descales q_descale, k_descale, v_descale [B, H];
    the value a code stands for is D * e4m3(code)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name in ("q", "k", "v"):
        out[name], out[name + "_descale"] = quantize_e4m3(rng.standard_normal((B, N, H, d), dtype=np.float32))
    return out


def quantize_e4m3(x: np.ndarray):
    """float32 x [B, N, H, d] as e4m3 codes with one float32 descale per
    (batch, head), D = max|x| / 224: returns (codes, D [B, H])."""
    amax = np.abs(x).max(axis=(1, 3)).astype(np.float32)            # [B, H]
    desc = (amax / np.float32(FP8_INPUT_AMAX)).astype(np.float32)
    return f64_to_e4m3_bits(x.astype(np.float64) / desc.astype(np.float64)[:, None, :, None]), desc


def mx_scale_codes(amax: np.ndarray) -> np.ndarray:
    """E8M0 codes of the OCP MX shared scale for e4m3 blocks with largest
    magnitude amax: X = floor(log2(amax)) - 8, code X + 127 (clamped to
    0..254; an all-zero block takes code 0)."""
    a = np.asarray(amax, dtype=np.float64)
    x = np.floor(np.log2(np.where(a > 0, a, 1.0))) - E4M3_EMAX
    return np.where(a > 0, np.clip(x + 127, 0, 254), 0).astype(np.uint8)


def quantize_mx_rows(x: np.ndarray):
    """float32 x [B, N, H, d] as e4m3 codes with one E8M0 scale per 32
    consecutive elements of a token along d: returns (codes [B, N, H, d],
    scales [B, N, H, d / 32])."""
    B, N, H, d = x.shape
    xb = x.astype(np.float64).reshape(B, N, H, d // 32, 32)
    sc = mx_scale_codes(np.abs(xb).max(axis=4))
    codes = f64_to_e4m3_bits(xb / np.exp2(sc.astype(np.float64) - 127.0)[..., None])
    return codes.reshape(B, N, H, d), sc


def quantize_mx_cols(x: np.ndarray):
    """float32 x [B, N, H, d] as e4m3 codes with one E8M0 scale per 32
    consecutive tokens of a column (the last block holds N % 32 tokens when
    N is not a multiple of 32): returns (codes [B, N, H, d], scales
    [B, ceil(N / 32), H, d])."""
    B, N, H, d = x.shape
    nb = (N + 31) // 32
    xp = np.zeros((B, nb * 32, H, d))
    xp[:, :N] = x
    xb = xp.reshape(B, nb, 32, H, d)
    sc = mx_scale_codes(np.abs(xb).max(axis=2))
    codes = f64_to_e4m3_bits(xb / np.exp2(sc.astype(np.float64) - 127.0)[:, :, None])
    return np.ascontiguousarray(codes.reshape(B, nb * 32, H, d)[:, :N]), sc


def _mx_quantize(x):
    q, qs = quantize_mx_rows(x["q"])
    k, ks = quantize_mx_rows(x["k"])
    v, vs = quantize_mx_cols(x["v"])
    return {"q": q, "q_scale": qs, "k": k, "k_scale": ks, "v": v, "v_scale": vs}


def draw_mxfp8(B: int, N: int, H: int, d: int, seed: int):
    """Q, K, V drawn as in draw_fp8 (float32 N(0,1), one PCG64 stream, in the
    order Q, K, V), quantized with block scales: Q and K by quantize_mx_rows,
    V by quantize_mx_cols. Returns uint8 codes q, k, v and uint8 E8M0 scales
    q_scale, k_scale, v_scale."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _mx_quantize({n: rng.standard_normal((B, N, H, d), dtype=np.float32) for n in ("q", "k", "v")})


def draw_mxfp8_growing_scores(B: int, N: int, H: int, d: int, seed: int, span: float):
    """Q, K, V of growing_scores_f32 with block scales (as in draw_mxfp8)."""
    return _mx_quantize(growing_scores_f32(B, N, H, d, seed, span))


def growing_scores_f32(B: int, N: int, H: int, d: int, seed: int, span: float):
    """Q, K, V, dO (float32) whose scores grow along the keys: queries are
    1 + 0.1 z and key j is t_j + 0.1 z in every column, with t_j running
    linearly from -span to +span over the N keys (z standard normal), so a
    row's largest score keeps moving to later keys (by about span * d *
    scale * 2 / N per key). V and dO are standard normal. One PCG64 stream,
    draws in the order Q, K, V, dO."""
    rng = np.random.Generator(np.random.PCG64(seed))
    t = np.linspace(-span, span, N, dtype=np.float32)[None, :, None, None]
    q = 1.0 + 0.1 * rng.standard_normal((B, N, H, d), dtype=np.float32)
    k = t + 0.1 * rng.standard_normal((B, N, H, d), dtype=np.float32)
    v = rng.standard_normal((B, N, H, d), dtype=np.float32)
    do = rng.standard_normal((B, N, H, d), dtype=np.float32)
    return {"q": q, "k": k.astype(np.float32), "v": v, "do": do}


def draw_growing_scores(B: int, N: int, H: int, d: int, seed: int, span: float):
    """growing_scores_f32 rounded to bf16 bits."""
    x = growing_scores_f32(B, N, H, d, seed, span)
    return {n: f32_to_bf16_bits(x[n]) for n in ("q", "k", "v", "do")}


def draw_fp8_growing_scores(B: int, N: int, H: int, d: int, seed: int, span: float):
    """Q, K, V of growing_scores_f32 as e4m3 codes with per-(batch, head)
    descales (as in draw_fp8)."""
    x = growing_scores_f32(B, N, H, d, seed, span)
    out = {}
    for name in ("q", "k", "v"):
        out[name], out[name + "_descale"] = quantize_e4m3(x[name])
    return out


def draw_negative_logsumexp(B: int, N: int, H: int, d: int, seed: int):
    """Q, K, V, dO bits whose scores all sit far below zero: queries are
    -4 + 0.5 z and keys 4 + 0.5 z in every column (z standard normal), so a
    score is about -16 d times the softmax scale and every row's logsumexp
    lies far below -88 (where exp of its negative overflows float32). V and
    dO are standard normal. One PCG64 stream, draws in the order Q, K, V, dO."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = -4.0 + 0.5 * rng.standard_normal((B, N, H, d), dtype=np.float32)
    k = 4.0 + 0.5 * rng.standard_normal((B, N, H, d), dtype=np.float32)
    v = rng.standard_normal((B, N, H, d), dtype=np.float32)
    do = rng.standard_normal((B, N, H, d), dtype=np.float32)
    return {n: f32_to_bf16_bits(x) for n, x in zip(("q", "k", "v", "do"), (q, k, v, do))}


BF16_NEG_INF = 0xFF80  # bfloat16 bits of -inf


def draw_bias_with_holes(B: int, H: int, N: int, seed: int, holes: bool = True):
    """A bf16 bias [B, H, N, N] of 1.5 z (z standard normal, PCG64(seed));
    with holes, three -inf patterns: part of row 1 of (0, 0) removed, the
    last row of (B-1, H-1) fully removed, and key 2 of (0, H-1) hidden from
    every row."""
    rng = np.random.Generator(np.random.PCG64(seed))
    b = f32_to_bf16_bits((rng.standard_normal((B, H, N, N)) * 1.5).astype(np.float32))
    if holes:
        b[0, 0, min(1, N - 1), : max(1, N // 3)] = BF16_NEG_INF
        b[-1, -1, N - 1, :] = BF16_NEG_INF
        b[0, -1, :, min(2, N - 1)] = BF16_NEG_INF
    return b
