"""fp64 CPU oracle for exact scaled-dot-product attention (forward and backward).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library.

What it computes, and where that comes from
-------------------------------------------
The pages describe attention in words only: tokens' representations are
compared and each one's information is weighted (IPLEX blog post on
FlashAttention-2 GPU work partitioning, section "Why long inputs put pressure
on memory"). The conventional way, which this oracle follows on purpose,
materialises the full score and probability matrices (same section; also the
FlashAttention-2 abstract on the "High-Bandwidth Memory" keyword page: runtime
and memory quadratic in sequence length). The tiled method must reach the same
globally normalised result (section "Tiling preserves the attention
calculation"), so the oracle is that plain definition written out:

    S = scale * Q K^T                     (N x N, fp64)
    causal: S[i, j] = -inf for j > i      (key j visible to query i iff j <= i)
    P = softmax over each row of S        (m = row max, l = sum exp(S - m))
    O = P V,   L = m + ln(l)              (natural-log logsumexp of scaled scores)

The pages print no formula, so this is the plain reading: softmax(scale*QK^T)V
with a caller-supplied scale (the benchmark uses 1/sqrt(d)).

Backward (the pages require gradients to match within tolerance, same
"Tiling" section; they give no equations). With the loss taken as sum(dO * O):

    dV = P^T dO
    dP = dO V^T
    D  = rowsum(dO * O)                   (equals rowsum(P * dP))
    dS = P * (dP - D)
    dQ = scale * dS K,   dK = scale * dS^T Q

Gradients are with respect to the unscaled inputs, hence the factor `scale`
on dQ and dK. D is taken from the oracle's own fp64 O.

Layout: Q, K, V, dO, O, dQ, dK, dV are float64 [B, N, H, d]; L is [B, H, N].
Rows of S may be processed in chunks to bound memory. Each chunk holds whole
rows of S, so every row's softmax is exactly the definition above; dK and dV
are sums over query rows and are accumulated chunk by chunk.
"""

from __future__ import annotations

import numpy as np

# Upper bound on elements of one fp64 score chunk (256 MiB).
_MAX_CHUNK_ELEMS = 1 << 25


def _row_chunks(n_rows: int, n_cols: int):
    rows = max(1, min(n_rows, _MAX_CHUNK_ELEMS // max(1, n_cols)))
    for r0 in range(0, n_rows, rows):
        yield r0, min(n_rows, r0 + rows)


def _scores(qh: np.ndarray, kh: np.ndarray, row0: int, causal: bool, scale: float) -> np.ndarray:
    """Scaled scores for query rows row0.. of one head, causal mask applied as -inf."""
    s = scale * (qh @ kh.T)
    if causal:
        qi = np.arange(row0, row0 + s.shape[0])[:, None]
        kj = np.arange(kh.shape[0])[None, :]
        s = np.where(kj > qi, -np.inf, s)
    return s


def _softmax_rows(s: np.ndarray):
    """Row softmax of a score block; returns (P, m, l).

    A row whose scores are all -inf (impossible for N_q = N_k causal, since key
    i is always visible to query i) yields P = 0 and m = -inf."""
    m = s.max(axis=1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)
    l = e.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)
    return p, m[:, 0], l[:, 0]


def _check(q, k, v):
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, N, H, d] shape")


def attention_forward(q, k, v, causal: bool, scale: float):
    """Forward pass. Returns (O [B,N,H,d], L [B,H,N]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    _check(q, k, v)
    B, N, H, d = q.shape
    o = np.zeros((B, N, H, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            qh, kh, vh = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :]
            for r0, r1 in _row_chunks(N, N):
                s = _scores(qh[r0:r1], kh, r0, causal, scale)
                p, m, l = _softmax_rows(s)
                o[b, r0:r1, h, :] = p @ vh
                with np.errstate(divide="ignore"):
                    lse[b, h, r0:r1] = m + np.log(l)
    return o, lse


def attention_forward_rows(q, k, v, causal: bool, scale: float, b: int, h: int, rows):
    """Forward outputs for selected query rows of one (batch, head).

    Each requested row is computed from its full score row, exactly as in
    `attention_forward`; this lets a test check sampled outputs of a problem
    too large to evaluate whole. Returns (O rows [len(rows), d], L rows)."""
    rows = np.asarray(rows, dtype=np.int64)
    kh = np.asarray(k[b, :, h, :], dtype=np.float64)
    vh = np.asarray(v[b, :, h, :], dtype=np.float64)
    o_rows = np.zeros((rows.size, kh.shape[1]))
    l_rows = np.zeros(rows.size)
    for t, i in enumerate(rows):
        qi = np.asarray(q[b, i : i + 1, h, :], dtype=np.float64)
        s = _scores(qi, kh, int(i), causal, scale)
        p, m, l = _softmax_rows(s)
        o_rows[t] = (p @ vh)[0]
        l_rows[t] = m[0] + np.log(l[0])
    return o_rows, l_rows


def attention_backward(q, k, v, do, causal: bool, scale: float):
    """Analytic backward of sum(dO * O). Returns (dQ, dK, dV, O, L, D).

    O, L are the forward outputs (fp64); D = rowsum(dO * O) is [B, H, N]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have the shape of Q")
    B, N, H, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    o = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    dsum = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :]
            for r0, r1 in _row_chunks(N, N):
                s = _scores(qh[r0:r1], kh, r0, causal, scale)
                p, m, l = _softmax_rows(s)
                oc = p @ vh
                o[b, r0:r1, h, :] = oc
                with np.errstate(divide="ignore"):
                    lse[b, h, r0:r1] = m + np.log(l)
                dp = doh[r0:r1] @ vh.T
                drow = np.sum(doh[r0:r1] * oc, axis=1)
                dsum[b, h, r0:r1] = drow
                ds = p * (dp - drow[:, None])
                dq[b, r0:r1, h, :] = scale * (ds @ kh)
                dk[b, :, h, :] += scale * (ds.T @ qh[r0:r1])
                dv[b, :, h, :] += p.T @ doh[r0:r1]
    return dq, dk, dv, o, lse, dsum


def attention_backward_head(q, k, v, do, causal: bool, scale: float, b: int, h: int):
    """Backward restricted to one (batch, head); returns (dQ, dK, dV) as [N, d].

    Heads are independent, so this equals the matching slice of
    `attention_backward` and lets a test check sampled heads of a large
    problem."""
    sl = (slice(b, b + 1), slice(None), slice(h, h + 1), slice(None))
    dq, dk, dv, _, _, _ = attention_backward(q[sl], k[sl], v[sl], do[sl], causal, scale)
    return dq[0, :, 0, :], dk[0, :, 0, :], dv[0, :, 0, :]


# ---------------------------------------------------------------------------
# Key-range chunks and their merge.
#
# The Ring Attention entry on the "High-Bandwidth Memory" keyword page
# describes attention computed block by block: each device keeps its own
# query block while key/value blocks circulate, and every pass attends the
# local queries to one key/value block. The IPLEX post (section "Tiling
# preserves the attention calculation") states that such blocks must
# combine into the globally normalised result. The pages print no formula
# for the combination; the plain reading, written out here, is that a chunk
# is ordinary attention restricted to its keys, reported with its own
# logsumexp, and that chunks combine by weighting each chunk's normalised
# output with its share of the total softmax mass:
#
#     chunk c over keys K_c:  O_c = softmax(S[:, K_c]) V[K_c],
#                             L_c = ln sum_{j in K_c} exp(S[:, j])
#     merge:  L = ln sum_c exp(L_c),   O = sum_c exp(L_c - L) O_c
#
# Positions are global: query row i of a chunk sits at q_start + i and key
# row j at k_start + j; with the causal mask key j is visible to query i iff
# k_start + j <= q_start + i. A row that sees no key of a chunk has O_c = 0
# and L_c = -inf (it carries no mass); a row that sees no key of any chunk
# merges to O = 0 and L = -inf.


def attention_forward_chunk(q, k, v, causal: bool, scale: float, q_start: int = 0, k_start: int = 0):
    """Attention of a query chunk (rows at global positions q_start..) over a
    key chunk (positions k_start..). q is [B, Nq, H, d]; k and v are
    [B, Nk, H, d]. Returns (O_c [B, Nq, H, d], L_c [B, H, Nq]) in float64,
    with O_c = 0 and L_c = -inf for rows that see no key of the chunk."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.shape != v.shape or k.ndim != 4 or q.shape[0] != k.shape[0] or q.shape[2:] != k.shape[2:]:
        raise ValueError("q must be [B, Nq, H, d] and k, v [B, Nk, H, d]")
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    o = np.zeros((B, Nq, H, d))
    lse = np.full((B, H, Nq), -np.inf)
    if Nk == 0:
        return o, lse
    for b in range(B):
        for h in range(H):
            qh, kh, vh = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :]
            for r0, r1 in _row_chunks(Nq, Nk):
                s = scale * (qh[r0:r1] @ kh.T)
                if causal:
                    qpos = (q_start + np.arange(r0, r1))[:, None]
                    kpos = (k_start + np.arange(Nk))[None, :]
                    s = np.where(kpos > qpos, -np.inf, s)
                p, m, l = _softmax_rows(s)
                o[b, r0:r1, h, :] = p @ vh
                with np.errstate(divide="ignore"):
                    lse[b, h, r0:r1] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def merge_chunks(o_parts, lse_parts):
    """Combine chunk results over disjoint key sets: o_parts [C, B, Nq, H, d],
    lse_parts [C, B, H, Nq] (natural log, -inf for an empty chunk row).
    Returns (O [B, Nq, H, d], L [B, H, Nq]) in float64."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    if o_parts.ndim != 5 or lse_parts.ndim != 4 or o_parts.shape[0] != lse_parts.shape[0]:
        raise ValueError("o_parts must be [C, B, Nq, H, d] and lse_parts [C, B, H, Nq]")
    C, B, Nq, H, d = o_parts.shape
    if lse_parts.shape != (C, B, H, Nq):
        raise ValueError("lse_parts must be [C, B, H, Nq]")
    mx = lse_parts.max(axis=0)                                  # [B, H, Nq]
    mx_safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lse_parts - mx_safe[None])                       # exp(-inf) = 0 for empty rows
    tot = w.sum(axis=0)                                         # [B, H, Nq]
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(tot > 0, mx_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
        frac = np.where(tot[None] > 0, w / np.where(tot > 0, tot, 1.0)[None], 0.0)  # [C, B, H, Nq]
    o = np.einsum("cbhn,cbnhd->bnhd", frac, o_parts)
    return o, lse


# ---------------------------------------------------------------------------
# Decode-shaped attention: a few new query rows against a long key/value
# history. The IPLEX post (section "Document the implementation
# difference") separates prefill from decoding as workloads with different
# bottlenecks but fixes no convention for the causal mask when the query and
# key lengths differ. The plain reading, used here, is that the Nq queries
# are the last Nq positions of the sequence the Nk keys cover (bottom-right
# alignment): query row i sits at position Nk - Nq + i and sees key j iff
# j <= Nk - Nq + i. That is the key-chunk definition above with
# q_start = Nk - Nq and k_start = 0.


def attention_decode(q, k, v, causal: bool, scale: float):
    """Decode-shaped attention: q [B, Nq, H, d] as the last Nq positions of
    the sequence of k, v [B, Nk, H, d]. Returns (O [B, Nq, H, d],
    L [B, H, Nq]) in float64; with Nq > Nk the first Nq - Nk rows see no key
    (O = 0, L = -inf)."""
    nq, nk = np.shape(q)[1], np.shape(k)[1]
    return attention_forward_chunk(q, k, v, causal, scale, q_start=nk - nq, k_start=0)


# ---------------------------------------------------------------------------
# Attention with an additive bias. One of the abstracts on the related-papers
# page for "FlashAttention on a Napkin" describes attention with bias as
# standard attention whose query-key scores receive an additive bias matrix
# carrying prior knowledge. The page gives no formula; the plain reading is
#
#     S = scale * Q K^T + Bias            (Bias [B, H, N, N], added after scaling)
#     causal: S[i, j] = -inf for j > i    (on top of the bias)
#     O = softmax(S) V,  L = logsumexp(S) (natural log)
#
# and, with the loss sum(dO * O), since dS is the gradient of the loss with
# respect to S and S depends on Bias with unit weight:
#
#     dBias = dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q,
#     dV = P^T dO  (as without bias).
#
# A bias entry of -inf removes that key for that query; a row whose every
# score is -inf gets O = 0 and L = -inf and contributes no gradient.


def _bias_scores(qh, kh, bh, row0, causal, scale):
    s = scale * (qh @ kh.T) + bh
    if causal:
        qi = np.arange(row0, row0 + s.shape[0])[:, None]
        kj = np.arange(kh.shape[0])[None, :]
        s = np.where(kj > qi, -np.inf, s)
    return s


def attention_forward_bias(q, k, v, bias, causal: bool, scale: float):
    """Forward with an additive bias [B, H, N, N] (float64, may hold -inf).
    Returns (O [B, N, H, d], L [B, H, N])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    _check(q, k, v)
    B, N, H, d = q.shape
    if bias.shape != (B, H, N, N):
        raise ValueError("bias must be [B, H, N, N]")
    o = np.zeros((B, N, H, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            qh, kh, vh = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :]
            for r0, r1 in _row_chunks(N, N):
                s = _bias_scores(qh[r0:r1], kh, bias[b, h, r0:r1], r0, causal, scale)
                p, m, l = _softmax_rows(s)
                o[b, r0:r1, h, :] = p @ vh
                with np.errstate(divide="ignore"):
                    lse[b, h, r0:r1] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def attention_backward_bias(q, k, v, bias, do, causal: bool, scale: float):
    """Backward of sum(dO * O) for the biased forward. Returns
    (dQ, dK, dV, dBias [B, H, N, N], O, L, D)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    _check(q, k, v)
    B, N, H, d = q.shape
    if bias.shape != (B, H, N, N) or do.shape != q.shape:
        raise ValueError("bias must be [B, H, N, N] and dO shaped like Q")
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    dbias = np.zeros((B, H, N, N))
    o = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    dsum = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :]
            for r0, r1 in _row_chunks(N, N):
                s = _bias_scores(qh[r0:r1], kh, bias[b, h, r0:r1], r0, causal, scale)
                p, m, l = _softmax_rows(s)
                oc = p @ vh
                o[b, r0:r1, h, :] = oc
                with np.errstate(divide="ignore"):
                    lse[b, h, r0:r1] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
                dp = doh[r0:r1] @ vh.T
                drow = np.sum(doh[r0:r1] * oc, axis=1)
                dsum[b, h, r0:r1] = drow
                ds = p * (dp - drow[:, None])
                dbias[b, h, r0:r1] = ds
                dq[b, r0:r1, h, :] = scale * (ds @ kh)
                dk[b, :, h, :] += scale * (ds.T @ qh[r0:r1])
                dv[b, :, h, :] += p.T @ doh[r0:r1]
    return dq, dk, dv, dbias, o, lse, dsum


# ---------------------------------------------------------------------------
# FP8 (e4m3) inputs. The related-papers page for "FlashAttention on a Napkin"
# lists an abstract on low-precision attention that runs attention on the
# narrow-format matrix units of a newer GPU to accelerate it; the MI355X
# analogue is the FP8 matrix unit. The page fixes no format or scaling; the
# plain reading taken here: Q, K and V arrive as OCP FP8 E4M3 codes together
# with one float32 descale factor per (batch, head) and tensor, a code c
# standing for descale * e4m3(c); attention is then computed exactly on those
# values (the oracle below). How much the low-precision arithmetic inside a
# kernel may move the result is a separate, derived bound (see the tests).


def e4m3_decode(codes):
    """Values of OCP FP8 E4M3 codes: 1 sign bit, 4 exponent bits (bias 7), 3
    mantissa bits; exponent field 0 is subnormal (mantissa * 2^-9); codes
    0x7F and 0xFF are NaN; there are no infinities."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def dequantize_fp8(codes, descale):
    """codes [B, N, H, d] (uint8) and descale [B, H] -> float64 values."""
    return e4m3_decode(codes) * np.asarray(descale, dtype=np.float64)[:, None, :, None]


def attention_forward_fp8(q8, k8, v8, q_descale, k_descale, v_descale, causal: bool, scale: float):
    """Attention on FP8 inputs: the plain forward on the dequantized values.
    Returns (O [B, N, H, d], L [B, H, N]) in float64."""
    return attention_forward(dequantize_fp8(q8, q_descale), dequantize_fp8(k8, k_descale),
                             dequantize_fp8(v8, v_descale), causal, scale)


# Microscaled FP8 inputs. The same abstract speaks of narrow-format matrix
# units; the MI355X ones take, besides the FP8 codes, one power-of-two scale
# per block of 32 consecutive elements along the reduction dimension (the OCP
# Microscaling (MX) layout: the scale is an 8-bit exponent, E8M0, standing for
# 2^(code - 127), code 255 being NaN). Reading: Q and K carry one scale per
# 32 consecutive head-dimension elements of a token (the reduction of
# Q K^T), V one per 32 consecutive tokens of a head-dimension column (the
# reduction of P V); attention is computed exactly on the values the codes and
# scales stand for.


def e8m0_decode(codes):
    """Values of E8M0 scale codes: 2^(code - 127) for codes 0..254, NaN for 255."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.exp2(c.astype(np.float64) - 127.0))


def dequantize_mx_rows(codes, scales):
    """codes [B, N, H, d] (e4m3) and scales [B, N, H, d / 32] (E8M0): element
    (b, n, h, i) stands for e4m3(code) * 2^(scales[b, n, h, i // 32] - 127)."""
    return e4m3_decode(codes) * np.repeat(e8m0_decode(scales), 32, axis=3)


def dequantize_mx_cols(codes, scales):
    """codes [B, N, H, d] (e4m3) and scales [B, ceil(N / 32), H, d] (E8M0):
    element (b, n, h, i) stands for e4m3(code) * 2^(scales[b, n // 32, h, i] - 127)."""
    n = np.asarray(codes).shape[1]
    return e4m3_decode(codes) * np.repeat(e8m0_decode(scales), 32, axis=1)[:, :n]


def attention_forward_mxfp8(q8, q_scale, k8, k_scale, v8, v_scale, causal: bool, scale: float):
    """Attention on microscaled FP8 inputs: the plain forward on the values
    the codes and block scales stand for. Returns (O [B, N, H, d], L [B, H, N])."""
    return attention_forward(dequantize_mx_rows(q8, q_scale), dequantize_mx_rows(k8, k_scale),
                             dequantize_mx_cols(v8, v_scale), causal, scale)

