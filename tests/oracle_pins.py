"""Pins for the fp64 attention oracle.

Each pin checks the oracle against something other than itself: a closed
form, an invariant the mathematics fixes, a brute-force scalar loop, finite
differences, an independent library implementation, or a hand-worked example.
Every pin takes the forward/backward callables as arguments so the same pins
can be run against deliberately broken copies of the oracle (the mutation
tests), each of which must fail at least one pin.

A pin raises AssertionError on failure.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TOL = 1e-11  # fp64 agreement for identities that hold exactly in real arithmetic


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol * scale:.3e}"


# --------------------------------------------------------------------------
# forward pins


def pin_rows_sum_to_one(mod):
    """With V = identity (N = d) the output is the probability matrix itself:
    each row sums to one, entries lie in [0, 1], and causal rows are zero
    past the diagonal."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    N = 8
    q = _rand((1, N, 2, N), 11)
    k = _rand((1, N, 2, N), 12)
    v = np.zeros((1, N, 2, N))
    for h in range(2):
        v[0, :, h, :] = np.eye(N)
    for causal in (False, True):
        o, _ = fwd(q, k, v, causal, 0.7)
        _close(o.sum(axis=3), np.ones((1, N, 2)), what="row sums")
        assert np.all(o >= -TOL) and np.all(o <= 1 + TOL)
        if causal:
            upper = np.triu(np.ones((N, N), dtype=bool), 1)
            for h in range(2):
                assert np.all(np.abs(o[0, :, h, :][upper]) <= TOL), "causal leak"
        else:
            assert np.all(o > 0), "non-causal probabilities must be positive"


def pin_q_zero(mod):
    """Q = 0 makes every score 0: non-causal O_i = mean_j V_j, L_i = ln N;
    causal O_i = mean_{j<=i} V_j, L_i = ln(i+1)."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    B, N, H, d = 2, 13, 3, 5
    k = _rand((B, N, H, d), 21)
    v = _rand((B, N, H, d), 22)
    q = np.zeros((B, N, H, d))
    o, lse = fwd(q, k, v, False, 0.3)
    _close(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), what="Q=0 mean")
    _close(lse, np.full((B, H, N), math.log(N)), what="Q=0 lse")
    o, lse = fwd(q, k, v, True, 0.3)
    prefix = np.cumsum(v, axis=1) / np.arange(1, N + 1)[None, :, None, None]
    _close(o, prefix, what="Q=0 causal prefix mean")
    _close(lse, np.broadcast_to(np.log(np.arange(1, N + 1)), (B, H, N)), what="Q=0 causal lse")


def pin_causal_row0(mod):
    """Causal query 0 sees key 0 only: O_0 = V_0 and L_0 = scale * q_0 . k_0."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    B, N, H, d = 2, 9, 2, 4
    q, k, v = _rand((B, N, H, d), 31), _rand((B, N, H, d), 32), _rand((B, N, H, d), 33)
    scale = 0.45
    o, lse = fwd(q, k, v, True, scale)
    _close(o[:, 0], v[:, 0], what="row 0 output")
    _close(lse[:, :, 0], scale * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]), what="row 0 lse")


def pin_causal_prefix(mod):
    """Causal attention of the first n tokens does not depend on later tokens,
    and the last causal row equals the last non-causal row."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    B, N, H, d = 1, 12, 2, 6
    q, k, v = _rand((B, N, H, d), 41), _rand((B, N, H, d), 42), _rand((B, N, H, d), 43)
    o, lse = fwd(q, k, v, True, 0.5)
    for n in (1, 5, 11):
        o2, lse2 = fwd(q[:, :n], k[:, :n], v[:, :n], True, 0.5)
        _close(o[:, :n], o2, what=f"prefix {n}")
        _close(lse[:, :, :n], lse2, what=f"prefix lse {n}")
    o_nc, lse_nc = fwd(q, k, v, False, 0.5)
    _close(o[:, -1], o_nc[:, -1], what="last row")
    _close(lse[:, :, -1], lse_nc[:, :, -1], what="last row lse")


def pin_permutations(mod):
    """Non-causal: permuting queries permutes outputs; permuting keys and values
    together changes nothing; swapping heads or batches permutes outputs."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    B, N, H, d = 2, 10, 3, 4
    q, k, v = _rand((B, N, H, d), 51), _rand((B, N, H, d), 52), _rand((B, N, H, d), 53)
    o, lse = fwd(q, k, v, False, 0.6)
    perm = np.random.Generator(np.random.PCG64(5)).permutation(N)
    o2, lse2 = fwd(q[:, perm], k, v, False, 0.6)
    _close(o2, o[:, perm], what="query permutation")
    _close(lse2, lse[:, :, perm], what="query permutation lse")
    o3, lse3 = fwd(q, k[:, perm], v[:, perm], False, 0.6)
    _close(o3, o, what="key/value permutation")
    _close(lse3, lse, what="key/value permutation lse")
    hp = [2, 0, 1]
    o4, lse4 = fwd(q[:, :, hp], k[:, :, hp], v[:, :, hp], True, 0.6)
    o4c, lse4c = fwd(q, k, v, True, 0.6)
    _close(o4, o4c[:, :, hp], what="head permutation")
    _close(lse4, lse4c[:, hp], what="head permutation lse")
    o5, _ = fwd(q[::-1], k[::-1], v[::-1], False, 0.6)
    _close(o5, o[::-1], what="batch permutation")


def pin_constant_v(mod):
    """V_j = c for all j gives O_i = c; then dS = 0, so dQ = dK = 0."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    B, N, H, d = 1, 7, 2, 3
    q, k = _rand((B, N, H, d), 61), _rand((B, N, H, d), 62)
    c = np.array([0.5, -1.25, 2.0])
    v = np.broadcast_to(c, (B, N, H, d)).copy()
    for causal in (False, True):
        o, _ = fwd(q, k, v, causal, 0.8)
        _close(o, v, what="constant V output")
        if bwd is not None:
            do = _rand((B, N, H, d), 63)
            dq, dk, dv = bwd(q, k, v, do, causal, 0.8)[:3]
            _close(dq, np.zeros_like(dq), what="constant V dQ")
            _close(dk, np.zeros_like(dk), what="constant V dK")


def pin_linear_in_v(mod):
    """O is linear in V for fixed Q, K."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    B, N, H, d = 1, 9, 2, 4
    q, k = _rand((B, N, H, d), 71), _rand((B, N, H, d), 72)
    v1, v2 = _rand((B, N, H, d), 73), _rand((B, N, H, d), 74)
    for causal in (False, True):
        o1, _ = fwd(q, k, v1, causal, 0.4)
        o2, _ = fwd(q, k, v2, causal, 0.4)
        o12, _ = fwd(q, k, 2.0 * v1 - 3.0 * v2, causal, 0.4)
        _close(o12, 2.0 * o1 - 3.0 * o2, what="linearity")


def pin_key_shift(mod):
    """K_j -> K_j + c adds scale * q_i . c to every score of row i: the
    softmax (hence O) is unchanged and L_i shifts by exactly that amount."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    B, N, H, d = 1, 8, 2, 5
    q, k, v = _rand((B, N, H, d), 81), _rand((B, N, H, d), 82), _rand((B, N, H, d), 83)
    c = _rand((d,), 84)
    scale = 0.35
    for causal in (False, True):
        o, lse = fwd(q, k, v, causal, scale)
        o2, lse2 = fwd(q, k + c, v, causal, scale)
        _close(o2, o, what="key shift output")
        shift = scale * np.einsum("bnhd,d->bhn", q, c)
        _close(lse2, lse + shift, what="key shift lse")


def pin_single_token(mod):
    """N = 1: O = V and L = scale * q . k, causal or not."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    q, k, v = _rand((3, 1, 2, 6), 91), _rand((3, 1, 2, 6), 92), _rand((3, 1, 2, 6), 93)
    for causal in (False, True):
        o, lse = fwd(q, k, v, causal, 0.9)
        _close(o, v, what="N=1 output")
        _close(lse, 0.9 * np.einsum("bnhd,bnhd->bhn", q, k), what="N=1 lse")


def _brute_forward(q, k, v, causal, scale):
    """Scalar loops with math.exp / math.fsum, no matrix products."""
    B, N, H, d = q.shape
    o = np.zeros((B, N, H, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                s = [scale * math.fsum(q[b, i, h, t] * k[b, j, h, t] for t in range(d)) for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = math.fsum(w)
                for t in range(d):
                    o[b, i, h, t] = math.fsum(w[n] * v[b, j, h, t] for n, j in enumerate(keys)) / tot
                lse[b, h, i] = m + math.log(tot)
    return o, lse


def pin_brute_force(mod):
    """Agreement with an independent scalar-loop implementation on tiny inputs."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    for (B, N, H, d), seed in (((1, 5, 2, 3), 101), ((2, 16, 1, 4), 102)):
        q = _rand((B, N, H, d), seed)
        k = _rand((B, N, H, d), seed + 1000)
        v = _rand((B, N, H, d), seed + 2000)
        for causal in (False, True):
            o, lse = fwd(q, k, v, causal, 0.55)
            ob, lseb = _brute_forward(q, k, v, causal, 0.55)
            _close(o, ob, 1e-13, what="brute output")
            _close(lse, lseb, 1e-13, what="brute lse")


def pin_torch_sdpa(mod):
    """Agreement with torch's CPU fp64 scaled_dot_product_attention (math path)
    and its autograd gradients."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    import torch

    for (B, N, H, d), seed in (((2, 11, 3, 8), 111), ((1, 32, 2, 16), 112)):
        q = _rand((B, N, H, d), seed)
        k = _rand((B, N, H, d), seed + 1)
        v = _rand((B, N, H, d), seed + 2)
        do = _rand((B, N, H, d), seed + 3)
        for causal in (False, True):
            tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3).copy(), requires_grad=True) for x in (q, k, v))
            with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
                to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.3)
            to.backward(torch.tensor(do.transpose(0, 2, 1, 3).copy()))
            o, _ = fwd(q, k, v, causal, 0.3)
            _close(o, to.detach().numpy().transpose(0, 2, 1, 3), 1e-12, what="sdpa output")
            if bwd is not None:
                dq, dk, dv = bwd(q, k, v, do, causal, 0.3)[:3]
                for name, mine, ref in (("dq", dq, tq.grad), ("dk", dk, tk.grad), ("dv", dv, tv.grad)):
                    _close(mine, ref.numpy().transpose(0, 2, 1, 3), 1e-12, what=f"sdpa {name}")


# --------------------------------------------------------------------------
# backward pins


def pin_backward_invariants(mod):
    """Rows of dS sum to zero, so sum_j dK_j = 0 per (b, h); rows of P sum to
    one, so sum_j dV_j = sum_i dO_i; causal dQ_0 = 0 because dS_00 = 0."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    B, N, H, d = 2, 9, 2, 5
    q, k, v, do = (_rand((B, N, H, d), s) for s in (121, 122, 123, 124))
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, causal, 0.7)[:3]
        _close(dk.sum(axis=1), np.zeros((B, H, d)), what="sum dK")
        _close(dv.sum(axis=1), do.sum(axis=1), what="sum dV")
        if causal:
            _close(dq[:, 0], np.zeros((B, H, d)), what="causal dQ_0")


def pin_finite_differences(mod):
    """Central differences of f = sum(dO * O) match the analytic gradients."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    h = 1e-6
    for (B, N, H, d), causal, seed in (
        ((1, 1, 2, 4), False, 131),
        ((1, 3, 2, 1), True, 132),
        ((1, 3, 2, 4), False, 133),
        ((1, 8, 2, 4), True, 134),
        ((1, 8, 2, 1), False, 135),
    ):
        q, k, v, do = (_rand((B, N, H, d), seed + 10 * t) for t in range(4))
        scale = 0.6
        grads = bwd(q, k, v, do, causal, scale)[:3]

        def f(qq, kk, vv):
            return float(np.sum(do * fwd(qq, kk, vv, causal, scale)[0]))

        for which, g in zip(range(3), grads):
            num = np.zeros_like(g)
            for idx in np.ndindex(*g.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                fp = f(*args)
                args[which][idx] -= 2 * h
                fm = f(*args)
                num[idx] = (fp - fm) / (2 * h)
            _close(g, num, 1e-6, what=f"finite differences grad {which}")


# --------------------------------------------------------------------------
# hand-worked examples


def pin_worked_examples(mod):
    """Small cases worked out by hand from the definition (tests/golden)."""
    fwd, bwd = mod.attention_forward, mod.attention_backward
    with open(os.path.join(GOLDEN, "worked_examples.json")) as fh:
        cases = json.load(fh)["cases"]
    def value(x):
        return math.log(x["ln"]) if isinstance(x, dict) else float(x)

    def vec(xs):
        return np.array([value(x) for x in xs], dtype=np.float64)

    for case in cases:
        for key in ("o", "lse", "dq", "dk", "dv"):
            if key in case:
                case[key] = vec(case[key])

        def arr(name):
            return vec(case[name]).reshape(1, -1, 1, 1)

        q, k, v = arr("q"), arr("k"), arr("v")
        o, lse = fwd(q, k, v, case["causal"], case["scale"])
        _close(o.reshape(-1), case["o"], 1e-14, what=case["name"] + " O")
        _close(lse.reshape(-1), case["lse"], 1e-14, what=case["name"] + " L")
        if "do" in case and bwd is not None:
            dq, dk, dv = bwd(q, k, v, arr("do"), case["causal"], case["scale"])[:3]
            _close(dq.reshape(-1), case["dq"], 1e-14, what=case["name"] + " dQ")
            _close(dk.reshape(-1), case["dk"], 1e-14, what=case["name"] + " dK")
            _close(dv.reshape(-1), case["dv"], 1e-14, what=case["name"] + " dV")


def pin_sampled_rows(mod):
    """The sampled-row forward agrees with the scalar-loop implementation on
    the rows it is asked for (including a non-contiguous, unsorted sample)."""
    B, N, H, d = 2, 14, 3, 4
    q, k, v = _rand((B, N, H, d), 141), _rand((B, N, H, d), 142), _rand((B, N, H, d), 143)
    rows = [13, 0, 7, 6, 12]
    for causal in (False, True):
        ob, lseb = _brute_forward(q, k, v, causal, 0.65)
        for b, h in ((0, 2), (1, 0)):
            o, lse = mod.attention_forward_rows(q, k, v, causal, 0.65, b, h, rows)
            _close(o, ob[b, rows, h, :], 1e-13, what="sampled rows output")
            _close(lse, lseb[b, h, rows], 1e-13, what="sampled rows lse")


def pin_backward_head(mod):
    """The single-(batch, head) backward agrees with torch autograd on that
    head of a problem with B != H."""
    import torch

    B, N, H, d = 2, 9, 3, 4
    q, k, v, do = (_rand((B, N, H, d), s) for s in (151, 152, 153, 154))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3).copy(), requires_grad=True) for x in (q, k, v))
        with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
            to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.5)
        to.backward(torch.tensor(do.transpose(0, 2, 1, 3).copy()))
        for b, h in ((1, 2), (0, 1)):
            dq, dk, dv = mod.attention_backward_head(q, k, v, do, causal, 0.5, b, h)
            _close(dq, tq.grad[b, h].numpy(), 1e-12, what="head dQ")
            _close(dk, tk.grad[b, h].numpy(), 1e-12, what="head dK")
            _close(dv, tv.grad[b, h].numpy(), 1e-12, what="head dV")


# --------------------------------------------------------------------------
# key-range chunk and merge pins


def _brute_chunk(q, k, v, causal, scale, q_start, k_start):
    """Scalar loops over global positions, no matrix products; a row that
    sees no key of the chunk gives O = 0 and L = -inf."""
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    o = np.zeros((B, Nq, H, d))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                keys = [j for j in range(Nk) if not causal or k_start + j <= q_start + i]
                if not keys:
                    continue
                s = [scale * math.fsum(q[b, i, h, t] * k[b, j, h, t] for t in range(d)) for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = math.fsum(w)
                for t in range(d):
                    o[b, i, h, t] = math.fsum(w[n] * v[b, j, h, t] for n, j in enumerate(keys)) / tot
                lse[b, h, i] = m + math.log(tot)
    return o, lse


def _close_inf(a, b, tol=TOL, what=""):
    """_close that also accepts matching -inf entries."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    ninf = np.isneginf(b)
    assert np.array_equal(np.isneginf(a), ninf), f"{what}: -inf pattern differs"
    _close(np.where(ninf, 0.0, a), np.where(ninf, 0.0, b), tol, what)


def pin_chunk_brute_force(mod):
    """A query chunk against a key chunk at global offsets agrees with scalar
    loops, including rows that see part of the chunk or none of it."""
    cases = [((1, 6, 7, 2, 3), (0, 0), 301), ((1, 5, 9, 1, 4), (4, 2), 302),
             ((2, 7, 4, 1, 2), (3, 6), 303), ((1, 5, 8, 2, 3), (10, 0), 304)]
    for (B, Nq, Nk, H, d), (qs, ks), seed in cases:
        q = _rand((B, Nq, H, d), seed)
        k = _rand((B, Nk, H, d), seed + 1000)
        v = _rand((B, Nk, H, d), seed + 2000)
        for causal in (False, True):
            o, lse = mod.attention_forward_chunk(q, k, v, causal, 0.6, qs, ks)
            ob, lseb = _brute_chunk(q, k, v, causal, 0.6, qs, ks)
            _close(o, ob, 1e-13, what="chunk brute output")
            _close_inf(lse, lseb, 1e-13, what="chunk brute lse")


def pin_chunk_merge_is_full_attention(mod):
    """Splitting the keys into consecutive chunks (one of them empty) and
    merging the chunk results gives full attention; so does taking a query
    block at its global position."""
    B, N, H, d = 2, 37, 2, 5
    q, k, v = (_rand((B, N, H, d), 310 + t) for t in range(3))
    bounds = [0, 1, 9, 9, 20, 31, 37]
    for causal in (False, True):
        o_full, l_full = mod.attention_forward(q, k, v, causal, 0.45)
        for r0, r1 in ((0, N), (13, 29)):
            parts = [mod.attention_forward_chunk(q[:, r0:r1], k[:, a:b], v[:, a:b], causal, 0.45, r0, a)
                     for a, b in zip(bounds[:-1], bounds[1:])]
            o, lse = mod.merge_chunks(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
            _close(o, o_full[:, r0:r1], 1e-12, what="merged output")
            _close(lse, l_full[:, :, r0:r1], 1e-12, what="merged lse")


def pin_chunk_global_offsets(mod):
    """Causal chunks at global positions: keys wholly before the queries are
    all visible (the non-causal result), keys wholly after are invisible
    (O = 0, L = -inf), and moving both chunks by the same amount changes
    nothing."""
    q = _rand((1, 6, 2, 4), 320)
    k = _rand((1, 9, 2, 4), 321)
    v = _rand((1, 9, 2, 4), 322)
    o_nc, l_nc = mod.attention_forward_chunk(q, k, v, False, 0.8, 0, 0)
    o_past, l_past = mod.attention_forward_chunk(q, k, v, True, 0.8, 100, 91)
    _close(o_past, o_nc, what="past chunk output")
    _close(l_past, l_nc, what="past chunk lse")
    o_fut, l_fut = mod.attention_forward_chunk(q, k, v, True, 0.8, 0, 6)
    assert np.all(o_fut == 0.0) and np.all(np.isneginf(l_fut)), "future chunk must be empty"
    o_a, l_a = mod.attention_forward_chunk(q, k, v, True, 0.8, 4, 2)
    o_b, l_b = mod.attention_forward_chunk(q, k, v, True, 0.8, 1004, 1002)
    _close(o_a, o_b, what="shifted output")
    _close(l_a, l_b, what="shifted lse")
    # Query row i sees keys 0 .. i + 2 here: row 0 equals the first three keys alone.
    o_3, l_3 = mod.attention_forward_chunk(q[:, :1], k[:, :3], v[:, :3], False, 0.8, 0, 0)
    _close(o_a[:, :1], o_3, what="partial row output")
    _close(l_a[:, :, :1], l_3, what="partial row lse")


def pin_merge_closed_forms(mod):
    """Merge identities: one chunk passes through; two chunks with equal L
    average their outputs and add ln 2; a chunk with L = -inf carries no
    weight; chunk order does not matter; rows empty in every chunk give
    O = 0 and L = -inf."""
    C, B, Nq, H, d = 3, 2, 4, 2, 3
    o = _rand((C, B, Nq, H, d), 330)
    lse = _rand((C, B, H, Nq), 331) * 3.0
    m1, l1 = mod.merge_chunks(o[:1], lse[:1])
    _close(m1, o[0], what="single chunk output")
    _close(l1, lse[0], what="single chunk lse")
    eq = np.stack([lse[0], lse[0]])
    m2, l2 = mod.merge_chunks(o[:2], eq)
    _close(m2, 0.5 * (o[0] + o[1]), what="equal-weight output")
    _close(l2, lse[0] + math.log(2.0), what="equal-weight lse")
    dead = lse.copy()
    dead[1] = -np.inf
    m3, l3 = mod.merge_chunks(o, dead)
    m3b, l3b = mod.merge_chunks(o[[0, 2]], dead[[0, 2]])
    _close(m3, m3b, what="empty chunk ignored (output)")
    _close(l3, l3b, what="empty chunk ignored (lse)")
    perm = [2, 0, 1]
    m4, l4 = mod.merge_chunks(o[perm], lse[perm])
    m5, l5 = mod.merge_chunks(o, lse)
    _close(m4, m5, what="chunk order (output)")
    _close(l4, l5, what="chunk order (lse)")
    # Closed form for two chunks: weights are logistic in the lse difference.
    w0 = 1.0 / (1.0 + np.exp(lse[1] - lse[0]))                     # [B, H, Nq]
    want = w0.transpose(0, 2, 1)[..., None] * o[0] + (1 - w0).transpose(0, 2, 1)[..., None] * o[1]
    m6, l6 = mod.merge_chunks(o[:2], lse[:2])
    _close(m6, want, what="two-chunk weights")
    _close(l6, np.logaddexp(lse[0], lse[1]), what="two-chunk lse")
    allneg = np.full((C, B, H, Nq), -np.inf)
    m7, l7 = mod.merge_chunks(o, allneg)
    assert np.all(m7 == 0.0) and np.all(np.isneginf(l7)), "all-empty rows"


def pin_decode_alignment(mod):
    """Decode-shaped attention (queries are the last Nq positions): with
    Nq = Nk it is ordinary causal attention; a single causal query sees every
    key (the non-causal result); each decode row equals the matching row of
    causal attention over the whole sequence; and extra leading rows beyond
    Nk see nothing."""
    B, N, H, d = 1, 19, 2, 4
    q, k, v = (_rand((B, N, H, d), 340 + t) for t in range(3))
    o_full, l_full = mod.attention_forward(q, k, v, True, 0.7)
    o_sq, l_sq = mod.attention_decode(q, k, v, True, 0.7)
    _close(o_sq, o_full, what="square decode output")
    _close(l_sq, l_full, what="square decode lse")
    for nq in (1, 5):
        o_dec, l_dec = mod.attention_decode(q[:, N - nq:], k, v, True, 0.7)
        _close(o_dec, o_full[:, N - nq:], what="decode rows output")
        _close(l_dec, l_full[:, :, N - nq:], what="decode rows lse")
    o1, l1 = mod.attention_decode(q[:, :1], k, v, True, 0.7)
    o1n, l1n = mod.attention_decode(q[:, :1], k, v, False, 0.7)
    _close(o1, o1n, what="single query output")
    _close(l1, l1n, what="single query lse")
    o_long, l_long = mod.attention_decode(q[:, :7], k[:, :4], v[:, :4], True, 0.7)
    assert np.all(o_long[:, :3] == 0.0) and np.all(np.isneginf(l_long[:, :, :3])), "rows before the first key"
    o_tail, l_tail = mod.attention_forward_chunk(q[:, 3:7], k[:, :4], v[:, :4], True, 0.7, 0, 0)
    _close(o_long[:, 3:], o_tail, what="rows from the first key on")
    _close(l_long[:, :, 3:], l_tail, what="rows from the first key on (lse)")


# --------------------------------------------------------------------------
# additive-bias pins


def _brute_bias_forward(q, k, v, bias, causal, scale):
    """Scalar loops with math.exp / math.fsum for the biased forward."""
    B, N, H, d = q.shape
    o = np.zeros((B, N, H, d))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = [j for j in (range(i + 1) if causal else range(N)) if bias[b, h, i, j] != -np.inf]
                if not keys:
                    continue
                s = [scale * math.fsum(q[b, i, h, t] * k[b, j, h, t] for t in range(d)) + bias[b, h, i, j]
                     for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = math.fsum(w)
                for t in range(d):
                    o[b, i, h, t] = math.fsum(w[n] * v[b, j, h, t] for n, j in enumerate(keys)) / tot
                lse[b, h, i] = m + math.log(tot)
    return o, lse


def pin_bias_brute_force(mod):
    """Biased forward against scalar loops, with some -inf bias entries
    (including a row that loses every key)."""
    for (B, N, H, d), seed in (((1, 6, 2, 3), 401), ((2, 9, 1, 4), 402)):
        q, k, v = (_rand((B, N, H, d), seed + 1000 * t) for t in range(3))
        bias = _rand((B, H, N, N), seed + 3000) * 2.0
        bias[0, 0, 1, :3] = -np.inf
        bias[0, 0, 2, :] = -np.inf
        for causal in (False, True):
            o, lse = mod.attention_forward_bias(q, k, v, bias, causal, 0.6)
            ob, lseb = _brute_bias_forward(q, k, v, bias, causal, 0.6)
            _close(o, ob, 1e-13, what="bias brute output")
            _close_inf(lse, lseb, 1e-13, what="bias brute lse")


def pin_bias_special_cases(mod):
    """Bias = 0 is plain attention (and dBias = dS has zero row sums); a -inf
    strictly-upper-triangular bias is the causal mask; a bias constant along
    each row leaves O unchanged and shifts L by that constant."""
    B, N, H, d = 2, 11, 2, 4
    q, k, v, do = (_rand((B, N, H, d), 410 + t) for t in range(4))
    zero = np.zeros((B, H, N, N))
    for causal in (False, True):
        o0, l0 = mod.attention_forward(q, k, v, causal, 0.5)
        o, l = mod.attention_forward_bias(q, k, v, zero, causal, 0.5)
        _close(o, o0, what="zero bias output")
        _close(l, l0, what="zero bias lse")
        g0 = mod.attention_backward(q, k, v, do, causal, 0.5)
        g = mod.attention_backward_bias(q, k, v, zero, do, causal, 0.5)
        for a, b_, name in zip(g[:3], g0[:3], ("dQ", "dK", "dV")):
            _close(a, b_, what=f"zero bias {name}")
        _close(g[3].sum(axis=3), np.zeros((B, H, N)), what="dBias row sums")
    tri = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, 0.0)
    mask = np.broadcast_to(tri, (B, H, N, N)).copy()
    oc, lc = mod.attention_forward(q, k, v, True, 0.5)
    om, lm = mod.attention_forward_bias(q, k, v, mask, False, 0.5)
    _close(om, oc, what="-inf triangle output")
    _close(lm, lc, what="-inf triangle lse")
    gc = mod.attention_backward(q, k, v, do, True, 0.5)
    gm = mod.attention_backward_bias(q, k, v, mask, do, False, 0.5)
    for a, b_, name in zip(gm[:3], gc[:3], ("dQ", "dK", "dV")):
        _close(a, b_, what=f"-inf triangle {name}")
    assert np.all(gm[3][..., np.triu_indices(N, 1)[0], np.triu_indices(N, 1)[1]] == 0.0), "masked dBias"
    row = _rand((B, H, N, 1), 420) * 3.0
    ob, lb = mod.attention_forward_bias(q, k, v, np.broadcast_to(row, (B, H, N, N)).copy(), False, 0.5)
    o0, l0 = mod.attention_forward(q, k, v, False, 0.5)
    _close(ob, o0, what="row-constant bias output")
    _close(lb, l0 + row[..., 0], what="row-constant bias lse")


def pin_bias_torch_sdpa(mod):
    """Forward and all four gradients against torch's fp64 CPU
    scaled_dot_product_attention with an additive float mask (autograd)."""
    import torch

    B, N, H, d = 2, 13, 3, 5
    q, k, v, do = (_rand((B, N, H, d), 430 + t) for t in range(4))
    bias = _rand((B, H, N, N), 434)
    t = [torch.tensor(x.transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    tb = torch.tensor(bias, dtype=torch.float64, requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(t[0], t[1], t[2], attn_mask=tb, scale=0.45)
    out.backward(torch.tensor(do.transpose(0, 2, 1, 3), dtype=torch.float64))
    dq, dk, dv, db, o, _, _ = mod.attention_backward_bias(q, k, v, bias, do, False, 0.45)
    _close(o, out.detach().numpy().transpose(0, 2, 1, 3), 1e-12, what="sdpa bias output")
    for got, ref, name in ((dq, t[0], "dQ"), (dk, t[1], "dK"), (dv, t[2], "dV")):
        _close(got, ref.grad.numpy().transpose(0, 2, 1, 3), 1e-12, what=f"sdpa bias {name}")
    _close(db, tb.grad.numpy(), 1e-12, what="sdpa dBias")


def pin_bias_finite_differences(mod):
    """dBias (and dQ) against central differences of sum(dO * O)."""
    B, N, H, d = 1, 4, 1, 3
    q, k, v, do = (_rand((B, N, H, d), 440 + t) for t in range(4))
    bias = _rand((B, H, N, N), 444)
    for causal in (False, True):
        dq, _, _, db, _, _, _ = mod.attention_backward_bias(q, k, v, bias, do, causal, 0.8)
        f = lambda bb, qq: float(np.sum(do * mod.attention_forward_bias(qq, k, v, bb, causal, 0.8)[0]))
        h = 1e-6
        for (i, j) in ((0, 0), (2, 1), (3, 3), (1, 3)):
            bp, bm = bias.copy(), bias.copy()
            bp[0, 0, i, j] += h
            bm[0, 0, i, j] -= h
            num = (f(bp, q) - f(bm, q)) / (2 * h)
            assert abs(num - db[0, 0, i, j]) <= 1e-7 * max(1.0, abs(num)), f"dBias[{i},{j}] {num} vs {db[0, 0, i, j]}"
        for (i, t) in ((1, 0), (3, 2)):
            qp, qm = q.copy(), q.copy()
            qp[0, i, 0, t] += h
            qm[0, i, 0, t] -= h
            num = (f(bias, qp) - f(bias, qm)) / (2 * h)
            assert abs(num - dq[0, i, 0, t]) <= 1e-7 * max(1.0, abs(num)), f"dQ[{i},{t}]"


# --------------------------------------------------------------------------
# FP8 (e4m3) input pins


def pin_e4m3_decode(mod):
    """The e4m3 decode against values fixed by the format (1.0, 448, the
    smallest subnormal and normal, signs, NaN codes) and, for all 256 codes,
    against torch's independent float8_e4m3fn implementation."""
    import torch

    dec = mod.e4m3_decode(np.arange(256))
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
             0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x80: -0.0}
    for code, val in fixed.items():
        assert dec[code] == val, f"code {code:#x}: {dec[code]} != {val}"
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(dec)
    assert np.all(both_nan | (ref == dec)), "decode differs from torch float8_e4m3fn"
    # monotone over the positive finite codes
    pos = dec[:0x7F]
    assert np.all(np.diff(pos) > 0)


def pin_fp8_forward(mod):
    """FP8 attention is the forward on the dequantized values: checked
    against scalar loops on the decoded inputs, and the descale of V scales
    the output while the descales of Q and K act only through their product."""
    B, N, H, d = 1, 7, 2, 4
    rng = np.random.Generator(np.random.PCG64(350))
    codes = [rng.integers(0, 0x7F, (B, N, H, d)).astype(np.uint8) | (rng.integers(0, 2, (B, N, H, d)) * 0x80).astype(np.uint8)
             for _ in range(3)]
    desc = [np.abs(rng.standard_normal((B, H))) * 0.01 + 0.002 for _ in range(3)]
    for causal in (False, True):
        o, lse = mod.attention_forward_fp8(*codes, *desc, causal, 0.5)
        vals = [mod.e4m3_decode(c) * dd[:, None, :, None] for c, dd in zip(codes, desc)]
        ob, lseb = _brute_forward(*vals, causal, 0.5)
        _close(o, ob, 1e-13, what="fp8 brute output")
        _close(lse, lseb, 1e-13, what="fp8 brute lse")
        o2, l2 = mod.attention_forward_fp8(codes[0], codes[1], codes[2], desc[0] * 2.0, desc[1] / 2.0,
                                           desc[2] * 3.0, causal, 0.5)
        _close(o2, 3.0 * o, what="descale V scales O")
        _close(l2, lse, what="only the product of the Q and K descales matters")


def pin_e8m0_decode(mod):
    """The E8M0 scale decode against values fixed by the format (2^-127 at
    code 0, 1 at 127, 2^127 at 254, NaN at 255) and, for all 256 codes,
    against torch's independent float8_e8m0fnu implementation."""
    import torch

    dec = mod.e8m0_decode(np.arange(256))
    fixed = {0: 2.0 ** -127, 1: 2.0 ** -126, 126: 0.5, 127: 1.0, 128: 2.0, 130: 8.0, 254: 2.0 ** 127}
    for code, val in fixed.items():
        assert dec[code] == val, f"code {code}: {dec[code]} != {val}"
    assert np.isnan(dec[255])
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(dec)
    assert np.all(both_nan | (ref == dec)), "decode differs from torch float8_e8m0fnu"


def _mx_values_by_loops(mod, codes, scales, along_tokens):
    """Values of microscaled codes element by element (the block of element
    (b, n, h, i) is i // 32 of its token, or n // 32 of its column)."""
    B, N, H, d = codes.shape
    out = np.empty((B, N, H, d))
    for b in range(B):
        for n in range(N):
            for h in range(H):
                for i in range(d):
                    sc = scales[b, n // 32, h, i] if along_tokens else scales[b, n, h, i // 32]
                    out[b, n, h, i] = float(mod.e4m3_decode(codes[b, n, h, i])) * 2.0 ** (int(sc) - 127)
    return out


def pin_mxfp8_forward(mod):
    """Microscaled FP8 attention is the forward on the values the codes and
    block scales stand for: checked against scalar loops (37 tokens: a short
    last block of V; d = 64: two blocks per Q and K token). All scales at
    2^0 reduce it to the per-head FP8 form with unit descales; one V block
    scaled up by 2 adds exactly that block's share of P V once more; Q
    scales raised by one double the scores; Q and K blocks shifted in
    opposite directions leave the result unchanged."""
    B, N, H, d = 1, 37, 2, 64
    rng = np.random.Generator(np.random.PCG64(351))
    codes = [rng.integers(0, 0x7F, (B, N, H, d)).astype(np.uint8) | (rng.integers(0, 2, (B, N, H, d)) * 0x80).astype(np.uint8)
             for _ in range(3)]
    qs = rng.integers(118, 124, (B, N, H, d // 32)).astype(np.uint8)
    ks = rng.integers(118, 124, (B, N, H, d // 32)).astype(np.uint8)
    vs = rng.integers(110, 140, (B, (N + 31) // 32, H, d)).astype(np.uint8)
    for causal in (False, True):
        o, lse = mod.attention_forward_mxfp8(codes[0], qs, codes[1], ks, codes[2], vs, causal, 0.5)
        vals = [_mx_values_by_loops(mod, codes[0], qs, False), _mx_values_by_loops(mod, codes[1], ks, False),
                _mx_values_by_loops(mod, codes[2], vs, True)]
        ob, lseb = _brute_forward(*vals, causal, 0.5)
        _close(o, ob, 1e-13, what="mxfp8 brute output")
        _close(lse, lseb, 1e-13, what="mxfp8 brute lse")
        one = lambda a: np.full(a.shape, 127, np.uint8)
        o1, l1 = mod.attention_forward_mxfp8(codes[0], one(qs), codes[1], one(ks), codes[2], one(vs), causal, 0.5)
        unit = np.ones((B, H))
        of, lf = mod.attention_forward_fp8(*codes, unit, unit, unit, causal, 0.5)
        _close(o1, of, 1e-13, what="unit block scales = per-head form")
        _close(l1, lf, 1e-13, what="unit block scales = per-head form (lse)")
        vs2 = vs.copy()
        vs2[0, 1, :, 5] += 1
        o2, l2 = mod.attention_forward_mxfp8(codes[0], qs, codes[1], ks, codes[2], vs2, causal, 0.5)
        vblk = np.zeros_like(vals[2])
        vblk[0, 32:, :, 5] = vals[2][0, 32:, :, 5]
        extra, _ = mod.attention_forward(vals[0], vals[1], vblk, causal, 0.5)
        _close(o2, o + extra, what="V block scale doubles that block's share")
        _close(l2, lse, what="V scales leave the logsumexp")
        o3, l3 = mod.attention_forward_mxfp8(codes[0], qs + 1, codes[1], ks, codes[2], vs, causal, 0.5)
        o4, l4 = mod.attention_forward_mxfp8(codes[0], qs, codes[1], ks, codes[2], vs, causal, 1.0)
        _close(o3, o4, what="Q scales + 1 = doubled softmax scale")
        _close(l3, l4, what="Q scales + 1 = doubled softmax scale (lse)")
        qs5, ks5 = qs.copy(), ks.copy()
        qs5[..., 1] += 2
        ks5[..., 1] -= 2
        o5, l5 = mod.attention_forward_mxfp8(codes[0], qs5, codes[1], ks5, codes[2], vs, causal, 0.5)
        _close(o5, o, 1e-13, what="opposite Q and K block shifts cancel")
        _close(l5, lse, 1e-13, what="opposite Q and K block shifts cancel (lse)")


FORWARD_PINS = [
    pin_rows_sum_to_one,
    pin_q_zero,
    pin_causal_row0,
    pin_causal_prefix,
    pin_permutations,
    pin_linear_in_v,
    pin_key_shift,
    pin_single_token,
    pin_brute_force,
    pin_sampled_rows,
]
CHUNK_PINS = [
    pin_chunk_brute_force,
    pin_chunk_merge_is_full_attention,
    pin_chunk_global_offsets,
    pin_merge_closed_forms,
    pin_decode_alignment,
]
BIAS_PINS = [
    pin_bias_brute_force,
    pin_bias_special_cases,
    pin_bias_torch_sdpa,
    pin_bias_finite_differences,
]
FP8_PINS = [
    pin_e4m3_decode,
    pin_fp8_forward,
    pin_e8m0_decode,
    pin_mxfp8_forward,
]
BACKWARD_PINS = [
    pin_constant_v,
    pin_backward_invariants,
    pin_finite_differences,
    pin_torch_sdpa,
    pin_worked_examples,
    pin_backward_head,
]
ALL_PINS = FORWARD_PINS + CHUNK_PINS + BIAS_PINS + FP8_PINS + BACKWARD_PINS
