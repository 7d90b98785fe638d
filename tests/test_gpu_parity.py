"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every test feeds the same seeded bf16 bits to both sides and compares element
by element. Tolerances: O, dQ, dK, dV max-abs <= 2e-2 and mean-abs <= 2e-3;
the fp32 logsumexp max-abs <= 1e-3. Small shapes (several tiles plus a ragged
tail) are compared whole; the five benchmark workloads run at full size in the
same launch configuration the benchmark times, and are compared with the
oracle on every element (the oracle runs head by head in a thread pool).
"""

import math
import sys

import numpy as np
import pytest

import exact_tiled_attention_37_amd as fa
import oracle
import seeded_inputs as si
from tests import parity_log
from tests import kernel_rounding as kr
from tests import oracle_heads as oh

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL, LSE_TOL = 2e-2, 2e-3, 1e-3


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
    return torch.device("cuda:0")


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


def gpu_fwd(bits, causal, scale):
    import torch

    q, k, v = dev(bits["q"]), dev(bits["k"]), dev(bits["v"])
    o, lse = fa.fa_fwd(q, k, v, causal, scale)
    torch.cuda.synchronize()
    return q, k, v, o, lse


def gpu_bwd(q, k, v, o, lse, do_bits, causal, scale, workspace=None):
    import torch

    do = dev(do_bits)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, do, causal, scale, workspace=workspace)
    torch.cuda.synchronize()
    return dq, dk, dv


# ---------------------------------------------------------------------------
# small shapes: whole-tensor comparison, forward and backward

SMALL = [
    (1, 1, 1, 64), (1, 3, 2, 64), (2, 17, 3, 128), (1, 64, 2, 64), (1, 127, 2, 128),
    (2, 129, 1, 64), (1, 200, 2, 128), (1, 333, 3, 64), (1, 1000, 1, 128), (1, 256, 2, 128),
]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dN%dH%dd%d" % s)
def test_small_fwd_bwd(shape, causal):
    B, N, H, d = shape
    seed = 1000 + N * 7 + d + int(causal)
    scale = 1.0 / math.sqrt(d)
    announce(f"small fwd+bwd shape={shape} causal={causal} seed={seed}")
    bits = si.draw(B, N, H, d, seed, backward=True)
    q64, k64, v64, do64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v", "do"))
    rq, rk, rv, ro, rl, _ = oracle.attention_backward(q64, k64, v64, do64, causal, scale)
    q, k, v, o, lse = gpu_fwd(bits, causal, scale)
    check("O", f64(o), ro)
    check("LSE", f64(lse), rl, LSE_TOL, LSE_TOL)
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, bits["do"], causal, scale)
    check("dQ", f64(dq), rq)
    check("dK", f64(dk), rk)
    check("dV", f64(dv), rv)


def check_rel(name, got, ref):
    """Tolerance for scales other than 1/sqrt(d): the fixed absolute bounds
    assume O(1) outputs, but bf16 rounding of P, dS and of the outputs gives
    errors proportional to the output's magnitude M = max|ref|, which grows
    with |scale|. The bound keeps the absolute tolerance up to M = 2 and
    scales it with M beyond (2e-2 * M / 2 is about 2.5 bf16 ulps of M)."""
    m = max(1.0, float(np.max(np.abs(ref))) / 2.0)
    check(name, got, ref, MAX_TOL * m, MEAN_TOL * m)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.9, 2.5], ids=lambda s: f"scale{s}")
@pytest.mark.parametrize("d", [64, 128])
def test_other_scales(scale, d):
    B, N, H = 1, 150, 2
    for causal in (False, True):
        announce(f"scale={scale} d={d} causal={causal}")
        bits = si.draw(B, N, H, d, 77 + d, backward=True)
        q64, k64, v64, do64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v", "do"))
        rq, rk, rv, ro, rl, _ = oracle.attention_backward(q64, k64, v64, do64, causal, scale)
        q, k, v, o, lse = gpu_fwd(bits, causal, scale)
        check("O", f64(o), ro)
        check("LSE", f64(lse), rl, LSE_TOL, LSE_TOL)
        dq, dk, dv = gpu_bwd(q, k, v, o, lse, bits["do"], causal, scale)
        check_rel("dQ", f64(dq), rq)
        check_rel("dK", f64(dk), rk)
        check_rel("dV", f64(dv), rv)


# A derived bound may exceed the rounding model's own error by this factor
# (what the model leaves out: fp32 accumulation order, the running maximum's
# lag moving rounding boundaries).
MODEL_MARGIN = 1.5


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("d", [64, 128])
def test_very_negative_logsumexp_ragged_keys(d, causal):
    """Rows whose logsumexp is below -88 with a ragged last key tile (N = 100):
    a padded key's recomputed probability exp(0 - L) overflows float32, so
    the backward must mask keys past N rather than rely on their zero rows
    (0 * inf is NaN). Every key shares a large component along -q and all
    queries favour the same keys, so rounding errors add up coherently: the
    bf16 roundings alone exceed the plain gradient bounds
    (tests/test_rounding_bounds.py). The backward is therefore given the
    oracle's O (rounded to bf16) and logsumexp, so that its own roundings are
    the only error left, and each gradient is held to the larger of the
    magnitude-scaled bound and MODEL_MARGIN times the error of the fp64
    rounding model (tests/kernel_rounding.py) given the same O. The forward's
    O and logsumexp are checked against the plain bounds."""
    import torch

    B, N, H = 1, 100, 2
    scale = 1.0 / 8.0
    announce(f"very negative logsumexp d={d} causal={causal}")
    bits = si.draw_negative_logsumexp(B, N, H, d, 5 + d)
    q64, k64, v64, do64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v", "do"))
    rq, rk, rv, ro, rl, _ = oracle.attention_backward(q64, k64, v64, do64, causal, scale)
    assert rl.max() < -88.0
    q, k, v, o, lse = gpu_fwd(bits, causal, scale)
    check("O", f64(o), ro)
    check("LSE", f64(lse), rl, LSE_TOL, LSE_TOL)
    o_bits = si.f32_to_bf16_bits(ro.astype(np.float32))
    model = kr.emulate(q64, k64, v64, do64, causal, scale, o_in=si.bf16_bits_to_f64(o_bits))
    o_in = dev(o_bits)
    lse_in = torch.from_numpy(rl.astype(np.float32)).cuda()
    dq, dk, dv = gpu_bwd(q, k, v, o_in, lse_in, bits["do"], causal, scale)
    for name, got, ref in (("dQ", f64(dq), rq), ("dK", f64(dk), rk), ("dV", f64(dv), rv)):
        mmax, mmean = kr.error(model[name.lower()], ref)
        m = max(1.0, float(np.max(np.abs(ref))) / 2.0)
        gmax, gmean = kr.error(got, ref)
        report(f"[parity] negative-logsumexp d={d} causal={causal} {name}: max-abs {gmax:.3e} "
               f"(model {mmax:.3e}), mean-abs {gmean:.3e} (model {mmean:.3e})")
        check(name, got, ref, max(MAX_TOL * m, MODEL_MARGIN * mmax), max(MEAN_TOL * m, MODEL_MARGIN * mmean))


def tile_growth_share(q, k, causal, scale, tile=32):
    """Share of (row, key tile) pairs, past a row's first tile, where the
    row's running maximum of the scores (log2 units) grows by more than 8:
    the tiles whose probabilities, taken from the previous maximum, would
    exceed 2^8."""
    s = np.einsum("bihc,bjhc->bhij", q, k) * scale / np.log(2.0)
    N = k.shape[1]
    if causal:
        s = np.where(np.arange(N)[None, :] > np.arange(s.shape[2])[:, None], -np.inf, s)
    nt = (N + tile - 1) // tile
    tmax = np.stack([s[..., t * tile:(t + 1) * tile].max(axis=-1) for t in range(nt)], axis=-1)
    run = np.maximum.accumulate(tmax, axis=-1)
    grow = (tmax[..., 1:] > run[..., :-1] + 8.0) & np.isfinite(run[..., :-1])
    seen = np.isfinite(run[..., :-1]) & np.isfinite(tmax[..., 1:])
    return float(grow.sum() / max(1, seen.sum()))


@pytest.mark.parametrize("H", [2, 34], ids=["H2", "H34"])
@pytest.mark.parametrize("span", [4.0, 16.0], ids=["span4", "span16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("d", [64, 128])
def test_growing_scores_forward(d, causal, span, H):
    """Scores that grow along the keys, so each row's maximum keeps moving to
    later tiles. With span 16 the probabilities a tile takes from the running
    maximum overflow the 2^8 bound on nearly every tile, and the tile is
    taken again from its own row maxima; with span 4 they stay within it
    while the running maximum lags by several units. N = 1000 leaves a ragged
    last tile; at d = 128, 2 heads (16 workgroups) run the form whose wave
    groups split the keys and 34 heads (272) the plain one. O and the
    logsumexp are compared whole with the oracle."""
    B, N = 1, 1000
    scale = 1.0 / math.sqrt(d)
    seed = 7000 + d + 2 * int(causal) + int(span)
    announce(f"growing scores d={d} causal={causal} span={span} H={H} seed={seed}")
    bits = si.draw_growing_scores(B, N, H, d, seed, span)
    q64, k64, v64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v"))
    share = tile_growth_share(q64[:, :, :1], k64[:, :, :1], causal, scale)
    if span >= 16.0:
        assert share > 0.5, f"input does not exercise the rescale path (share {share:.2f})"
    ro, rl = oracle.attention_forward(q64, k64, v64, causal, scale)
    _, _, _, o, lse = gpu_fwd(bits, causal, scale)
    check("O", f64(o), ro)
    check("LSE", f64(lse), rl, LSE_TOL, LSE_TOL)


# ---------------------------------------------------------------------------
# closed forms and exact properties on the GPU


@pytest.mark.parametrize("d", [64, 128])
def test_zero_queries_closed_form(d):
    """Q = 0: causal O_i is the prefix mean of V and L_i = ln(i + 1)."""
    import torch

    B, N, H = 1, 300, 2
    announce(f"Q=0 closed form d={d}")
    bits = si.draw(B, N, H, d, 5 + d)
    bits["q"] = np.zeros_like(bits["q"])
    q, k, v, o, lse = gpu_fwd(bits, True, 1.0 / math.sqrt(d))
    v64 = si.bf16_bits_to_f64(bits["v"])
    prefix = np.cumsum(v64, axis=1) / np.arange(1, N + 1)[None, :, None, None]
    check("O prefix mean", f64(o), prefix, 2e-2, 2e-3)
    ref_l = np.broadcast_to(np.log(np.arange(1, N + 1)), (B, H, N))
    check("LSE ln(i+1)", f64(lse), ref_l, 1e-5, 1e-5)
    _, _, _, o2, lse2 = gpu_fwd(bits, False, 0.3)
    check("O mean", f64(o2), np.broadcast_to(v64.mean(axis=1, keepdims=True), o2.shape))
    check("LSE ln N", f64(lse2), np.full((B, H, N), math.log(N)), 1e-5, 1e-5)


@pytest.mark.parametrize("d", [64, 128])
def test_causal_row0_is_v0(d):
    """Causal query 0 sees only key 0, so O_0 = V_0 (expected bit-exact)."""
    announce(f"causal row0 d={d}")
    bits = si.draw(2, 130, 3, d, 9 + d)
    q, k, v, o, lse = gpu_fwd(bits, True, 1.0 / math.sqrt(d))
    got = si.torch_to_bits(o)[:, 0]
    ref = bits["v"][:, 0]
    diff_ulps = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    assert diff_ulps.max() <= 1 and np.mean(diff_ulps == 0) > 0.99


def test_deterministic_and_head_permutation():
    """The forward is bit-reproducible, and permuting heads permutes outputs
    bit-exactly (rows are independent; placement does not change the math)."""
    import torch

    B, N, H, d = 2, 700, 4, 128
    announce("determinism + head permutation")
    bits = si.draw(B, N, H, d, 31, backward=True)
    q, k, v, o1, l1 = gpu_fwd(bits, True, 0.1)
    _, _, _, o2, l2 = gpu_fwd(bits, True, 0.1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    perm = [2, 0, 3, 1]
    pbits = {n: np.ascontiguousarray(bits[n][:, :, perm]) for n in bits}
    _, _, _, o3, l3 = gpu_fwd(pbits, True, 0.1)
    assert torch.equal(o3, o1[:, :, perm]) and torch.equal(l3, l1[:, perm])
    dq1, dk1, dv1 = gpu_bwd(q, k, v, o1, l1, bits["do"], True, 0.1)
    dq2, dk2, dv2 = gpu_bwd(q, k, v, o1, l1, bits["do"], True, 0.1)
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    check("dQ repeat", f64(dq2), f64(dq1), 1e-2, 1e-4)


def test_workspace_contents_do_not_matter():
    import torch

    B, N, H, d = 1, 513, 2, 64
    announce("workspace garbage")
    bits = si.draw(B, N, H, d, 41, backward=True)
    q, k, v, o, lse = gpu_fwd(bits, False, 0.125)
    need = fa.fa_bwd_workspace_bytes(B, N, H, d)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    dq1, dk1, dv1 = gpu_bwd(q, k, v, o, lse, bits["do"], False, 0.125, workspace=ws)
    dq2, dk2, dv2 = gpu_bwd(q, k, v, o, lse, bits["do"], False, 0.125)
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    check("dQ", f64(dq1), f64(dq2), 1e-2, 1e-4)


# ---------------------------------------------------------------------------
# the benchmark workloads at full size, every element against the oracle


def bf16_floor(ref):
    """max |bf16(ref) - ref|: the error of rounding the exact result itself."""
    r = si.bf16_bits_to_f64(si.f32_to_bf16_bits(np.asarray(ref, dtype=np.float32)))
    return float(np.max(np.abs(r - ref)))


def check_whole(name, got, ref, max_tol=MAX_TOL, mean_tol=MEAN_TOL, floor=True):
    """check() over a whole tensor, printing its max-abs and mean-abs error
    (and the bf16 floor of the exact result) first."""
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    fl = f", bf16 floor {bf16_floor(ref):.3e}" if floor else ""
    report(f"[parity] {name}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}{fl} over {err.size} elements")
    check(name, got, ref, max_tol, mean_tol)


@pytest.mark.parametrize("name", ["tiny", "short_noncausal", "short_causal", "mid_causal", "long_causal"])
def test_workload_forward(name):
    """A forward workload in the benchmark's launch configuration: O and the
    logsumexp of every row of every head against the oracle."""
    w = si.WORKLOADS[name]
    announce(f"workload fwd {name} B={w.B} N={w.N} H={w.H} d={w.d} causal={w.causal}")
    bits = si.draw_workload(w)
    q, k, v, o, lse = gpu_fwd(bits, w.causal, w.scale)
    o_np, l_np = f64(o), f64(lse)
    del q, k, v, o, lse
    q64, k64, v64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v"))
    H = oh.head
    ro, rl = oh.by_head(lambda b, h: oracle.attention_forward(H(q64, b, h), H(k64, b, h), H(v64, b, h),
                                                              w.causal, w.scale), w.B, w.H, ("bnhd", "bhn"))
    check_whole(f"{name} O", o_np, ro)
    check_whole(f"{name} LSE", l_np, rl, LSE_TOL, LSE_TOL, floor=False)


def test_workload_train_forward_backward():
    """The benchmark step's workload: O, logsumexp, dQ, dK and dV of all 64
    heads against the oracle's forward and analytic backward."""
    w = si.WORKLOADS["train_causal"]
    announce(f"workload fwd+bwd train_causal B={w.B} N={w.N} H={w.H}")
    bits = si.draw_workload(w)
    q, k, v, o, lse = gpu_fwd(bits, w.causal, w.scale)
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, bits["do"], w.causal, w.scale)
    got = {n: f64(t) for n, t in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv))}
    del q, k, v, o, lse, dq, dk, dv
    q64, k64, v64, do64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v", "do"))
    H = oh.head
    rq, rk, rv, ro, rl = oh.by_head(
        lambda b, h: oracle.attention_backward(H(q64, b, h), H(k64, b, h), H(v64, b, h), H(do64, b, h),
                                               True, w.scale),
        w.B, w.H, ("bnhd", "bnhd", "bnhd", "bnhd", "bhn"))
    check_whole("train O", got["O"], ro)
    check_whole("train LSE", got["LSE"], rl, LSE_TOL, LSE_TOL, floor=False)
    check_whole("train dQ", got["dQ"], rq)
    check_whole("train dK", got["dK"], rk)
    check_whole("train dV", got["dV"], rv)


# ---------------------------------------------------------------------------
# the largest tensors the library accepts

MAX_ELEMS = (1 << 31) - (1 << 16)  # per tensor, the limit the library states


MAX_SHAPES = [
    (4681, 224, 16, 128),  # 224 = 128 + 96 rows: the 128-row forward
    (248, 4228, 16, 128),  # 4228 = 22 * 192 + 4 rows: the 192-row forward; its first causal block holds 4 rows
]


@pytest.mark.parametrize("shape", MAX_SHAPES, ids=lambda s: "B%dN%dH%dd%d" % s)
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_max_size_sampled_heads(causal, shape):
    """B*N*H*d exactly at the library's limit (4 GiB per bf16 tensor), N
    ragged, for each forward form: the heads farthest from the base pointers
    are compared whole, forward and backward, with the oracle. Heads are
    independent, so the other heads hold filler drawn on the device; their
    outputs are only required to be finite."""
    import torch

    B, N, H, d = shape
    assert B * N * H * d == MAX_ELEMS
    announce(f"max size B={B} N={N} H={H} d={d} causal={causal}")
    scale = d ** -0.5
    g = torch.Generator(device="cuda").manual_seed(7)
    q, k, v, do = (torch.randn(B, N, H, d, generator=g, device="cuda", dtype=torch.bfloat16) for _ in range(4))
    samples = [(0, 0), (B // 2, 7), (B - 1, H - 1)]
    head_bits = {}
    for i, (b, h) in enumerate(samples):
        bits = si.draw(1, N, 1, d, 900 + i, backward=True)
        head_bits[(b, h)] = bits
        for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
            t[b, :, h, :] = dev(bits[name])[0, :, 0, :]
    o, lse = fa.fa_fwd(q, k, v, causal, scale)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, do, causal, scale)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t).all()), "non-finite output"
    for (b, h), bits in head_bits.items():
        q64, k64, v64, do64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v", "do"))
        rq, rk, rv, ro, rl, _ = oracle.attention_backward(q64, k64, v64, do64, causal, scale)
        sl = lambda x: f64(x[b : b + 1, :, h : h + 1, :])
        check(f"O head {(b, h)}", sl(o), ro)
        check(f"LSE head {(b, h)}", f64(lse[b : b + 1, h : h + 1]), rl, LSE_TOL, LSE_TOL)
        check(f"dQ head {(b, h)}", sl(dq), rq)
        check(f"dK head {(b, h)}", sl(dk), rk)
        check(f"dV head {(b, h)}", sl(dv), rv)
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# d = 64 past 4096 keys (the launch switches the d = 64 kernel configuration
# by key count: four workgroups per CU up to 4096 keys, three beyond)

@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_d64_long_keys_sampled_rows(causal):
    B, N, H, d = 1, 5000, 2, 64
    scale = d ** -0.5
    announce(f"d64 long keys N={N} causal={causal}")
    bits = si.draw(B, N, H, d, 61)
    q, k, v, o, lse = gpu_fwd(bits, causal, scale)
    o_np, l_np = f64(o), f64(lse)
    assert np.all(np.isfinite(o_np)) and np.all(np.isfinite(l_np))
    q64, k64, v64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v"))
    rows = [0, 1, 63, 64, 127, 128, 2047, 4095, 4096, 4097, 4223, 4224, 4900, 4999]
    for h in range(H):
        ro, rl = oracle.attention_forward_rows(q64, k64, v64, causal, scale, 0, h, rows)
        check(f"O rows head {h}", o_np[0, rows, h, :], ro)
        check(f"LSE rows head {h}", l_np[0, h, rows], rl, LSE_TOL, LSE_TOL)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_d64_long_key_chunk(causal):
    """A 256-row query chunk at positions 4800.. over a 5000-key chunk at
    0.. (d = 64): the float32 chunk result against the oracle's chunk
    attention."""
    import torch

    H, d, Nq, Nk, q0 = 2, 64, 256, 5000, 4800
    scale = d ** -0.5
    announce(f"d64 long key chunk Nq={Nq} Nk={Nk} causal={causal}")
    qb = si.draw(1, Nq, H, d, 62)["q"]
    kvb = si.draw(1, Nk, H, d, 63)
    o, lse = fa.fa_fwd_chunk(dev(qb), dev(kvb["k"]), dev(kvb["v"]), causal, q_start=q0, k_start=0,
                             softmax_scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_chunk(si.bf16_bits_to_f64(qb), si.bf16_bits_to_f64(kvb["k"]),
                                            si.bf16_bits_to_f64(kvb["v"]), causal, scale, q0, 0)
    check("O_c", o.cpu().numpy().astype(np.float64), ro)
    check("L_c", lse.cpu().numpy().astype(np.float64), rl, LSE_TOL, LSE_TOL)


# ---------------------------------------------------------------------------
# d = 128 on both sides of the launch switch at one workgroup per CU: 16
# heads of 2000 rows (16 blocks each, 256 workgroups) run the form whose
# workgroups split the key tiles between two groups of waves and combine
# them, 17 heads (272 workgroups) the plain one. Both are compared whole
# with the oracle and with each other.

@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_launch_forms_agree(causal):
    import torch

    B, N, H, d = 1, 2000, 17, 128
    scale = d ** -0.5
    announce(f"launch forms N={N} H={H} vs {H - 1} causal={causal}")
    bits = si.draw(B, N, H, d, 64)
    q, k, v, o17, l17 = gpu_fwd(bits, causal, scale)
    q16, k16, v16 = (x[:, :, : H - 1, :].contiguous() for x in (q, k, v))
    o16, l16 = fa.fa_fwd(q16, k16, v16, causal, scale)
    torch.cuda.synchronize()
    q64, k64, v64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v"))
    ro, rl = oracle.attention_forward(q64, k64, v64, causal, scale)
    check("O (17 heads)", f64(o17), ro)
    check("LSE (17 heads)", f64(l17), rl, LSE_TOL, LSE_TOL)
    check("O (16 heads)", f64(o16), ro[:, :, : H - 1])
    check("LSE (16 heads)", f64(l16), rl[:, : H - 1], LSE_TOL, LSE_TOL)
    check("O forms", f64(o16), f64(o17[:, :, : H - 1]), 2e-2, 1e-3)


# d = 128 launches of more than one workgroup per CU: ragged lengths,
# lengths below one tile, many heads, every element against the oracle.
LARGE = [(1, 1000, 40), (2, 333, 100), (1, 4100, 9), (3, 17, 100), (1, 129, 300), (2, 2080, 9)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", LARGE, ids=lambda s: "B%dN%dH%d" % s)
def test_large_launch_forward(shape, causal):
    B, N, H = shape
    d = 128
    assert B * H * ((N + 127) // 128) > 256  # more than one workgroup per CU
    seed = 3000 + N + H + int(causal)
    announce(f"large launch fwd shape={(B, N, H, d)} causal={causal} seed={seed}")
    bits = si.draw(B, N, H, d, seed)
    q, k, v, o, lse = gpu_fwd(bits, causal, d ** -0.5)
    q64, k64, v64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v"))
    ro, rl = oracle.attention_forward(q64, k64, v64, causal, d ** -0.5)
    check("O", f64(o), ro)
    check("LSE", f64(lse), rl, LSE_TOL, LSE_TOL)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.9, 2.5], ids=lambda s: f"scale{s}")
def test_large_launch_forward_scales(scale):
    """Other softmax scales on a launch of more than one workgroup per CU (a
    negative one negates Q; 2.5 makes the running maximum move many times).
    At large scales the softmax is nearly one-hot and |O| reaches the size
    of V's largest entries, where bf16 rounding alone approaches 2e-2: O
    takes the magnitude-scaled bound (tests/test_rounding_bounds.py)."""
    B, N, H, d = 1, 700, 50, 128
    for causal in (False, True):
        announce(f"large launch fwd scale={scale} causal={causal}")
        bits = si.draw(B, N, H, d, 3100)
        q, k, v, o, lse = gpu_fwd(bits, causal, scale)
        q64, k64, v64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v"))
        ro, rl = oracle.attention_forward(q64, k64, v64, causal, scale)
        check_rel("O", f64(o), ro)
        check("LSE", f64(lse), rl, LSE_TOL, LSE_TOL)


@pytest.mark.parametrize("offsets", [(1500, 0), (700, 300), (0, 900), (-50, 0)], ids=lambda o: "q%d_k%d" % o)
def test_large_launch_chunk(offsets):
    """fa_fwd_chunk launches above one workgroup per CU (float32 output and a
    causal offset): a 1000-row query chunk of 40 heads over a 1500-key chunk,
    including rows that see no key."""
    import torch

    q0, k0 = offsets
    H, d, Nq, Nk = 40, 128, 1000, 1500
    scale = d ** -0.5
    announce(f"large launch chunk q_start={q0} k_start={k0}")
    qb = si.draw(1, Nq, H, d, 3200)["q"]
    kvb = si.draw(1, Nk, H, d, 3201)
    for causal in (False, True):
        o, lse = fa.fa_fwd_chunk(dev(qb), dev(kvb["k"]), dev(kvb["v"]), causal, q_start=q0, k_start=k0,
                                 softmax_scale=scale)
        torch.cuda.synchronize()
        ro, rl = oracle.attention_forward_chunk(si.bf16_bits_to_f64(qb), si.bf16_bits_to_f64(kvb["k"]),
                                                si.bf16_bits_to_f64(kvb["v"]), causal, scale, q0, k0)
        got_l = lse.cpu().numpy().astype(np.float64)
        empty = np.isneginf(rl)
        assert np.array_equal(np.isneginf(got_l), empty), "rows without a visible key differ"
        check("O_c", o.cpu().numpy().astype(np.float64), ro)
        check("L_c", got_l[~empty], rl[~empty], LSE_TOL, LSE_TOL)
