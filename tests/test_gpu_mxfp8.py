"""GPU parity of the microscaled FP8 forward (fa_fwd_mxfp8) against the fp64
oracle, through the C ABI.

The reference is exact attention on the values the codes and block scales
stand for (oracle.attention_forward_mxfp8). The matrix instruction applies
the power-of-two block scales exactly, so the products stay exact in fp32 as
in the per-head FP8 form, and the kernel's own low-precision step is again
the e4m3 rounding of the probabilities for the P V product: every output
element is held to the same derived bound (tests/fp8_bound.py), the
logsumexp to 1e-3.
"""

import math
import sys

import numpy as np
import pytest

import exact_tiled_attention_37_amd as fa
import oracle
import seeded_inputs as si
from tests import parity_log
from tests.fp8_bound import head_bound

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-3


def announce(msg):
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")
    fa.load_library()


def run(b8, causal, scale):
    import torch

    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in b8.items()}
    o, lse = fa.fa_fwd_mxfp8(t["q"], t["q_scale"], t["k"], t["k_scale"], t["v"], t["v_scale"], causal, scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def values(b8):
    """The values the codes and scales stand for (the oracle's dequantization)."""
    return (oracle.dequantize_mx_rows(b8["q"], b8["q_scale"]), oracle.dequantize_mx_rows(b8["k"], b8["k_scale"]),
            oracle.dequantize_mx_cols(b8["v"], b8["v_scale"]))


def check_head(o_gpu, l_gpu, ro, rl, q, k, v, causal, scale, what=""):
    bo, _, bd = head_bound(q, k, v, causal, scale)
    assert np.allclose(bo, ro, rtol=1e-12, atol=1e-12), f"{what}: bound reference differs from the oracle"
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    err = np.abs(o_gpu - ro)
    ratio = err / bd
    worst = np.unravel_index(int(ratio.argmax()), ratio.shape)
    assert ratio.max() <= 1.0, (f"{what}: error {err[worst]:.3e} exceeds its bound {bd[worst]:.3e} at {worst} "
                                f"(max ratio {ratio.max():.3f})")
    lerr = np.abs(l_gpu - rl).max()
    assert lerr <= LSE_TOL, f"{what}: logsumexp max-abs {lerr:.3e}"
    return float(ratio.max()), float(err.max()), float(err.mean()), float(lerr)


def check_all(b8, causal, scale, o, lse):
    ro, rl = oracle.attention_forward_mxfp8(b8["q"], b8["q_scale"], b8["k"], b8["k_scale"], b8["v"], b8["v_scale"],
                                            causal, scale)
    q, k, v = values(b8)
    B, _, H, _ = q.shape
    for bb in range(B):
        for h in range(H):
            check_head(o[bb, :, h], lse[bb, h], ro[bb, :, h], rl[bb, h], q[bb, :, h], k[bb, :, h], v[bb, :, h],
                       causal, scale, what=f"b{bb} h{h}")


# N: a single token, short V blocks (N % 32 != 0), whole and ragged 64-key tiles
SMALL = [(1, 1, 1), (1, 17, 2), (2, 64, 2), (1, 129, 3), (1, 200, 2), (2, 333, 1), (1, 1000, 1)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dN%dH%d" % s)
def test_mxfp8_small(shape, causal, d):
    B, N, H = shape
    seed = 12100 + N + int(causal) + d
    scale = 1.0 / math.sqrt(d)
    announce(f"mxfp8 fwd shape={(B, N, H, d)} causal={causal} seed={seed}")
    b8 = si.draw_mxfp8(B, N, H, d, seed)
    o, lse = run(b8, causal, scale)
    check_all(b8, causal, scale, o, lse)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("span", [4.0, 16.0], ids=["span4", "span16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_mxfp8_growing_scores(causal, span, d):
    """Scores that grow along the keys (the running max moves on most tiles
    with span 16, lags within e4m3's range with span 4)."""
    B, N, H = 1, 1000, 2
    scale = 1.0 / math.sqrt(d)
    announce(f"mxfp8 growing scores causal={causal} span={span} d={d}")
    b8 = si.draw_mxfp8_growing_scores(B, N, H, d, 7300 + int(span) + d, span)
    o, lse = run(b8, causal, scale)
    check_all(b8, causal, scale, o, lse)


@pytest.mark.parametrize("d", [64, 128])
def test_mxfp8_block_scales_matter(d):
    """Scales that differ from block to block by large factors, so that a
    scale applied to the wrong block (or to the wrong half of a lane's
    operand, or to the wrong keys of a tile) moves the result far outside the
    bound: Q's d-blocks at 2^-6 .. 2^+3 of each other, K's the other way
    round, V's key blocks alternating by 2^5 and its columns by 2^3, and a
    negative softmax scale."""
    B, N, H = 1, 300, 2
    announce(f"mxfp8 block scales far apart d={d}")
    b8 = si.draw_mxfp8(B, N, H, d, 12300 + d)
    rng = np.random.Generator(np.random.PCG64(12301))
    b8["q_scale"] = (b8["q_scale"].astype(np.int64) + np.array([-6, 3, 0, -2])[: d // 32]).astype(np.uint8)
    b8["k_scale"] = (b8["k_scale"].astype(np.int64) + np.array([4, -3, 1, 0])[: d // 32]).astype(np.uint8)
    vs = b8["v_scale"].astype(np.int64)
    vs += 5 * (np.arange(vs.shape[1]) % 2)[None, :, None, None] + 3 * (np.arange(d) % 3 == 0)[None, None, None, :]
    vs += rng.integers(-2, 3, vs.shape)
    b8["v_scale"] = vs.astype(np.uint8)
    for causal, scale in ((True, 0.09), (False, -0.07)):
        o, lse = run(b8, causal, scale)
        check_all(b8, causal, scale, o, lse)


def test_mxfp8_unit_scales_match_the_per_head_form():
    """With every block scale at 2^0 the microscaled call and the per-head
    call (unit descales) compute attention on the same values: both within
    the bound of the same oracle result."""
    import torch

    B, N, H, d = 1, 257, 2, 128
    announce("mxfp8 unit scales vs per-head form")
    # codes of N(0, 1) values themselves (no scaling needed at unit scales)
    rng = np.random.Generator(np.random.PCG64(12400))
    b8 = {n: si.f64_to_e4m3_bits(rng.standard_normal((B, N, H, d))) for n in ("q", "k", "v")}
    one = lambda *s: np.full(s, 127, np.uint8)
    mx = {"q": b8["q"], "k": b8["k"], "v": b8["v"], "q_scale": one(B, N, H, d // 32),
          "k_scale": one(B, N, H, d // 32), "v_scale": one(B, (N + 31) // 32, H, d)}
    o, lse = run(mx, True, 0.1)
    check_all(mx, True, 0.1, o, lse)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in b8.items() if k in ("q", "k", "v")}
    unit = torch.ones(B, H, dtype=torch.float32, device="cuda")
    o2, l2 = fa.fa_fwd_fp8(t["q"], t["k"], t["v"], unit, unit, unit, True, 0.1)
    torch.cuda.synchronize()
    check_all(mx, True, 0.1, o2.float().cpu().numpy().astype(np.float64), l2.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("name", list(si.MXFP8_WORKLOADS))
def test_mxfp8_workload(name):
    """The microscaled workloads at full size: every element of every head
    against the oracle within the derived bound (heads in a thread pool)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from tests import oracle_heads as oh

    w = si.MXFP8_WORKLOADS[name]
    announce(f"mxfp8 workload {name}: B={w.B} H={w.H} N={w.N} d={w.d}")
    b8 = si.draw_mxfp8(w.B, w.N, w.H, w.d, w.seed)
    o, lse = run(b8, w.causal, w.scale)

    def one(bh):
        bb, h = bh
        sl = lambda n: b8[n][bb : bb + 1, :, h : h + 1, :]
        ro, rl = oracle.attention_forward_mxfp8(sl("q"), sl("q_scale"), sl("k"), sl("k_scale"), sl("v"),
                                                sl("v_scale"), w.causal, w.scale)
        q = oracle.dequantize_mx_rows(sl("q"), sl("q_scale"))[0, :, 0, :]
        k = oracle.dequantize_mx_rows(sl("k"), sl("k_scale"))[0, :, 0, :]
        v = oracle.dequantize_mx_cols(sl("v"), sl("v_scale"))[0, :, 0, :]
        return check_head(o[bb, :, h], lse[bb, h], ro[0, :, 0, :], rl[0, 0], q, k, v, w.causal, w.scale,
                          what=f"b{bb} h{h}")

    pairs = [(bb, h) for bb in range(w.B) for h in range(w.H)]
    with threadpool_limits(1), ThreadPoolExecutor(oh.workers()) as ex:
        res = list(ex.map(one, pairs))
    msg = (f"[parity] {name} O: max error / bound {max(r[0] for r in res):.3f}, max-abs "
           f"{max(r[1] for r in res):.3e} mean-abs {sum(r[2] for r in res) / len(res):.3e} over {o.size} "
           f"elements; LSE max-abs {max(r[3] for r in res):.3e}")
    announce(msg)
    parity_log.record(msg)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_mxfp8_d64_short_sequences(causal):
    """d = 64 at the short-sequence shape (B=32 H=16 N=512): every element of
    every head within the bound."""
    B, N, H, d = 32, 512, 16, 64
    scale = 1.0 / math.sqrt(d)
    announce(f"mxfp8 d=64 B={B} N={N} H={H} causal={causal}")
    b8 = si.draw_mxfp8(B, N, H, d, 12500 + int(causal))
    o, lse = run(b8, causal, scale)
    check_all(b8, causal, scale, o, lse)


@pytest.mark.parametrize("d", [64, 128])
def test_mxfp8_deterministic(d):
    """Two calls on the same inputs give bit-identical outputs (no atomics or
    order-dependent reductions on the path)."""
    B, N, H = 2, 700, 3
    announce(f"mxfp8 determinism d={d}")
    b8 = si.draw_mxfp8(B, N, H, d, 12600 + d)
    o1, l1 = run(b8, True, 0.11)
    o2, l2 = run(b8, True, 0.11)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)

