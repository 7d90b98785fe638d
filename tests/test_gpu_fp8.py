"""GPU parity of the FP8 (e4m3) forward (fa_fwd_fp8) against the fp64 oracle,
through the C ABI.

The reference is exact attention on the dequantized inputs. The kernel's own
low-precision step is the rounding of the probabilities to e4m3 for the P V
product (the products of e4m3 inputs are exact in fp32). A probability p' =
exp(s - max) is held as P = c p' with c between 2^4 and 2^8 (the running
max lags by at most 2^4) and rounded to nearest: the error is at most
2^-4 P in the normal range and 2^-10 below 2^-6. Divided by the fp32 row sum
sum(P), the error of output element (i, d) is therefore at most

    sum_j max(2^-4 p'_ij, 2^-14) |v_jd| / sum_j p'_ij

plus the bf16 rounding of the output (2^-9 |O|, taken as 2^-8 |O|); the
fp32 accumulation and exp2 errors are orders of magnitude smaller. Every
output element must lie within that bound. The logsumexp uses the fp32
values and keeps the core 1e-3 bound.
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


def run(b8, causal, scale):
    import torch

    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in b8.items()}
    o, lse = fa.fa_fwd_fp8(t["q"], t["k"], t["v"], t["q_descale"], t["k_descale"], t["v_descale"], causal, scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_head(o_gpu, l_gpu, ro, rl, q, k, v, causal, scale, what=""):
    """One head: the GPU output against the oracle's (ro, rl), element by
    element within the derived bound. The bound's own fp64 reference rows
    must equal the oracle's, so the bound is centred on the oracle's result."""
    bo, _, bd = head_bound(q, k, v, causal, scale)
    assert np.allclose(bo, ro, rtol=1e-12, atol=1e-12), f"{what}: bound reference differs from the oracle"
    err = np.abs(o_gpu - ro)
    ratio = err / bd
    worst = np.unravel_index(int(ratio.argmax()), ratio.shape)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    assert ratio.max() <= 1.0, (f"{what}: error {err[worst]:.3e} exceeds its bound {bd[worst]:.3e} at {worst} "
                                f"(max ratio {ratio.max():.3f})")
    lerr = np.abs(l_gpu - rl).max()
    assert lerr <= LSE_TOL, f"{what}: logsumexp max-abs {lerr:.3e}"
    return float(ratio.max()), float(err.max()), float(err.mean()), float(lerr)


def deq(b8, name):
    return oracle.dequantize_fp8(b8[name], b8[name + "_descale"])


SMALL = [(1, 1, 1), (1, 17, 2), (2, 64, 2), (1, 129, 3), (1, 200, 2), (2, 333, 1), (1, 1000, 1)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dN%dH%d" % s)
def test_fp8_small(shape, causal, d):
    B, N, H = shape
    seed = 10100 + N + int(causal) + d
    scale = 1.0 / math.sqrt(d)
    announce(f"fp8 fwd shape={(B, N, H, d)} causal={causal} seed={seed}")
    b8 = si.draw_fp8(B, N, H, d, seed)
    o, lse = run(b8, causal, scale)
    q, k, v = deq(b8, "q"), deq(b8, "k"), deq(b8, "v")
    ro, rl = oracle.attention_forward_fp8(b8["q"], b8["k"], b8["v"], b8["q_descale"], b8["k_descale"],
                                          b8["v_descale"], causal, scale)
    for bb in range(B):
        for h in range(H):
            check_head(o[bb, :, h], lse[bb, h], ro[bb, :, h], rl[bb, h], q[bb, :, h], k[bb, :, h], v[bb, :, h],
                       causal, scale, what=f"b{bb} h{h}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("span", [4.0, 16.0], ids=["span4", "span16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_fp8_growing_scores(causal, span, d):
    """Scores that grow along the keys: with span 16 a tile's P taken from
    the running maximum leaves e4m3's range on nearly every tile and is taken
    again from the tile's own row maxima; with span 4 it stays within 448
    while the running maximum lags. Every element within the derived bound."""
    B, N, H = 1, 1000, 2
    scale = 1.0 / math.sqrt(d)
    announce(f"fp8 growing scores causal={causal} span={span} d={d}")
    b8 = si.draw_fp8_growing_scores(B, N, H, d, 7200 + int(span) + d, span)
    o, lse = run(b8, causal, scale)
    q, k, v = deq(b8, "q"), deq(b8, "k"), deq(b8, "v")
    ro, rl = oracle.attention_forward_fp8(b8["q"], b8["k"], b8["v"], b8["q_descale"], b8["k_descale"],
                                          b8["v_descale"], causal, scale)
    for h in range(H):
        check_head(o[0, :, h], lse[0, h], ro[0, :, h], rl[0, h], q[0, :, h], k[0, :, h], v[0, :, h],
                   causal, scale, what=f"h{h}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("qd_sign", [1.0, -1.0], ids=["pos", "neg"])
def test_fp8_descales(qd_sign, d):
    """Descales far from 1 and a negative Q descale (negates the scores)."""
    B, N, H = 1, 300, 2
    announce(f"fp8 descales sign={qd_sign} d={d}")
    b8 = si.draw_fp8(B, N, H, d, 10200 + d)
    b8["q_descale"] = (b8["q_descale"] * np.float32(qd_sign) * np.float32(8.0)).astype(np.float32)
    b8["k_descale"] = (b8["k_descale"] / np.float32(4.0)).astype(np.float32)
    b8["v_descale"] = (b8["v_descale"] * np.float32(1000.0)).astype(np.float32)
    o, lse = run(b8, True, 0.09)
    q, k, v = deq(b8, "q"), deq(b8, "k"), deq(b8, "v")
    ro, rl = oracle.attention_forward_fp8(b8["q"], b8["k"], b8["v"], b8["q_descale"], b8["k_descale"],
                                          b8["v_descale"], True, 0.09)
    for h in range(H):
        check_head(o[0, :, h], lse[0, h], ro[0, :, h], rl[0, h], q[0, :, h], k[0, :, h], v[0, :, h], True, 0.09,
                   what=f"h{h}")


@pytest.mark.parametrize("name", list(si.FP8_WORKLOADS))
def test_fp8_workload(name):
    """The FP8 workloads at full size, as the benchmark runs them: every
    element of every head against the oracle's result on the dequantized
    inputs, within the derived bound (the oracle and the bound run head by
    head in a thread pool)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from tests import oracle_heads as oh

    w = si.FP8_WORKLOADS[name]
    announce(f"fp8 workload {name}: B={w.B} H={w.H} N={w.N} d={w.d}")
    b8 = si.draw_fp8(w.B, w.N, w.H, w.d, w.seed)
    o, lse = run(b8, w.causal, w.scale)

    def one(bh):
        bb, h = bh
        sl = lambda n: b8[n][bb : bb + 1, :, h : h + 1, :]
        ds = lambda n: b8[n + "_descale"][bb : bb + 1, h : h + 1]
        ro, rl = oracle.attention_forward_fp8(sl("q"), sl("k"), sl("v"), ds("q"), ds("k"), ds("v"),
                                              w.causal, w.scale)
        q, k, v = (oracle.dequantize_fp8(sl(n), ds(n))[0, :, 0, :] for n in ("q", "k", "v"))
        return check_head(o[bb, :, h], lse[bb, h], ro[0, :, 0, :], rl[0, 0], q, k, v, w.causal, w.scale,
                          what=f"b{bb} h{h}")

    pairs = [(bb, h) for bb in range(w.B) for h in range(w.H)]
    with threadpool_limits(1), ThreadPoolExecutor(oh.workers()) as ex:
        res = list(ex.map(one, pairs))
    ratio = max(r[0] for r in res)
    mx = max(r[1] for r in res)
    mean = sum(r[2] for r in res) / len(res)
    lerr = max(r[3] for r in res)
    report(f"[parity] {name} O: max error / bound {ratio:.3f}, max-abs {mx:.3e} mean-abs {mean:.3e} over "
             f"{o.size} elements; LSE max-abs {lerr:.3e}")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_fp8_d64_short_sequences(causal):
    """d = 64 at the short-sequence shape (B=32 H=16 N=512; 2048 workgroups,
    four per CU): every element of every head within the bound."""
    B, N, H, d = 32, 512, 16, 64
    scale = 1.0 / math.sqrt(d)
    announce(f"fp8 d=64 B={B} N={N} H={H} causal={causal}")
    b8 = si.draw_fp8(B, N, H, d, 10300 + int(causal))
    o, lse = run(b8, causal, scale)
    ro, rl = oracle.attention_forward_fp8(b8["q"], b8["k"], b8["v"], b8["q_descale"], b8["k_descale"],
                                          b8["v_descale"], causal, scale)
    q, k, v = deq(b8, "q"), deq(b8, "k"), deq(b8, "v")
    res = [check_head(o[bb, :, h], lse[bb, h], ro[bb, :, h], rl[bb, h], q[bb, :, h], k[bb, :, h], v[bb, :, h],
                      causal, scale, what=f"b{bb} h{h}") for bb in range(B) for h in range(H)]
    report(f"[parity] fp8 d=64 B={B} N={N} H={H} causal={causal} O: max error / bound "
           f"{max(r[0] for r in res):.3f}; LSE max-abs {max(r[3] for r in res):.3e}")


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_deterministic(d):
    """Two calls on the same inputs give bit-identical outputs."""
    B, N, H = 2, 700, 3
    announce(f"fp8 determinism d={d}")
    b8 = si.draw_fp8(B, N, H, d, 10400 + d)
    o1, l1 = run(b8, True, 0.11)
    o2, l2 = run(b8, True, 0.11)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)

