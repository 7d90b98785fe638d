"""GPU parity of decode-shaped attention (fa_decode) against the fp64 oracle,
through the C ABI.

The queries are the last Nq positions of the key sequence (bottom-right
causal alignment). Keys are split into ranges whose float32 results are
merged, so the outputs carry the same roundings as the prefill path: O
max-abs 2e-2 / mean-abs 2e-3, logsumexp max-abs 1e-3; rows that see no key
must be exactly o = 0, lse = -inf.
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
    if got.size == 0:
        return
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    assert mx <= max_tol and mn <= mean_tol, (
        f"{name}: max-abs {mx:.3e} (tol {max_tol}), mean-abs {mn:.3e} (tol {mean_tol}), "
        f"at {np.unravel_index(int(err.argmax()), err.shape)}"
    )


def check_out(o, lse, ro, rl):
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), "rows without a visible key differ"
    assert np.all(o[empty.transpose(0, 2, 1)] == 0.0), "rows without a visible key must be zero"
    check("O", o, ro)
    check("LSE", lse[~empty], rl[~empty], LSE_TOL, LSE_TOL)


SMALL = [
    # (B, Nq, Nk, H, d)
    (2, 1, 1000, 3, 128),
    (1, 16, 4097, 2, 64),
    (3, 5, 300, 2, 128),
    (1, 40, 1000, 2, 128),   # more than one 32-row query block
    (1, 7, 4, 2, 64),        # more queries than keys: the first 3 rows see none
    (1, 1, 1, 1, 64),
    (2, 32, 12345, 1, 128),
    (1, 3, 33, 2, 128),
]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dNq%dNk%dH%dd%d" % s)
def test_decode_small(shape, causal):
    import torch

    B, Nq, Nk, H, d = shape
    seed = 7000 + Nq + 5 * Nk + d
    scale = 1.0 / math.sqrt(d)
    announce(f"decode shape={shape} causal={causal} seed={seed} splits_ws={fa.fa_decode_workspace_bytes(B, Nq, Nk, H, d)}")
    bits = si.draw_qkv(B, Nq, Nk, H, d, seed)
    ro, rl = oracle.attention_decode(*(si.bf16_bits_to_f64(bits[t]) for t in ("q", "k", "v")), causal, scale)
    o, lse = fa.fa_decode(dev(bits["q"]), dev(bits["k"]), dev(bits["v"]), causal, scale)
    torch.cuda.synchronize()
    check_out(f64(o), f64(lse), ro, rl)


def test_decode_workspace_garbage_and_reuse():
    """The workspace's contents on entry do not matter, and two calls of
    different shapes may share one workspace in sequence."""
    import torch

    announce("decode workspace reuse")
    shapes = [(2, 4, 3000, 2, 128), (1, 9, 777, 3, 64)]
    need = max(fa.fa_decode_workspace_bytes(*s) for s in shapes)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    for i, (B, Nq, Nk, H, d) in enumerate(shapes):
        bits = si.draw_qkv(B, Nq, Nk, H, d, 7500 + i)
        ro, rl = oracle.attention_decode(*(si.bf16_bits_to_f64(bits[t]) for t in ("q", "k", "v")), True,
                                         1.0 / math.sqrt(d))
        o, lse = fa.fa_decode(dev(bits["q"]), dev(bits["k"]), dev(bits["v"]), True, workspace=ws)
        torch.cuda.synchronize()
        check_out(f64(o), f64(lse), ro, rl)


def test_decode_matches_prefill_rows():
    """Decode of the last rows equals those rows of the causal prefill
    (within tolerance of each other: different key orders and splits)."""
    import torch

    announce("decode vs prefill rows")
    B, N, H, d = 1, 2000, 2, 128
    bits = si.draw(B, N, H, d, 7600)
    q, k, v = dev(bits["q"]), dev(bits["k"]), dev(bits["v"])
    o_pre, l_pre = fa.fa_fwd(q, k, v, True)
    o_dec, l_dec = fa.fa_decode(q[:, N - 8:].contiguous(), k, v, True)
    torch.cuda.synchronize()
    check("decode vs prefill O", f64(o_dec), f64(o_pre[:, N - 8:]))
    check("decode vs prefill LSE", f64(l_dec), f64(l_pre[:, :, N - 8:]), LSE_TOL, LSE_TOL)


@pytest.mark.parametrize("name", list(si.DECODE_WORKLOADS))
def test_decode_workloads(name):
    """The decode workloads at full size, as the benchmark runs them: every
    (batch, head) against the oracle (run head by head in a thread pool)."""
    import torch

    from tests import oracle_heads as oh

    w = si.DECODE_WORKLOADS[name]
    announce(f"decode workload {name}: B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d}")
    bits = si.draw_decode(w)
    o, lse = fa.fa_decode(dev(bits["q"]), dev(bits["k"]), dev(bits["v"]), w.causal, w.scale)
    torch.cuda.synchronize()
    o, lse = f64(o), f64(lse)
    x = {t: si.bf16_bits_to_f64(bits[t]) for t in ("q", "k", "v")}
    H = oh.head
    ro, rl = oh.by_head(lambda b, h: oracle.attention_decode(H(x["q"], b, h), H(x["k"], b, h), H(x["v"], b, h),
                                                             w.causal, w.scale), w.B, w.H, ("bnhd", "bhn"))
    err = np.abs(o - ro)
    report(f"[parity] {name} O: max-abs {err.max():.3e} mean-abs {err.mean():.3e} over {err.size} elements; "
             f"LSE max-abs {np.abs(lse - rl).max():.3e}")
    check_out(o, lse, ro, rl)
