"""GPU parity of the d = 128 forward in the form large self-attention
launches take: workgroups of 192 query rows (four waves of 48 rows on
16x16x32 matrix instructions); causal blocks are aligned to the end of the
sequence, so that the one partial block is the first, lightest one,
non-causal ones start at row 0. The library takes it at d = 128 for at least
2048 keys when B * H * ceil(N / 192) exceeds 512 (more than one round of two
workgroups per CU); every shape here is just above those limits, so that
the form's edge cases are reached: a first causal block that holds a single
row, waves with no row at all, rows that start inside a wave, N a multiple
of the block, partial last blocks and ragged last key tiles. O and the
logsumexp are compared with the oracle on every element (the oracle runs
head by head in a thread pool)."""

import math
import sys

import numpy as np
import pytest

import exact_tiled_attention_37_amd as fa
import oracle
import seeded_inputs as si
from tests import oracle_heads as oh

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL, LSE_TOL = 2e-2, 2e-3, 1e-3
BLOCK_ROWS, ONE_ROUND, MIN_KEYS = 192, 512, 2048  # rows per workgroup; two workgroups on each of 256 CUs

CAUSAL_CASES = [
    # (B, N, H)
    (1, 2113, 48),  # 12 blocks per head: the first (causal) holds only row 0, in its last wave
    (1, 2200, 44),  # block 0 starts at row -104: its first two waves have no row, the third starts at row 0
    (1, 2304, 45),  # N a multiple of 192: no partial block
    (1, 2900, 40),  # 16 blocks, ragged last key tile
    (48, 2050, 1),  # one head per batch: 256-byte token stride, batch offsets carry the heads
]
NONCAUSAL_CASES = [
    (1, 2100, 48),  # partial last block (rows past N absent), ragged last key tile
    (1, 4096, 24),  # whole blocks and tiles except the last block
]


def announce(msg):
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")
    fa.load_library()
    return torch.device("cuda:0")


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, got, ref, max_tol, mean_tol):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    announce(f"{name}: max-abs {mx:.3e} mean-abs {mn:.3e} over {err.size} elements")
    assert mx <= max_tol and mn <= mean_tol, (
        f"{name}: max-abs {mx:.3e} (tol {max_tol}), mean-abs {mn:.3e} (tol {mean_tol}), "
        f"at {np.unravel_index(int(err.argmax()), err.shape)}"
    )


def in_regime(B, N, H):
    return N >= MIN_KEYS and B * H * math.ceil(N / BLOCK_ROWS) > ONE_ROUND


def run_and_compare(bits, B, N, H, scale, scaled=False, causal=True):
    """scaled: O's bounds grow with its magnitude M = max|ref| beyond 2 (as
    the other parity tests do for scales other than 1/sqrt(d)): the bf16
    roundings of P and of O are relative, 2e-2 * M / 2 is about 2.5 bf16
    ulps of M."""
    import torch

    q, k, v = (si.bits_to_torch(bits[n], "cuda") for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, causal, scale)
    torch.cuda.synchronize()
    q64, k64, v64 = (si.bf16_bits_to_f64(bits[n]) for n in ("q", "k", "v"))
    ro, rl = oh.by_head(
        lambda b, h: oracle.attention_forward(oh.head(q64, b, h), oh.head(k64, b, h), oh.head(v64, b, h), causal, scale),
        B, H, ("bnhd", "bhn"))
    m = max(1.0, float(np.max(np.abs(ro))) / 2.0) if scaled else 1.0
    check("O", f64(o), ro, MAX_TOL * m, MEAN_TOL * m)
    check("LSE", f64(lse), rl, LSE_TOL, LSE_TOL)
    return o, lse


@pytest.mark.parametrize("case", CAUSAL_CASES, ids=lambda c: "B%dN%dH%d" % c)
def test_large_causal_launch(case):
    B, N, H = case
    assert in_regime(B, N, H)
    seed = 4800 + N
    announce(f"192-row causal forward B={B} N={N} H={H} seed={seed}")
    bits = si.draw(B, N, H, 128, seed)
    run_and_compare(bits, B, N, H, 1.0 / math.sqrt(128))


@pytest.mark.parametrize("case", NONCAUSAL_CASES, ids=lambda c: "B%dN%dH%d" % c)
def test_large_noncausal_launch(case):
    B, N, H = case
    assert in_regime(B, N, H)
    seed = 4850 + N
    announce(f"192-row non-causal forward B={B} N={N} H={H} seed={seed}")
    bits = si.draw(B, N, H, 128, seed)
    run_and_compare(bits, B, N, H, 1.0 / math.sqrt(128), causal=False)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.9], ids=lambda s: f"scale{s}")
def test_large_launch_other_scales(scale, causal):
    """A negative scale (Q negated on load), zero (every visible key equally
    likely: causal rows are prefix means of V) and a large one."""
    B, N, H = 1, 2200, 44
    announce(f"192-row forward scale={scale} causal={causal}")
    bits = si.draw(B, N, H, 128, 4900)
    run_and_compare(bits, B, N, H, scale, scaled=True, causal=causal)


@pytest.mark.parametrize("span", [4.0, 16.0], ids=["span4", "span16"])
def test_large_causal_launch_growing_scores(span):
    """Scores that grow along the keys, so the running maximum keeps moving:
    with span 16 most tiles fail the 2^8 sum test and are taken again from
    their row maxima (the rescale path), with span 4 the maximum lags."""
    B, N, H = 1, 2200, 44
    announce(f"192-row causal forward growing scores span={span}")
    bits = si.draw_growing_scores(B, N, H, 128, 4950 + int(span), span)
    run_and_compare(bits, B, N, H, 1.0 / math.sqrt(128))


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_large_launch_deterministic_and_head_permutation(causal):
    """Bit-reproducible, and permuting heads permutes the outputs bit for bit
    (a head's blocks may land on other CUs and XCDs; the rows do not change)."""
    import torch

    B, N, H = 1, 2304, 45
    announce(f"192-row forward determinism + head permutation causal={causal}")
    bits = si.draw(B, N, H, 128, 4990)
    dv = {n: si.bits_to_torch(bits[n], "cuda") for n in ("q", "k", "v")}
    o1, l1 = fa.fa_fwd(dv["q"], dv["k"], dv["v"], causal, 0.1)
    o2, l2 = fa.fa_fwd(dv["q"], dv["k"], dv["v"], causal, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    perm = np.random.Generator(np.random.PCG64(3)).permutation(H)
    pv = {n: si.bits_to_torch(np.ascontiguousarray(bits[n][:, :, perm]), "cuda") for n in ("q", "k", "v")}
    o3, l3 = fa.fa_fwd(pv["q"], pv["k"], pv["v"], causal, 0.1)
    torch.cuda.synchronize()
    p = torch.as_tensor(perm, device="cuda")
    assert torch.equal(o3, o1.index_select(2, p)) and torch.equal(l3, l1.index_select(1, p))


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("case", [(1, 2048, 46), (1, 2048, 47), (1, 2047, 60)], ids=lambda c: "B%dN%dH%d" % c)
def test_switch_boundary(case, causal):
    """Both sides of the launch switch at N = 2048: 46 heads (506 workgroups
    of 192 rows, one round or less: the 128-row form), 47 heads (517: the
    192-row form) and N = 2047 (below the key limit: the 128-row form), each
    against the oracle."""
    B, N, H = case
    assert in_regime(B, N, H) == (H == 47)
    announce(f"switch boundary B={B} N={N} H={H} causal={causal}")
    bits = si.draw(B, N, H, 128, 5000 + H)
    run_and_compare(bits, B, N, H, 1.0 / math.sqrt(128), causal=causal)
