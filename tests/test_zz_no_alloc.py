"""fa_decode_noalloc (no workspace argument, no allocation: the key-split
partial results live in the library's static 32 MiB device scratch) against
fa_decode with a caller-supplied workspace, through the C ABI.

Both run the same kernels with the same key split, so the outputs must be
bit-identical. The calls run back to back on one device, the second with a
smaller input than the first (the scratch keeps the first call's contents),
then a shape that needs no scratch at all, then the first shape again.
"""

import sys

import numpy as np
import pytest

import exact_tiled_attention_37_amd as fa
import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

FA_ERR_SCRATCH = 9


def announce(msg):
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")
    fa.load_library()


def draw(B, Nq, Nk, H, d, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return {n: si.f32_to_bf16_bits(rng.standard_normal((B, rows, H, d), dtype=np.float32))
            for n, rows in (("q", Nq), ("k", Nk), ("v", Nk))}


# (B, Nq, Nk, H, d, causal): scratch needed 16.1 MiB, 0.02 MiB, none, 16.1 MiB
SHAPES = [(4, 16, 16384, 16, 128, True), (2, 3, 1000, 4, 64, False), (1, 1, 100, 1, 64, True),
          (4, 16, 16384, 16, 128, False)]


def test_noalloc_matches_decode_on_successive_calls():
    import torch

    for i, (B, Nq, Nk, H, d, causal) in enumerate(SHAPES):
        announce(f"decode_noalloc call {i}: B={B} Nq={Nq} Nk={Nk} H={H} d={d} causal={causal}")
        bits = draw(B, Nq, Nk, H, d, 700 + i)
        q, k, v = (si.bits_to_torch(bits[n], "cuda") for n in ("q", "k", "v"))
        scale = d ** -0.5
        o_ref, l_ref = fa.fa_decode(q, k, v, causal, scale)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
        fa.fa_decode_noalloc(q, k, v, causal, scale, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"call {i}: O differs from fa_decode"
        assert torch.equal(lse, l_ref), f"call {i}: LSE differs from fa_decode"
        # and one head against the oracle, to the core tolerances
        x = {n: si.bf16_bits_to_f64(bits[n][:1, :, :1]) for n in ("q", "k", "v")}
        ro, rl = oracle.attention_decode(x["q"], x["k"], x["v"], causal, scale)
        got = o[:1, :, :1].float().cpu().numpy().astype(np.float64)
        assert np.abs(got - ro).max() <= 2e-2 and np.abs(got - ro).mean() <= 2e-3
        assert np.abs(lse[:1, :1].cpu().numpy() - rl).max() <= 1e-3
        del q, k, v, o, lse, o_ref, l_ref


def test_noalloc_rejects_calls_beyond_its_scratch():
    import torch

    B, Nq, Nk, H, d = 1, 32, 218560, 3, 128
    assert fa.fa_decode_workspace_bytes(B, Nq, Nk, H, d) > 32 << 20
    q = torch.zeros((B, Nq, H, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Nk, H, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_decode_noalloc(q, k, k, True)
    assert e.value.status == FA_ERR_SCRATCH
