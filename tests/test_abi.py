"""Host-side tests of the C ABI (no GPU needed).

Every call here fails argument validation, which the library performs before
it touches the device, so no kernel is ever launched and fake non-null
pointers are never dereferenced.
"""

import ctypes
import os
import re

import pytest

import exact_tiled_attention_37_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEADDIM, FA_ERR_ALIGN = 0, 1, 2, 3, 4
FA_ERR_SCALE, FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_DEVICE = 5, 6, 7, 8

P = 0x10000  # a fake, 256-byte aligned device address; never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"FA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.lib_path()):
        pytest.fail("libfa_mi355x.so is not built: run `python -m exact_tiled_attention_37_amd.build`")
    return fa.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    assert sorted(names) == sorted(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(fa.lib_path())
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} is declared in fa.h but not exported"


def test_status_strings_and_version(lib):
    for st in range(9):
        s = fa.fa_status_string(st)
        assert isinstance(s, str) and s
    assert fa.fa_status_string(FA_OK) == "ok"
    assert fa.fa_status_string(1234) == "unknown status"
    assert fa.fa_version() == 100


def test_workspace_bytes(lib):
    pad = lambda x: (x + 255) // 256 * 256
    assert fa.fa_bwd_workspace_bytes(4, 4096, 16, 128) == 2 * pad(4 * 16 * 4096 * 4)
    assert fa.fa_bwd_workspace_bytes(1, 3, 1, 64) == 2 * pad(3 * 4)
    assert fa.fa_bwd_workspace_bytes(1, 3, 1, 96) == 0
    assert fa.fa_bwd_workspace_bytes(0, 3, 1, 64) == 0
    assert fa.fa_bwd_workspace_bytes(1 << 14, 1 << 14, 16, 128) == 0  # > 2^31 elements


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, N=8, H=2, d=64, causal=0, scale=0.125):
    return lib.fa_fwd(q, k, v, o, lse, B, N, H, d, causal, scale, None)


def bwd(lib, ws_bytes=1 << 20, ws=P, B=1, N=8, H=2, d=64, scale=0.125, **ptrs):
    p = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P)
    p.update(ptrs)
    return lib.fa_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                      ws, ws_bytes, B, N, H, d, 0, scale, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_fwd_null_pointer(lib, which):
    assert fwd(lib, **{which: None}) == FA_ERR_NULL


@pytest.mark.parametrize("d", [0, 32, 80, 96, 256])
def test_fwd_head_dim(lib, d):
    assert fwd(lib, d=d) == FA_ERR_HEADDIM


@pytest.mark.parametrize("B,N,H", [(0, 8, 2), (1, 0, 2), (1, 8, 0), (-1, 8, 2), (4096, 65536, 16)])
def test_fwd_shape(lib, B, N, H):
    assert fwd(lib, B=B, N=N, H=H) == FA_ERR_SHAPE


@pytest.mark.parametrize("scale", [float("inf"), float("-inf"), float("nan")])
def test_fwd_scale(lib, scale):
    assert fwd(lib, scale=scale) == FA_ERR_SCALE


@pytest.mark.parametrize("which,addr", [("q", P + 8), ("k", P + 2), ("v", P + 4), ("o", P + 1), ("lse", P + 2)])
def test_fwd_alignment(lib, which, addr):
    assert fwd(lib, **{which: addr}) == FA_ERR_ALIGN


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"])
def test_bwd_null_pointer(lib, which):
    assert bwd(lib, **{which: None}) == FA_ERR_NULL


def test_bwd_workspace(lib):
    need = fa.fa_bwd_workspace_bytes(1, 8, 2, 64)
    assert bwd(lib, ws_bytes=need - 1) == FA_ERR_WORKSPACE
    assert bwd(lib, ws=None) == FA_ERR_WORKSPACE
    assert bwd(lib, ws=P + 128, ws_bytes=need) == FA_ERR_ALIGN


def test_bwd_shape_headdim_scale(lib):
    assert bwd(lib, d=96) == FA_ERR_HEADDIM
    assert bwd(lib, N=0) == FA_ERR_SHAPE
    assert bwd(lib, scale=float("nan")) == FA_ERR_SCALE


@pytest.mark.parametrize("which", ["q", "do", "dq", "dk", "dv"])
def test_bwd_alignment(lib, which):
    assert bwd(lib, **{which: P + 8}) == FA_ERR_ALIGN


def test_binding_rejects_wrong_tensors(lib):
    import torch

    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # host tensor
        fa.fa_fwd(q, q, q, causal=False)
    with pytest.raises(TypeError):
        fa.fa_fwd(q.float(), q, q, causal=False)
    with pytest.raises(ValueError):
        fa.fa_fwd(q[0], q, q, causal=False)


def chunk(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Nq=8, Nk=8, H=2, d=64, causal=1, qs=0, ks=0, scale=0.125):
    return lib.fa_fwd_chunk(q, k, v, o, lse, B, Nq, Nk, H, d, causal, qs, ks, scale, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_chunk_null_pointer(lib, which):
    assert chunk(lib, **{which: None}) == FA_ERR_NULL


@pytest.mark.parametrize("B,Nq,Nk,H", [(0, 8, 8, 2), (1, 0, 8, 2), (1, 8, -1, 2), (1, 8, 8, 0),
                                       (4096, 65536, 8, 16), (1, 8, 1 << 28, 16)])
def test_chunk_shape(lib, B, Nq, Nk, H):
    assert chunk(lib, B=B, Nq=Nq, Nk=Nk, H=H) == FA_ERR_SHAPE


def test_chunk_headdim_scale_alignment(lib):
    assert chunk(lib, d=96) == FA_ERR_HEADDIM
    assert chunk(lib, scale=float("nan")) == FA_ERR_SCALE
    assert chunk(lib, o=P + 8) == FA_ERR_ALIGN  # float32 rows still need 16 bytes
    assert chunk(lib, lse=P + 2) == FA_ERR_ALIGN


def merge(lib, op=P, lp=P, C=3, o=P, lse=P, B=1, N=8, H=2, d=64):
    return lib.fa_merge(op, lp, C, o, lse, B, N, H, d, None)


@pytest.mark.parametrize("which", ["op", "lp", "o", "lse"])
def test_merge_null_pointer(lib, which):
    assert merge(lib, **{which: None}) == FA_ERR_NULL


@pytest.mark.parametrize("C,B,N,H", [(0, 1, 8, 2), (65537, 1, 8, 2), (3, 0, 8, 2), (3, 1, 0, 2), (3, 1, 8, 0)])
def test_merge_shape(lib, C, B, N, H):
    assert merge(lib, C=C, B=B, N=N, H=H) == FA_ERR_SHAPE


def test_merge_headdim_alignment(lib):
    assert merge(lib, d=32) == FA_ERR_HEADDIM
    assert merge(lib, op=P + 4) == FA_ERR_ALIGN
    assert merge(lib, o=P + 8) == FA_ERR_ALIGN
    assert merge(lib, lp=P + 1) == FA_ERR_ALIGN


def test_binding_rejects_wrong_chunk_tensors(lib):
    import torch

    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # host tensors
        fa.fa_fwd_chunk(q, q, q, causal=True)
    with pytest.raises(ValueError):
        fa.fa_merge(torch.zeros(2, 1, 8, 2, 64), torch.zeros(2, 1, 2, 8))


def _decode_split(B, Nq, Nk, H, d):
    """The library's key split for decode calls (mirrors its documented rule:
    about 2048 workgroups at d = 128 and 4096 at d = 64, ranges of at least
    256 keys, 32-key tiles)."""
    bc = 32
    nqb = (Nq + 31) // 32
    tiles = (Nk + bc - 1) // bc
    target = 4096 if d == 64 else 2048
    s = (target + B * H * nqb - 1) // (B * H * nqb)
    s = max(1, min(s, (Nk + 255) // 256, tiles))
    ln = (tiles + s - 1) // s * bc
    return (Nk + ln - 1) // ln, ln


@pytest.mark.parametrize("B,Nq,Nk,H,d", [(16, 1, 8192, 16, 128), (4, 16, 16384, 16, 128), (1, 1, 100, 1, 64),
                                         (2, 40, 1000, 3, 64), (1, 5, 300, 2, 128)])
def test_decode_workspace_bytes(lib, B, Nq, Nk, H, d):
    ns, _ = _decode_split(B, Nq, Nk, H, d)
    pad = lambda elems: (elems + 63) // 64 * 64
    rows = B * Nq * H
    want = 0 if ns == 1 else (pad(ns * rows * d) + pad(ns * rows)) * 4
    assert fa.fa_decode_workspace_bytes(B, Nq, Nk, H, d) == want
    assert fa.fa_decode_workspace_bytes(B, Nq, Nk, H, 96) == 0


def decode(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Nq=4, Nk=4096, H=2, d=64, causal=1, scale=0.125, ws=P,
           ws_bytes=1 << 24):
    return lib.fa_decode(q, k, v, o, lse, B, Nq, Nk, H, d, causal, scale, ws, ws_bytes, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_decode_null_pointer(lib, which):
    assert decode(lib, **{which: None}) == FA_ERR_NULL


def test_decode_errors(lib):
    assert decode(lib, d=80) == FA_ERR_HEADDIM
    assert decode(lib, Nq=0) == FA_ERR_SHAPE
    assert decode(lib, Nk=0) == FA_ERR_SHAPE
    assert decode(lib, scale=float("inf")) == FA_ERR_SCALE
    need = fa.fa_decode_workspace_bytes(1, 4, 4096, 2, 64)
    assert need > 0
    assert decode(lib, ws=None) == FA_ERR_WORKSPACE
    assert decode(lib, ws_bytes=need - 1) == FA_ERR_WORKSPACE
    assert decode(lib, ws=P + 64, ws_bytes=need) == FA_ERR_ALIGN
    assert decode(lib, q=P + 2) == FA_ERR_ALIGN


def fwdb(lib, q=P, k=P, v=P, bias=P, sb=0, sh=0, sr=16, o=P, lse=P, B=1, N=9, H=2, d=64, causal=0, scale=0.125):
    return lib.fa_fwd_bias(q, k, v, bias, sb, sh, sr, o, lse, B, N, H, d, causal, scale, None)


def bwdb(lib, dbias=P, dsr=16, ws=P, ws_bytes=1 << 20, sr=16, sb=0, sh=0, B=1, N=9, H=2, d=64, **ptrs):
    p = dict(q=P, k=P, v=P, bias=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P)
    p.update(ptrs)
    return lib.fa_bwd_bias(p["q"], p["k"], p["v"], p["bias"], sb, sh, sr, p["o"], p["lse"], p["do"], p["dq"],
                           p["dk"], p["dv"], dbias, dsr, ws, ws_bytes, B, N, H, d, 0, 0.125, None)


def test_bias_validation(lib):
    assert fwdb(lib, bias=None) == FA_ERR_NULL
    assert fwdb(lib, sr=8) == FA_ERR_SHAPE          # row stride below N
    assert fwdb(lib, sr=12) == FA_ERR_SHAPE         # not a multiple of 8
    assert fwdb(lib, sb=-8) == FA_ERR_SHAPE
    assert fwdb(lib, sh=4) == FA_ERR_SHAPE
    assert fwdb(lib, bias=P + 8) == FA_ERR_ALIGN
    assert fwdb(lib, N=70000, sr=70000) == FA_ERR_SHAPE  # slice beyond 32-bit byte offsets
    assert fwdb(lib, d=96) == FA_ERR_HEADDIM
    assert bwdb(lib, bias=None) == FA_ERR_NULL
    assert bwdb(lib, dsr=12) == FA_ERR_SHAPE
    assert bwdb(lib, dbias=P + 8) == FA_ERR_ALIGN
    assert bwdb(lib, ws=None) == FA_ERR_WORKSPACE
    assert bwdb(lib, dq=None) == FA_ERR_NULL


def test_binding_bias_layout(lib):
    import torch

    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd_bias(q, q, q, torch.zeros(1, 2, 8, 8, dtype=torch.bfloat16), causal=False)
    pb = fa.padded_bias(2, 3, 13)
    assert tuple(pb.shape) == (2, 3, 13, 13) and pb.stride(2) == 16 and pb.stride(3) == 1


def fp8(lib, q=P, k=P, v=P, qd=P, kd=P, vd=P, o=P, lse=P, B=1, N=9, H=2, d=128, causal=1, scale=0.1):
    return lib.fa_fwd_fp8(q, k, v, qd, kd, vd, o, lse, B, N, H, d, causal, scale, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "qd", "kd", "vd", "o", "lse"])
def test_fp8_null_pointer(lib, which):
    assert fp8(lib, **{which: None}) == FA_ERR_NULL


def test_fp8_errors(lib):
    assert fp8(lib, d=96) == FA_ERR_HEADDIM
    assert fp8(lib, d=256) == FA_ERR_HEADDIM
    assert fp8(lib, N=0) == FA_ERR_SHAPE
    assert fp8(lib, scale=float("nan")) == FA_ERR_SCALE
    assert fp8(lib, q=P + 8) == FA_ERR_ALIGN
    assert fp8(lib, kd=P + 2) == FA_ERR_ALIGN


def mxfp8(lib, q=P, qs=P, k=P, ks=P, v=P, vs=P, o=P, lse=P, B=1, N=9, H=2, d=128, causal=1, scale=0.1):
    return lib.fa_fwd_mxfp8(q, qs, k, ks, v, vs, o, lse, B, N, H, d, causal, scale, None)


@pytest.mark.parametrize("which", ["q", "qs", "k", "ks", "v", "vs", "o", "lse"])
def test_mxfp8_null_pointer(lib, which):
    assert mxfp8(lib, **{which: None}) == FA_ERR_NULL


def test_mxfp8_errors(lib):
    assert mxfp8(lib, d=32) == FA_ERR_HEADDIM
    assert mxfp8(lib, d=96) == FA_ERR_HEADDIM
    assert mxfp8(lib, N=0) == FA_ERR_SHAPE
    assert mxfp8(lib, H=0) == FA_ERR_SHAPE
    assert mxfp8(lib, scale=float("inf")) == FA_ERR_SCALE
    assert mxfp8(lib, v=P + 8) == FA_ERR_ALIGN
    assert mxfp8(lib, vs=P + 2) == FA_ERR_ALIGN
    assert mxfp8(lib, lse=P + 2) == FA_ERR_ALIGN


def test_binding_mxfp8_scale_shapes():
    """The binding checks the block-scale shapes before anything reaches the
    library (host tensors never get that far either)."""
    import torch

    q = torch.zeros(1, 40, 2, 128, dtype=torch.uint8)
    qs = torch.zeros(1, 40, 2, 4, dtype=torch.uint8)
    vs = torch.zeros(1, 2, 2, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):
        fa.fa_fwd_mxfp8(q, qs, q, qs, q, vs, causal=True)  # host tensors
    if torch.cuda.is_available():  # pragma: no cover - GPU machine only
        return
    assert fa.fa_fwd_mxfp8.__doc__ and "E8M0" in fa.fa_fwd_mxfp8.__doc__


def test_binding_rejects_host_or_mistyped_workspace():
    """A caller-supplied workspace must be a contiguous uint8 tensor on the
    calling device with enough bytes; a host tensor (whose pointer the
    kernels would write through) is refused before anything is launched."""
    import torch

    dev = torch.device("cuda", 0)
    with pytest.raises(ValueError, match="workspace"):
        fa._check_workspace(torch.empty(1024, dtype=torch.uint8), 512, dev)  # host memory
    with pytest.raises(ValueError, match="workspace"):
        fa._check_workspace(torch.empty(1024, dtype=torch.float32), 512, dev)  # not bytes


def test_decode_noalloc_validation(lib):
    """Checks before any device work: the usual argument errors, and
    FA_ERR_SCRATCH for a call whose key-split partials exceed the 32 MiB
    static scratch (fa_decode with a workspace takes such calls)."""
    f = lib.fa_decode_noalloc
    assert f(None, P, P, P, P, 1, 1, 10, 1, 64, 1, 0.1, None) == FA_ERR_NULL
    assert f(P, P, P, P, P, 1, 1, 10, 1, 96, 1, 0.1, None) == FA_ERR_HEADDIM
    assert f(P, P, P, P, P, 1, 1, 0, 1, 64, 1, 0.1, None) == FA_ERR_SHAPE
    assert f(P, P, P, P, P, 1, 1, 10, 1, 64, 1, float("nan"), None) == FA_ERR_SCALE
    assert f(P + 2, P, P, P, P, 1, 1, 10, 1, 64, 1, 0.1, None) == FA_ERR_ALIGN
    B, Nq, Nk, H, d = 1, 32, 218560, 3, 128
    assert fa.fa_decode_workspace_bytes(B, Nq, Nk, H, d) > 32 << 20
    assert f(P, P, P, P, P, B, Nq, Nk, H, d, 1, 0.1, None) == 9
    assert fa.fa_status_string(9).startswith("the call needs more scratch")
