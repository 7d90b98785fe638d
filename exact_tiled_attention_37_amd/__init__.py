"""Exact tiled attention for MI355X (gfx950): thin Python binding.

The binding only marshals arguments. Every step of the computation runs in
the HIP kernels of libfa_mi355x.so, reached through the C ABI declared in
include/fa.h; PyTorch is used only to own device memory and streams. There
is no fallback: if the library is missing or cannot be loaded, every call
raises.

Tensors use the library's layouts: q, k, v, o, do, dq, dk, dv are
torch.bfloat16 [B, N, H, d] contiguous CUDA (HIP) tensors; lse is
torch.float32 [B, H, N]. Chunk outputs (fa_fwd_chunk) are torch.float32
[B, Nq, H, d]; fa_merge takes C of them stacked as [C, B, N, H, d].
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = [
    "FaError",
    "lib_path",
    "load_library",
    "fa_fwd",
    "fa_bwd",
    "fa_bwd_workspace_bytes",
    "fa_fwd_chunk",
    "fa_merge",
    "fa_decode",
    "fa_decode_workspace_bytes",
    "fa_decode_noalloc",
    "fa_fwd_bias",
    "fa_bwd_bias",
    "fa_fwd_fp8",
    "fa_fwd_mxfp8",
    "fa_status_string",
    "fa_version",
    "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfa_mi355x.so"
EXPORTED_SYMBOLS = ("fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd_chunk", "fa_merge", "fa_decode",
                    "fa_decode_workspace_bytes", "fa_decode_noalloc", "fa_fwd_bias", "fa_bwd_bias", "fa_fwd_fp8",
                    "fa_fwd_mxfp8", "fa_status_string", "fa_version")

_lib = None


class FaError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")


def lib_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load_library():
    """Load libfa_mi355x.so (built by exact_tiled_attention_37_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_tiled_attention_37_amd.build` "
            "(there is no non-HIP fallback)"
        )
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, vp]
    lib.fa_bwd.restype = i
    ll = ctypes.c_longlong
    lib.fa_fwd_chunk.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, ll, ll, f, vp]
    lib.fa_fwd_chunk.restype = i
    lib.fa_merge.argtypes = [vp, vp, i, vp, vp, i, i, i, i, vp]
    lib.fa_merge.restype = i
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    lib.fa_decode.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_decode_noalloc.restype = i
    lib.fa_fwd_bias.argtypes = [vp, vp, vp, vp, ll, ll, i, vp, vp, i, i, i, i, i, f, vp]
    lib.fa_fwd_bias.restype = i
    lib.fa_bwd_bias.argtypes = [vp, vp, vp, vp, ll, ll, i, vp, vp, vp, vp, vp, vp, vp, i, vp, sz, i, i, i, i, i, f, vp]
    lib.fa_bwd_bias.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_fwd_mxfp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.fa_fwd_mxfp8.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_version() -> int:
    return int(load_library().fa_version())


def fa_bwd_workspace_bytes(B: int, N: int, H: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, N, H, d))


def _check_bnhd(name, t, shape=None):
    import torch

    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be torch.bfloat16, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, N, H, d], got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_lse(t, B, N, H):
    import torch

    if t.dtype != torch.float32 or tuple(t.shape) != (B, H, N) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 device tensor of shape {(B, H, N)}")


def _check_workspace(ws, need: int, device):
    """A caller-supplied workspace: a contiguous uint8 device tensor on
    `device` with at least `need` bytes (the kernels write through its
    pointer, so a host tensor would fault the GPU)."""
    import torch

    if ws.dtype != torch.uint8 or not ws.is_cuda or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {device}")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} are needed")


def _stream_handle(device) -> int:
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def fa_fwd(q, k, v, causal: bool, softmax_scale: Optional[float] = None, out=None, lse=None):
    """Forward pass on the current stream of q's device. Returns (o, lse)."""
    import torch

    _check_bnhd("q", q)
    B, N, H, d = q.shape
    _check_bnhd("k", k, q.shape)
    _check_bnhd("v", v, q.shape)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _check_bnhd("out", out, q.shape)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_lse(lse, B, N, H)
    st = load_library().fa_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
        B, N, H, d, int(bool(causal)), scale, _stream_handle(q.device),
    )
    if st != 0:
        raise FaError(st, "fa_fwd")
    return out, lse


def fa_bwd(q, k, v, o, lse, do, causal: bool, softmax_scale: Optional[float] = None,
           dq=None, dk=None, dv=None, workspace=None) -> Tuple:
    """Backward pass on the current stream of q's device. Returns (dq, dk, dv)."""
    import torch

    _check_bnhd("q", q)
    B, N, H, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _check_bnhd(name, t, q.shape)
    _check_lse(lse, B, N, H)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_bnhd(name, t, q.shape)
    need = fa_bwd_workspace_bytes(B, N, H, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    st = load_library().fa_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
        B, N, H, d, int(bool(causal)), scale, _stream_handle(q.device),
    )
    if st != 0:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def fa_fwd_chunk(q, k, v, causal: bool, q_start: int = 0, k_start: int = 0,
                 softmax_scale: Optional[float] = None, out=None, lse=None):
    """Attention of the query chunk q (rows at global positions q_start..)
    over the key chunk k, v (positions k_start..). Returns (o float32
    [B, Nq, H, d], lse float32 [B, H, Nq]); rows that see no key get o = 0
    and lse = -inf."""
    import torch

    _check_bnhd("q", q)
    B, Nq, H, d = q.shape
    _check_bnhd("k", k)
    Nk = k.shape[1]
    if k.shape[0] != B or tuple(k.shape[2:]) != (H, d):
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [{B}, Nk, {H}, {d}]")
    _check_bnhd("v", v, k.shape)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, Nq, H, d), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, Nq, H, d) or not out.is_cuda or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous float32 device tensor of shape {(B, Nq, H, d)}")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_lse(lse, B, Nq, H)
    kp = k.data_ptr() if Nk > 0 else q.data_ptr()  # an empty chunk is not read
    vp = v.data_ptr() if Nk > 0 else q.data_ptr()
    st = load_library().fa_fwd_chunk(
        q.data_ptr(), kp, vp, out.data_ptr(), lse.data_ptr(), B, Nq, Nk, H, d, int(bool(causal)),
        int(q_start), int(k_start), scale, _stream_handle(q.device),
    )
    if st != 0:
        raise FaError(st, "fa_fwd_chunk")
    return out, lse


def fa_merge(o_parts, lse_parts, out=None, lse=None):
    """Combine C chunk results (o_parts float32 [C, B, N, H, d], lse_parts
    float32 [C, B, H, N]) into (o bf16 [B, N, H, d], lse float32 [B, H, N])."""
    import torch

    if o_parts.dtype != torch.float32 or o_parts.dim() != 5 or not o_parts.is_cuda or not o_parts.is_contiguous():
        raise ValueError("o_parts must be a contiguous float32 device tensor [C, B, N, H, d]")
    C, B, N, H, d = o_parts.shape
    if (lse_parts.dtype != torch.float32 or tuple(lse_parts.shape) != (C, B, H, N) or not lse_parts.is_cuda
            or not lse_parts.is_contiguous()):
        raise ValueError(f"lse_parts must be a contiguous float32 device tensor of shape {(C, B, H, N)}")
    if out is None:
        out = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=o_parts.device)
    _check_bnhd("out", out, (B, N, H, d))
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    _check_lse(lse, B, N, H)
    st = load_library().fa_merge(
        o_parts.data_ptr(), lse_parts.data_ptr(), C, out.data_ptr(), lse.data_ptr(), B, N, H, d,
        _stream_handle(o_parts.device),
    )
    if st != 0:
        raise FaError(st, "fa_merge")
    return out, lse


def fa_decode_workspace_bytes(B: int, Nq: int, Nk: int, H: int, d: int) -> int:
    return int(load_library().fa_decode_workspace_bytes(B, Nq, Nk, H, d))


def fa_decode(q, k, v, causal: bool, softmax_scale: Optional[float] = None, out=None, lse=None,
              workspace=None):
    """Decode-shaped attention: q [B, Nq, H, d] holds the last Nq positions
    of the sequence whose keys and values are k, v [B, Nk, H, d]. Returns
    (o bf16 [B, Nq, H, d], lse float32 [B, H, Nq])."""
    import torch

    _check_bnhd("q", q)
    B, Nq, H, d = q.shape
    _check_bnhd("k", k)
    Nk = k.shape[1]
    if k.shape[0] != B or tuple(k.shape[2:]) != (H, d):
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [{B}, Nk, {H}, {d}]")
    _check_bnhd("v", v, k.shape)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _check_bnhd("out", out, q.shape)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_lse(lse, B, Nq, H)
    need = fa_decode_workspace_bytes(B, Nq, Nk, H, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check_workspace(workspace, need, q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().fa_decode(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Nq, Nk, H, d,
        int(bool(causal)), scale, ws_ptr, ws_len, _stream_handle(q.device),
    )
    if st != 0:
        raise FaError(st, "fa_decode")
    return out, lse


def fa_decode_noalloc(q, k, v, causal: bool, softmax_scale: Optional[float] = None, out=None, lse=None):
    """fa_decode without a workspace: the library keeps the key-split partial
    results in its own static device scratch (32 MiB per device), so the call
    allocates nothing when out and lse are given. Calls that may overlap on
    one device must not be issued (they share that scratch). Returns
    (o bf16 [B, Nq, H, d], lse float32 [B, H, Nq])."""
    import torch

    _check_bnhd("q", q)
    B, Nq, H, d = q.shape
    _check_bnhd("k", k)
    Nk = k.shape[1]
    if k.shape[0] != B or tuple(k.shape[2:]) != (H, d):
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [{B}, Nk, {H}, {d}]")
    _check_bnhd("v", v, k.shape)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _check_bnhd("out", out, q.shape)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_lse(lse, B, Nq, H)
    st = load_library().fa_decode_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Nq, Nk, H, d,
        int(bool(causal)), scale, _stream_handle(q.device),
    )
    if st != 0:
        raise FaError(st, "fa_decode_noalloc")
    return out, lse


def _bias_layout(bias, B, N, H):
    """(pointer, stride_b, stride_h, stride_row) of a bf16 bias tensor viewed
    as [B or 1, H or 1, N, >= N] (a size-1 batch or head dimension is
    broadcast); the last dimension must be contiguous."""
    import torch

    if bias.dtype != torch.bfloat16 or not bias.is_cuda or bias.dim() != 4:
        raise ValueError("bias must be a bfloat16 device tensor [B or 1, H or 1, N, N]")
    if bias.shape[2] != N or bias.shape[3] != N or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, H):
        raise ValueError(f"bias has shape {tuple(bias.shape)}, expected [{B} or 1, {H} or 1, {N}, {N}]")
    if bias.stride(3) != 1:
        raise ValueError("bias rows must be contiguous")
    sb = 0 if bias.shape[0] == 1 else bias.stride(0)
    sh = 0 if bias.shape[1] == 1 else bias.stride(1)
    return bias.data_ptr(), sb, sh, bias.stride(2)


def padded_bias(B: int, H: int, N: int, device=None):
    """An empty bf16 bias [B, H, N, N] whose rows are padded to a multiple of
    8 elements (a view of [B, H, N, ceil8(N)] storage), as the biased entry
    points require."""
    import torch

    n8 = (N + 7) // 8 * 8
    return torch.empty((B, H, N, n8), dtype=torch.bfloat16, device=device)[..., :N]


def fa_fwd_bias(q, k, v, bias, causal: bool, softmax_scale: Optional[float] = None, out=None, lse=None):
    """Forward with an additive bf16 bias on the scaled scores. Returns (o, lse)."""
    import torch

    _check_bnhd("q", q)
    B, N, H, d = q.shape
    _check_bnhd("k", k, q.shape)
    _check_bnhd("v", v, q.shape)
    bp, sb, sh, sr = _bias_layout(bias, B, N, H)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _check_bnhd("out", out, q.shape)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_lse(lse, B, N, H)
    st = load_library().fa_fwd_bias(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), bp, sb, sh, sr, out.data_ptr(), lse.data_ptr(),
        B, N, H, d, int(bool(causal)), scale, _stream_handle(q.device),
    )
    if st != 0:
        raise FaError(st, "fa_fwd_bias")
    return out, lse


def fa_bwd_bias(q, k, v, bias, o, lse, do, causal: bool, softmax_scale: Optional[float] = None,
                dq=None, dk=None, dv=None, dbias=None, want_dbias: bool = True, workspace=None):
    """Backward of fa_fwd_bias. Returns (dq, dk, dv, dbias); dbias is a bf16
    [B, H, N, N] view with rows padded to a multiple of 8 (None when
    want_dbias is False and no dbias is given)."""
    import torch

    _check_bnhd("q", q)
    B, N, H, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _check_bnhd(name, t, q.shape)
    _check_lse(lse, B, N, H)
    bp, sb, sh, sr = _bias_layout(bias, B, N, H)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_bnhd(name, t, q.shape)
    if dbias is None and want_dbias:
        dbias = padded_bias(B, H, N, q.device)
    if dbias is not None:
        if (dbias.dtype != torch.bfloat16 or tuple(dbias.shape) != (B, H, N, N) or dbias.stride(3) != 1
                or dbias.stride(1) != N * dbias.stride(2) or dbias.stride(0) != H * N * dbias.stride(2)):
            raise ValueError("dbias must be a bf16 [B, H, N, N] view with unit key stride and packed rows")
        if not dbias.is_cuda or dbias.device != q.device:
            raise ValueError(f"dbias must be a device tensor on {q.device}")
    need = fa_bwd_workspace_bytes(B, N, H, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    st = load_library().fa_bwd_bias(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), bp, sb, sh, sr, o.data_ptr(), lse.data_ptr(), do.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dbias.data_ptr() if dbias is not None else None,
        dbias.stride(2) if dbias is not None else 0, workspace.data_ptr(), workspace.numel(),
        B, N, H, d, int(bool(causal)), scale, _stream_handle(q.device),
    )
    if st != 0:
        raise FaError(st, "fa_bwd_bias")
    return dq, dk, dv, dbias


def fa_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, causal: bool, softmax_scale: Optional[float] = None,
               out=None, lse=None):
    """FP8 forward: q8, k8, v8 are uint8 e4m3 codes [B, N, H, d] (d = 64 or
    128) and the descales float32 [B, H]. Returns (o bf16 [B, N, H, d], lse
    float32 [B, H, N])."""
    import torch

    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        if t.dtype != torch.uint8 or t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 device tensor [B, N, H, d]")
        if tuple(t.shape) != tuple(q8.shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(q8.shape)}")
    B, N, H, d = q8.shape
    for name, t in (("q_descale", q_descale), ("k_descale", k_descale), ("v_descale", v_descale)):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 device tensor of shape {(B, H)}")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=q8.device)
    _check_bnhd("out", out, (B, N, H, d))
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    _check_lse(lse, B, N, H)
    st = load_library().fa_fwd_fp8(
        q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_descale.data_ptr(), k_descale.data_ptr(),
        v_descale.data_ptr(), out.data_ptr(), lse.data_ptr(), B, N, H, d, int(bool(causal)), scale,
        _stream_handle(q8.device),
    )
    if st != 0:
        raise FaError(st, "fa_fwd_fp8")
    return out, lse


def fa_fwd_mxfp8(q8, q_scale, k8, k_scale, v8, v_scale, causal: bool, softmax_scale: Optional[float] = None,
                 out=None, lse=None):
    """Microscaled FP8 forward: q8, k8, v8 are uint8 e4m3 codes [B, N, H, d]
    (d = 64 or 128); q_scale, k_scale uint8 E8M0 [B, N, H, d / 32] (one per 32
    consecutive d of a token); v_scale uint8 E8M0 [B, ceil(N / 32), H, d] (one
    per 32 consecutive tokens of a column). Returns (o bf16 [B, N, H, d], lse
    float32 [B, H, N])."""
    import torch

    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        if t.dtype != torch.uint8 or t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 device tensor [B, N, H, d]")
        if tuple(t.shape) != tuple(q8.shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(q8.shape)}")
    B, N, H, d = q8.shape
    shapes = {"q_scale": (B, N, H, d // 32), "k_scale": (B, N, H, d // 32), "v_scale": (B, (N + 31) // 32, H, d)}
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        if t.dtype != torch.uint8 or tuple(t.shape) != shapes[name] or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 device tensor of shape {shapes[name]}")
        if t.device != q8.device:
            raise ValueError(f"{name} is on {t.device}, expected {q8.device}")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=q8.device)
    _check_bnhd("out", out, (B, N, H, d))
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    _check_lse(lse, B, N, H)
    st = load_library().fa_fwd_mxfp8(
        q8.data_ptr(), q_scale.data_ptr(), k8.data_ptr(), k_scale.data_ptr(), v8.data_ptr(), v_scale.data_ptr(),
        out.data_ptr(), lse.data_ptr(), B, N, H, d, int(bool(causal)), scale, _stream_handle(q8.device),
    )
    if st != 0:
        raise FaError(st, "fa_fwd_mxfp8")
    return out, lse
