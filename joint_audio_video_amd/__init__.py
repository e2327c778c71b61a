"""joint_audio_video_amd: one block of the joint audio-video DiT on MI355X.

Thin ctypes binding over ``libdit.so`` (the C ABI declared in
``include/dit.h``).  This module only marshals arguments: every step of the
block runs in the library's HIP kernels.  PyTorch supplies device memory and
the current HIP stream.  If the library is missing this module raises at
import; there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np
# torch first: libdit binds to the HIP runtime torch has already loaded (one
# HIP/HSA runtime per process), see build.py.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdit.so")

DIT_OK, DIT_EINVAL, DIT_EUNSUPPORTED, DIT_EWORKSPACE, DIT_EHIP = range(5)
DIT_F32, DIT_BF16 = 0, 1
MOD_VIDEO, MOD_AUDIO, MOD_TEXT = 0, 1, 2
STAGES = ("adaln", "qkv", "rope", "attn", "out")

_STATUS_NAMES = {1: "DIT_EINVAL", 2: "DIT_EUNSUPPORTED", 3: "DIT_EWORKSPACE", 4: "DIT_EHIP"}

EXPORTED = (
    "dit_abi_version", "dit_last_error", "dit_grid_from_media", "dit_pack_layout",
    "dit_pack_count", "dit_block_intermediates",
    "adaln_modulate", "rope3d_apply", "attn_packed", "qkv_project", "out_proj_gated",
    "dit_block_workspace_bytes", "dit_block_forward", "dit_profile_enable", "dit_profile_read",
    "ffn_up_gelu", "ffn_down_gated", "dit_ffn_workspace_bytes", "dit_ffn_forward",
    "denoise_step", "dit_nft_workspace_bytes", "nft_loss", "rope3d_apply_to",
    "quantize_rows_fp8", "linear_fp8", "adaln_modulate_fp8", "dit_block_fp8_workspace_bytes",
    "dit_block_forward_fp8", "dit_ffn_fp8_workspace_bytes", "dit_ffn_forward_fp8",
    "attn_packed_lse", "dit_attn_backward_workspace_bytes", "attn_packed_backward",
    "dit_block_backward_workspace_bytes", "dit_block_backward",
    "dit_ffn_backward_workspace_bytes", "dit_ffn_backward",
    "dit_attn_fp8_workspace_bytes", "dit_attn_fp8_layout", "attn_fp8_prepare", "attn_packed_fp8",
    "dit_block_fp8_attn_workspace_bytes", "dit_block_forward_fp8_attn",
    "dit_attn_backward_noalloc_max_elements", "attn_packed_backward_noalloc",
)


class DitError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class _Media(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("height_px", ctypes.c_int32),
                ("width_px", ctypes.c_int32), ("audio_samples_per_ch", ctypes.c_int64),
                ("text_len", ctypes.c_int32)]


class _Grid(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32),
                ("audio_per_ch", ctypes.c_int32), ("text_len", ctypes.c_int32)]


class BlockDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("d_model", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_sections", ctypes.c_int32 * 3), ("rope_theta", ctypes.c_float),
                ("ln_eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
                ("causal", ctypes.c_int32)]


class FfnDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("ln_eps", ctypes.c_float)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python joint_audio_video_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    sig = {
        "dit_abi_version": (ctypes.c_int, []),
        "dit_last_error": (ctypes.c_char_p, []),
        "dit_grid_from_media": (ctypes.c_int, [ctypes.POINTER(_Media), ctypes.POINTER(_Grid)]),
        "dit_pack_layout": (ctypes.c_int, [ctypes.POINTER(_Grid), I32, P, P, P, I64,
                                           ctypes.POINTER(I64), ctypes.POINTER(I32)]),
        "dit_pack_count": (ctypes.c_int, [ctypes.POINTER(_Grid), I32, ctypes.POINTER(I64),
                                          ctypes.POINTER(I32)]),
        "adaln_modulate": (ctypes.c_int, [ctypes.c_int, P, I64, P, P, P, I64, I64, I32, F32, P]),
        "rope3d_apply": (ctypes.c_int, [ctypes.c_int, P, I64, P, I64, P, I64, I32, I32,
                                        ctypes.POINTER(I32), F32, P]),
        "rope3d_apply_to": (ctypes.c_int, [ctypes.c_int, P, I64, P, I64, P, I64, P, I64, P, I64,
                                           I32, I32, ctypes.POINTER(I32), F32, P]),
        "attn_packed": (ctypes.c_int, [ctypes.c_int, P, I64, P, I64, P, I64, P, I64, P, I32, I32,
                                       I64, I32, I32, F32, I32, P]),
        "qkv_project": (ctypes.c_int, [ctypes.c_int, P, I64, P, P, P, I64, I64, I32, P]),
        "out_proj_gated": (ctypes.c_int, [ctypes.c_int, P, I64, P, P, P, I64, P, P, P, I64, I64,
                                          I32, P]),
        "dit_block_workspace_bytes": (SZ, [ctypes.POINTER(BlockDesc), I64]),
        "dit_block_intermediates": (ctypes.c_int, [ctypes.POINTER(BlockDesc), I64,
                                                   ctypes.POINTER(I64)]),
        "dit_block_forward": (ctypes.c_int, [ctypes.POINTER(BlockDesc), P, P, P, P, P, I32, I32,
                                             I64, P, P, P, P, P, P, SZ, P]),
        "ffn_up_gelu": (ctypes.c_int, [ctypes.c_int, P, I64, P, P, P, I64, I64, I32, I32, P]),
        "ffn_down_gated": (ctypes.c_int, [ctypes.c_int, P, I64, P, P, P, I64, P, P, P, I64, I64,
                                          I32, I32, P]),
        "dit_ffn_workspace_bytes": (SZ, [ctypes.POINTER(FfnDesc), I64]),
        "dit_ffn_forward": (ctypes.c_int, [ctypes.POINTER(FfnDesc), P, P, P, I64, P, P, P, P, P,
                                           P, SZ, P]),
        "denoise_step": (ctypes.c_int, [ctypes.c_int, P, I64, P, I64, P, I64, P, P, P, I64, I64,
                                        I32, ctypes.POINTER(F32), I32, P]),
        "dit_nft_workspace_bytes": (SZ, [I32, I32]),
        "nft_loss": (ctypes.c_int, [ctypes.c_int, P, I64, P, I64, P, I64, P, P, I32, I32, I64, I32,
                                    P, F32, I32, F32, P, I64, P, P, SZ, P]),
        "quantize_rows_fp8": (ctypes.c_int, [ctypes.c_int, P, I64, P, I64, P, I64, I32, P]),
        "linear_fp8": (ctypes.c_int, [P, I64, P, P, P, P, ctypes.c_int, P, I64, P, P, P, I64, I64,
                                      I32, I32, P]),
        "adaln_modulate_fp8": (ctypes.c_int, [ctypes.c_int, P, I64, P, P, P, I64, P, I64, I32, F32,
                                              P]),
        "dit_block_fp8_workspace_bytes": (SZ, [ctypes.POINTER(BlockDesc), I64]),
        "dit_block_forward_fp8": (ctypes.c_int, [ctypes.POINTER(BlockDesc), P, P, P, P, P, I32,
                                                 I32, I64, P, P, P, P, P, P, P, P, SZ, P]),
        "dit_block_fp8_attn_workspace_bytes": (SZ, [ctypes.POINTER(BlockDesc), I64, I32]),
        "dit_block_forward_fp8_attn": (ctypes.c_int, [ctypes.POINTER(BlockDesc), P, P, P, P, P,
                                                      I32, I32, I64, P, P, P, P, P, P, P, P, SZ,
                                                      P]),
        "dit_ffn_fp8_workspace_bytes": (SZ, [ctypes.POINTER(FfnDesc), I64]),
        "dit_ffn_forward_fp8": (ctypes.c_int, [ctypes.POINTER(FfnDesc), P, P, P, I64, P, P, P, P,
                                               P, P, P, P, SZ, P]),
        "attn_packed_lse": (ctypes.c_int, [ctypes.c_int, P, I64, P, I64, P, I64, P, I64, P, P,
                                           I32, I32, I64, I32, I32, F32, I32, P]),
        "dit_attn_backward_workspace_bytes": (SZ, [I64, I32]),
        "attn_packed_backward": (ctypes.c_int, [ctypes.c_int, P, I64, P, I64, P, I64, P, I64, P,
                                                I64, P, P, I64, P, I64, P, I64, P, I32, I32, I64,
                                                I32, I32, F32, I32, P, SZ, P]),
        "dit_attn_backward_noalloc_max_elements": (SZ, []),
        "attn_packed_backward_noalloc": (ctypes.c_int, [ctypes.c_int, P, I64, P, I64, P, I64, P,
                                                        I64, P, I64, P, P, I64, P, I64, P, I64, P,
                                                        I32, I32, I64, I32, I32, F32, I32, P]),
        "dit_block_backward_workspace_bytes": (SZ, [ctypes.POINTER(BlockDesc), I64]),
        "dit_block_backward": (ctypes.c_int, [ctypes.POINTER(BlockDesc), P, P, P, P, P, I32, I32,
                                              I64, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "dit_ffn_backward_workspace_bytes": (SZ, [ctypes.POINTER(FfnDesc), I64]),
        "dit_ffn_backward": (ctypes.c_int, [ctypes.POINTER(FfnDesc), P, P, P, I64, P, P, P, P, P,
                                            P, P, P, P, P, P, P, SZ, P]),
        "dit_attn_fp8_workspace_bytes": (SZ, [I64, I32, I32, I32]),
        "dit_attn_fp8_layout": (ctypes.c_int, [I64, I32, I32, I32, ctypes.POINTER(I64)]),
        "attn_fp8_prepare": (ctypes.c_int, [P, I64, P, I64, P, I64, P, I32, I32, I64, I32, I32, P,
                                            SZ, P]),
        "attn_packed_fp8": (ctypes.c_int, [P, SZ, P, I64, P, I32, I32, I64, I32, I32, F32, I32,
                                           P]),
        "dit_profile_enable": (ctypes.c_int, [I32]),
        "dit_profile_read": (ctypes.c_int, [ctypes.POINTER(F32), ctypes.POINTER(I32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def abi_version() -> int:
    return _lib.dit_abi_version()


def last_error() -> str:
    return _lib.dit_last_error().decode()


def _check(status: int) -> None:
    if status != DIT_OK:
        raise DitError(status, last_error())


# ---------------------------------------------------------------------------
# host layout
# ---------------------------------------------------------------------------

def grid_from_media(frames: int, height_px: int, width_px: int, audio_samples_per_ch: int,
                    text_len: int) -> Tuple[int, int, int, int, int]:
    m = _Media(frames, height_px, width_px, audio_samples_per_ch, text_len)
    g = _Grid()
    _check(_lib.dit_grid_from_media(ctypes.byref(m), ctypes.byref(g)))
    return (g.t, g.h, g.w, g.audio_per_ch, g.text_len)


def pack_count(grids: Sequence[Sequence[int]]) -> Tuple[int, int]:
    """(n_tokens, max_seqlen) of the pack of these request grids (libdit dit_pack_count)."""
    n = len(grids)
    arr = (_Grid * max(n, 1))(*[_Grid(*map(int, g)) for g in grids])
    nt = ctypes.c_int64(0)
    ms = ctypes.c_int32(0)
    _check(_lib.dit_pack_count(arr, n, ctypes.byref(nt), ctypes.byref(ms)))
    return nt.value, ms.value


def pack_layout(grids: Sequence[Sequence[int]], capacity: Optional[int] = None) -> dict:
    """Returns dict(modality uint8[N], pos int32[N][3], cu_seqlens int32[R+1], max_seqlen, n_tokens)."""
    n = len(grids)
    arr = (_Grid * max(n, 1))(*[_Grid(*map(int, g)) for g in grids])
    if capacity is None:
        capacity = pack_count(grids)[0]
    cap = max(int(capacity), 1)
    mod = np.zeros(cap, dtype=np.uint8)
    pos = np.zeros((cap, 3), dtype=np.int32)
    cu = np.zeros(n + 1, dtype=np.int32)
    nt = ctypes.c_int64(0)
    ms = ctypes.c_int32(0)
    _check(_lib.dit_pack_layout(arr, n, mod.ctypes.data, pos.ctypes.data, cu.ctypes.data,
                                int(capacity), ctypes.byref(nt), ctypes.byref(ms)))
    k = nt.value
    return dict(modality=mod[:k], pos=pos[:k], cu_seqlens=cu, max_seqlen=ms.value, n_tokens=k)


# ---------------------------------------------------------------------------
# device stages (torch tensors in, results written in place / into `out`)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DIT_BF16
    if t.dtype == torch.float32:
        return DIT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _rows(t) -> Tuple[int, int]:
    """(pointer, ld) of a 2-D row-major view with unit column stride."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with contiguous rows")
    return t.data_ptr(), t.stride(0)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def adaln_modulate(x, modality, table, eps: float = 1e-6, out=None, n_tokens=None,
                   stream=None):
    """y = LN(x) * (1 + table[m][1]) + table[m][0] per token (libdit adaln_modulate)."""
    torch = _torch()
    n = x.shape[0] if n_tokens is None else int(n_tokens)
    d = x.shape[1]
    if out is None:
        out = torch.empty((x.shape[0], d), dtype=x.dtype, device=x.device)
    px, ldx = _rows(x)
    py, ldy = _rows(out)
    _check(_lib.adaln_modulate(_dtype_code(x), px, ldx, modality.data_ptr(), table.data_ptr(),
                               py, ldy, n, d, float(eps), _stream(stream)))
    return out


def rope3d_apply(q, k, pos, n_heads: int, head_dim: int, sections: Sequence[int],
                 theta: float = 10000.0, n_tokens=None, stream=None):
    """Rotate q (and k, unless None) in place (libdit rope3d_apply)."""
    n = q.shape[0] if n_tokens is None else int(n_tokens)
    pq, ldq = _rows(q)
    pk, ldk = (0, 0) if k is None else _rows(k)
    sec = (ctypes.c_int32 * 3)(*[int(s) for s in sections])
    _check(_lib.rope3d_apply(_dtype_code(q), pq, ldq, pk, ldk, pos.data_ptr(), n, n_heads,
                             head_dim, sec, float(theta), _stream(stream)))


def rope3d_apply_to(q, k, q_out, k_out, pos, n_heads: int, head_dim: int,
                    sections: Sequence[int], theta: float = 10000.0, n_tokens=None, stream=None):
    """Rotate q into q_out and k into k_out (libdit rope3d_apply_to)."""
    n = q.shape[0] if n_tokens is None else int(n_tokens)
    pq, ldq = _rows(q)
    pqo, ldqo = _rows(q_out)
    pk, ldk = (0, 0) if k is None else _rows(k)
    pko, ldko = (0, 0) if k_out is None else _rows(k_out)
    sec = (ctypes.c_int32 * 3)(*[int(s) for s in sections])
    _check(_lib.rope3d_apply_to(_dtype_code(q), pq, ldq, pk, ldk, pqo, ldqo, pko, ldko,
                                pos.data_ptr(), n, n_heads, head_dim, sec, float(theta),
                                _stream(stream)))


def attn_packed(q, k, v, cu_seqlens, max_seqlen: int, n_heads: int, head_dim: int,
                softmax_scale: float = 0.0, causal: bool = False, out=None, n_tokens=None,
                stream=None):
    """Packed-sequence softmax attention (libdit attn_packed)."""
    torch = _torch()
    n = q.shape[0] if n_tokens is None else int(n_tokens)
    if out is None:
        out = torch.empty((q.shape[0], n_heads * head_dim), dtype=q.dtype, device=q.device)
    pq, ldq = _rows(q)
    pk, ldk = _rows(k)
    pv, ldv = _rows(v)
    po, ldo = _rows(out)
    n_seqs = cu_seqlens.numel() - 1
    _check(_lib.attn_packed(_dtype_code(q), pq, ldq, pk, ldk, pv, ldv, po, ldo,
                            cu_seqlens.data_ptr(), n_seqs, int(max_seqlen), n, n_heads,
                            head_dim, float(softmax_scale), int(bool(causal)), _stream(stream)))
    return out


def attn_packed_lse(q, k, v, cu_seqlens, max_seqlen: int, n_heads: int, head_dim: int,
                    softmax_scale: float = 0.0, causal: bool = False, out=None, lse=None,
                    n_tokens=None, stream=None):
    """attn_packed that also writes lse [n_heads][n_tokens] float32, each row's
    log-sum-exp of the scaled scores (libdit attn_packed_lse)."""
    torch = _torch()
    n = q.shape[0] if n_tokens is None else int(n_tokens)
    if out is None:
        out = torch.empty((q.shape[0], n_heads * head_dim), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((n_heads, n), dtype=torch.float32, device=q.device)
    pq, ldq = _rows(q)
    pk, ldk = _rows(k)
    pv, ldv = _rows(v)
    po, ldo = _rows(out)
    _check(_lib.attn_packed_lse(_dtype_code(q), pq, ldq, pk, ldk, pv, ldv, po, ldo,
                                lse.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                                int(max_seqlen), n, n_heads, head_dim, float(softmax_scale),
                                int(bool(causal)), _stream(stream)))
    return out, lse


def attn_fp8_workspace_bytes(n_tokens: int, n_seqs: int, n_heads: int, head_dim: int = 128) -> int:
    return int(_lib.dit_attn_fp8_workspace_bytes(int(n_tokens), int(n_seqs), int(n_heads),
                                                 int(head_dim)))


def attn_fp8_layout(n_tokens: int, n_seqs: int, n_heads: int, head_dim: int = 128) -> dict:
    """Byte offsets of the FP8 attention operands in the workspace
    (libdit dit_attn_fp8_layout): q8, k8, vt, sq, sk, sv, amax, and the row
    strides ld8 (bytes per token of q8 / k8) and ld_vt (bytes per d row of vt)."""
    out = (ctypes.c_int64 * 9)()
    _check(_lib.dit_attn_fp8_layout(int(n_tokens), int(n_seqs), int(n_heads), int(head_dim), out))
    keys = ("q8", "k8", "vt", "sq", "sk", "sv", "amax", "ld8", "ld_vt")
    return {k: int(v) for k, v in zip(keys, out)}


def attn_fp8_prepare(q, k, v, cu_seqlens, max_seqlen: int, n_heads: int, head_dim: int = 128,
                     workspace=None, n_tokens=None, stream=None):
    """FP8 operands of attn_packed_fp8 from bf16 q, k, v rows
    (libdit attn_fp8_prepare); returns the workspace (uint8, device)."""
    torch = _torch()
    n = q.shape[0] if n_tokens is None else int(n_tokens)
    n_seqs = cu_seqlens.numel() - 1
    if workspace is None:
        workspace = torch.empty(max(attn_fp8_workspace_bytes(n, n_seqs, n_heads, head_dim), 1),
                                dtype=torch.uint8, device=q.device)
    pq, ldq = _rows(q)
    pk, ldk = _rows(k)
    pv, ldv = _rows(v)
    _check(_lib.attn_fp8_prepare(pq, ldq, pk, ldk, pv, ldv, cu_seqlens.data_ptr(), n_seqs,
                                 int(max_seqlen), n, n_heads, head_dim, workspace.data_ptr(),
                                 workspace.numel(), _stream(stream)))
    return workspace


def attn_packed_fp8(workspace, cu_seqlens, max_seqlen: int, n_tokens: int, n_heads: int,
                    head_dim: int = 128, softmax_scale: float = 0.0, causal: bool = False,
                    out=None, stream=None):
    """bf16 o [n_tokens][n_heads*head_dim] of the FP8 attention over operands
    that attn_fp8_prepare wrote (libdit attn_packed_fp8)."""
    torch = _torch()
    n = int(n_tokens)
    if out is None:
        out = torch.empty((n, n_heads * head_dim), dtype=torch.bfloat16, device=workspace.device)
    po, ldo = _rows(out)
    _check(_lib.attn_packed_fp8(workspace.data_ptr(), workspace.numel(), po, ldo,
                                cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, int(max_seqlen), n,
                                n_heads, head_dim, float(softmax_scale), int(bool(causal)),
                                _stream(stream)))
    return out


def attn_backward_workspace_bytes(n_tokens: int, n_heads: int) -> int:
    return int(_lib.dit_attn_backward_workspace_bytes(int(n_tokens), int(n_heads)))


def attn_packed_backward(q, k, v, o, dout, lse, cu_seqlens, max_seqlen: int, n_heads: int,
                         head_dim: int, softmax_scale: float = 0.0, causal: bool = False,
                         dq=None, dk=None, dv=None, workspace=None, n_tokens=None, stream=None):
    """(dq, dk, dv) of attn_packed given dout and the forward's o and lse
    (libdit attn_packed_backward)."""
    torch = _torch()
    n = q.shape[0] if n_tokens is None else int(n_tokens)
    w = n_heads * head_dim
    dq = torch.empty((q.shape[0], w), dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty((q.shape[0], w), dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty((q.shape[0], w), dtype=q.dtype, device=q.device) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(max(attn_backward_workspace_bytes(n, n_heads), 1),
                                dtype=torch.uint8, device=q.device)
    args = []
    for t in (q, k, v, o, dout):
        args += list(_rows(t))
    args.append(lse.data_ptr())
    for t in (dq, dk, dv):
        args += list(_rows(t))
    _check(_lib.attn_packed_backward(_dtype_code(q), *args, cu_seqlens.data_ptr(),
                                     cu_seqlens.numel() - 1, int(max_seqlen), n, n_heads,
                                     head_dim, float(softmax_scale), int(bool(causal)),
                                     workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return dq, dk, dv


def attn_backward_noalloc_max_elements() -> int:
    return int(_lib.dit_attn_backward_noalloc_max_elements())


def attn_packed_backward_noalloc(q, k, v, o, dout, lse, cu_seqlens, max_seqlen: int,
                                 n_heads: int, head_dim: int, softmax_scale: float = 0.0,
                                 causal: bool = False, dq=None, dk=None, dv=None, n_tokens=None,
                                 stream=None):
    """attn_packed_backward with its scratch in the library's fixed device array
    (libdit attn_packed_backward_noalloc): no workspace argument.  dq, dk, dv
    must be given (caller-owned) or are allocated here by torch."""
    torch = _torch()
    n = q.shape[0] if n_tokens is None else int(n_tokens)
    w = n_heads * head_dim
    dq = torch.empty((q.shape[0], w), dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty((q.shape[0], w), dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty((q.shape[0], w), dtype=q.dtype, device=q.device) if dv is None else dv
    args = []
    for t in (q, k, v, o, dout):
        args += list(_rows(t))
    args.append(lse.data_ptr())
    for t in (dq, dk, dv):
        args += list(_rows(t))
    _check(_lib.attn_packed_backward_noalloc(_dtype_code(q), *args, cu_seqlens.data_ptr(),
                                             cu_seqlens.numel() - 1, int(max_seqlen), n, n_heads,
                                             head_dim, float(softmax_scale), int(bool(causal)),
                                             _stream(stream)))
    return dq, dk, dv


def qkv_project(y, w_qkv, b_qkv=None, out=None, n_tokens=None, stream=None):
    """qkv = y W_qkv^T (+ b) (libdit qkv_project)."""
    torch = _torch()
    n = y.shape[0] if n_tokens is None else int(n_tokens)
    d = y.shape[1]
    if out is None:
        out = torch.empty((y.shape[0], 3 * d), dtype=y.dtype, device=y.device)
    py, ldy = _rows(y)
    po, ldo = _rows(out)
    _check(_lib.qkv_project(_dtype_code(y), py, ldy, w_qkv.data_ptr(), _ptr(b_qkv), po, ldo, n,
                            d, _stream(stream)))
    return out


def out_proj_gated(o, w_o, x, modality, table, b_o=None, out=None, n_tokens=None, stream=None):
    """out = x + table[m][2] * (o W_o^T + b) (libdit out_proj_gated)."""
    torch = _torch()
    n = o.shape[0] if n_tokens is None else int(n_tokens)
    d = w_o.shape[0]
    if out is None:
        out = torch.empty((x.shape[0], d), dtype=x.dtype, device=x.device)
    po, ldo = _rows(o)
    px, ldx = _rows(x)
    pout, ldout = _rows(out)
    _check(_lib.out_proj_gated(_dtype_code(o), po, ldo, w_o.data_ptr(), _ptr(b_o), px, ldx,
                               modality.data_ptr(), table.data_ptr(), pout, ldout, n, d,
                               _stream(stream)))
    return out


def block_desc(dtype_code: int, d_model: int, n_heads: int, head_dim: int,
               sections: Sequence[int], theta: float = 10000.0, eps: float = 1e-6,
               softmax_scale: float = 0.0, causal: bool = False) -> BlockDesc:
    return BlockDesc(dtype_code, d_model, n_heads, head_dim, (ctypes.c_int32 * 3)(*sections),
                     theta, eps, softmax_scale, int(bool(causal)))


def block_workspace_bytes(desc: BlockDesc, n_tokens: int) -> int:
    return int(_lib.dit_block_workspace_bytes(ctypes.byref(desc), int(n_tokens)))


def block_intermediates(desc: BlockDesc, n_tokens: int) -> dict:
    """Byte offsets of y, q', k', v and o in dit_block_forward's workspace
    (libdit dit_block_intermediates)."""
    out = (ctypes.c_int64 * 5)()
    _check(_lib.dit_block_intermediates(ctypes.byref(desc), int(n_tokens), out))
    return dict(zip(("y", "q_rot", "k_rot", "v", "o"), (int(v) for v in out)))


def block_planes(desc: BlockDesc, workspace, n_tokens: int) -> dict:
    """Views of the intermediates dit_block_forward left in `workspace`: y, q_rot,
    k_rot, v, o as [n_tokens][d_model] tensors of the block's dtype."""
    torch = _torch()
    dt = torch.bfloat16 if desc.dtype == DIT_BF16 else torch.float32
    es = 2 if desc.dtype == DIT_BF16 else 4
    nbytes = int(n_tokens) * desc.d_model * es
    views = {}
    for name, off in block_intermediates(desc, n_tokens).items():
        views[name] = workspace[off:off + nbytes].view(dt).view(int(n_tokens), desc.d_model)
    return views


def block_forward(desc: BlockDesc, x, modality, pos, cu_seqlens, max_seqlen: int, table, w_qkv,
                  w_o, b_qkv=None, b_o=None, out=None, workspace=None, n_tokens=None,
                  stream=None):
    """The attention half of one DiT block (libdit dit_block_forward)."""
    torch = _torch()
    n = x.shape[0] if n_tokens is None else int(n_tokens)
    if out is None:
        out = torch.empty_like(x)
    need = block_workspace_bytes(desc, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(_lib.dit_block_forward(ctypes.byref(desc), x.data_ptr(), out.data_ptr(),
                                  modality.data_ptr(), pos.data_ptr(), cu_seqlens.data_ptr(),
                                  cu_seqlens.numel() - 1, int(max_seqlen), n, table.data_ptr(),
                                  w_qkv.data_ptr(), _ptr(b_qkv), w_o.data_ptr(), _ptr(b_o),
                                  workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out


def ffn_up_gelu(y, w1, b1=None, out=None, n_tokens=None, stream=None):
    """h = gelu_tanh(y W1^T + b1) (libdit ffn_up_gelu)."""
    torch = _torch()
    n = y.shape[0] if n_tokens is None else int(n_tokens)
    d, f = y.shape[1], w1.shape[0]
    if out is None:
        out = torch.empty((y.shape[0], f), dtype=y.dtype, device=y.device)
    py, ldy = _rows(y)
    ph, ldh = _rows(out)
    _check(_lib.ffn_up_gelu(_dtype_code(y), py, ldy, w1.data_ptr(), _ptr(b1), ph, ldh, n, d, f,
                            _stream(stream)))
    return out


def ffn_down_gated(h, w2, x, modality, table, b2=None, out=None, n_tokens=None, stream=None):
    """out = x + table[m][2] * (h W2^T + b2) (libdit ffn_down_gated)."""
    torch = _torch()
    n = h.shape[0] if n_tokens is None else int(n_tokens)
    d, f = w2.shape
    if out is None:
        out = torch.empty((x.shape[0], d), dtype=x.dtype, device=x.device)
    ph, ldh = _rows(h)
    px, ldx = _rows(x)
    pout, ldout = _rows(out)
    _check(_lib.ffn_down_gated(_dtype_code(h), ph, ldh, w2.data_ptr(), _ptr(b2), px, ldx,
                               modality.data_ptr(), table.data_ptr(), pout, ldout, n, d, f,
                               _stream(stream)))
    return out


def ffn_desc(dtype_code: int, d_model: int, d_ff: int, eps: float = 1e-6) -> FfnDesc:
    return FfnDesc(dtype_code, d_model, d_ff, eps)


def ffn_workspace_bytes(desc: FfnDesc, n_tokens: int) -> int:
    return int(_lib.dit_ffn_workspace_bytes(ctypes.byref(desc), int(n_tokens)))


def ffn_forward(desc: FfnDesc, x, modality, table, w1, w2, b1=None, b2=None, out=None,
                workspace=None, n_tokens=None, stream=None):
    """The feed-forward half of one DiT block (libdit dit_ffn_forward)."""
    torch = _torch()
    n = x.shape[0] if n_tokens is None else int(n_tokens)
    if out is None:
        out = torch.empty_like(x)
    need = ffn_workspace_bytes(desc, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(_lib.dit_ffn_forward(ctypes.byref(desc), x.data_ptr(), out.data_ptr(),
                                modality.data_ptr(), n, table.data_ptr(), w1.data_ptr(), _ptr(b1),
                                w2.data_ptr(), _ptr(b2), workspace.data_ptr(), workspace.numel(),
                                _stream(stream)))
    return out


def profile_enable(max_calls: int) -> None:
    _check(_lib.dit_profile_enable(int(max_calls)))


def profile_read() -> Tuple[List[float], int]:
    """Summed per-stage milliseconds of the recorded dit_block_forward calls, and their count."""
    ms = (ctypes.c_float * len(STAGES))()
    n = ctypes.c_int32(0)
    _check(_lib.dit_profile_read(ms, ctypes.byref(n)))
    return list(ms), n.value


# ---------------------------------------------------------------------------
# denoising step around the block
# ---------------------------------------------------------------------------

def timestep_from_sigma(sigma: float) -> float:
    """H3's data-progress time for a scheduler noise level: t = 1 - sigma."""
    return 1.0 - float(sigma)


def denoise_step(z, v, modality, sigmas: Sequence[float], x0=None, anchor=None,
                 anchor_vals=None, velocity_sign: int = 1, n_rows=None, stream=None):
    """One step of the joint loop in place on z (libdit denoise_step).

    sigmas = (sigma_video, sigma_video_next, sigma_audio, sigma_audio_next);
    x0, if given, receives the clean estimate of every video/audio row.
    """
    n = z.shape[0] if n_rows is None else int(n_rows)
    c = z.shape[1]
    pz, ldz = _rows(z)
    pv, ldv = _rows(v)
    px, ldx = (0, 0) if x0 is None else _rows(x0)
    pa, lda = (0, 0) if anchor_vals is None else _rows(anchor_vals)
    sig = (ctypes.c_float * 4)(*[float(x) for x in sigmas])
    _check(_lib.denoise_step(_dtype_code(v), pz, ldz, pv, ldv, px, ldx, modality.data_ptr(),
                             _ptr(anchor), pa, lda, n, c, sig, int(velocity_sign),
                             _stream(stream)))
    return z


# ---------------------------------------------------------------------------
# DiffusionNFT loss
# ---------------------------------------------------------------------------

def nft_workspace_bytes(n_samples: int, max_rows: int) -> int:
    return int(_lib.dit_nft_workspace_bytes(int(n_samples), int(max_rows)))


def nft_loss(v_theta, v_old, v_target, cu_samples, max_rows: int, reward, beta: float,
             loss_mask=None, velocity_sign: int = 1, grad_scale=None, grad=None,
             loss_out=None, workspace=None, want_grad: bool = True, n_rows=None, stream=None):
    """DiffusionNFT loss per sample and its gradient (libdit nft_loss).

    Returns (loss_out [S][3] = (loss, mse_pos, mse_neg), grad or None)."""
    torch = _torch()
    n_s = cu_samples.numel() - 1
    n = v_theta.shape[0] if n_rows is None else int(n_rows)
    c = v_theta.shape[1]
    dev = v_theta.device
    if loss_out is None:
        loss_out = torch.empty((n_s, 3), dtype=torch.float32, device=dev)
    if grad is None and want_grad:
        grad = torch.empty((v_theta.shape[0], c), dtype=torch.float32, device=dev)
    need = nft_workspace_bytes(n_s, max(int(max_rows), 1))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    pt, ldt = _rows(v_theta)
    po, ldo = _rows(v_old)
    pg, ldg = (0, 0) if grad is None else _rows(grad)
    ptg, ldtg = _rows(v_target)
    scale = 1.0 / n_s if grad_scale is None else float(grad_scale)
    _check(_lib.nft_loss(_dtype_code(v_theta), pt, ldt, po, ldo, ptg, ldtg, _ptr(loss_mask),
                         cu_samples.data_ptr(), n_s, int(max_rows), n, c, reward.data_ptr(),
                         float(beta), int(velocity_sign), scale, pg, ldg, loss_out.data_ptr(),
                         workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return loss_out, grad


# ---------------------------------------------------------------------------
# FP8 projections
# ---------------------------------------------------------------------------

DIT_EPI_PLAIN, DIT_EPI_GATED, DIT_EPI_GELU = 0, 1, 2
_EPI = {"plain": DIT_EPI_PLAIN, "gated": DIT_EPI_GATED, "gelu": DIT_EPI_GELU}


def quantize_rows_fp8(x, codes=None, scales=None, n_rows=None, stream=None):
    """Per-row e4m3 codes and float32 scales of x (libdit quantize_rows_fp8)."""
    torch = _torch()
    n = x.shape[0] if n_rows is None else int(n_rows)
    d = x.shape[1]
    if codes is None:
        codes = torch.empty((x.shape[0], d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    px, ldx = _rows(x)
    pq, ldq = _rows(codes)
    _check(_lib.quantize_rows_fp8(_dtype_code(x), px, ldx, pq, ldq, scales.data_ptr(), n, d,
                                  _stream(stream)))
    return codes, scales


def linear_fp8(a_codes, a_scales, w_codes, w_scales, bias=None, epilogue: str = "plain", x=None,
               modality=None, table=None, out=None, n_tokens=None, stream=None):
    """out = epilogue(dequant(A) dequant(W)^T + bias) in bf16 (libdit linear_fp8)."""
    torch = _torch()
    n = a_codes.shape[0] if n_tokens is None else int(n_tokens)
    f, k = w_codes.shape
    if out is None:
        out = torch.empty((a_codes.shape[0], f), dtype=torch.bfloat16, device=a_codes.device)
    pa, lda = _rows(a_codes)
    po, ldo = _rows(out)
    px, ldx = (0, 0) if x is None else _rows(x)
    _check(_lib.linear_fp8(pa, lda, a_scales.data_ptr(), w_codes.data_ptr(), w_scales.data_ptr(),
                           _ptr(bias), _EPI[epilogue], px, ldx, _ptr(modality), _ptr(table), po,
                           ldo, n, k, f, _stream(stream)))
    return out


def adaln_modulate_fp8(x, modality, table, eps: float = 1e-6, codes=None, scales=None,
                       n_tokens=None, stream=None):
    """AdaLN with its output as per-row e4m3 codes and float32 scales (libdit
    adaln_modulate_fp8)."""
    torch = _torch()
    n = x.shape[0] if n_tokens is None else int(n_tokens)
    d = x.shape[1]
    if codes is None:
        codes = torch.empty((x.shape[0], d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    px, ldx = _rows(x)
    pq, ldq = _rows(codes)
    _check(_lib.adaln_modulate_fp8(_dtype_code(x), px, ldx, modality.data_ptr(), table.data_ptr(),
                                   pq, ldq, scales.data_ptr(), n, d, float(eps), _stream(stream)))
    return codes, scales


def block_fp8_workspace_bytes(desc: BlockDesc, n_tokens: int) -> int:
    return int(_lib.dit_block_fp8_workspace_bytes(ctypes.byref(desc), int(n_tokens)))


def block_fp8_attn_workspace_bytes(desc: BlockDesc, n_tokens: int, n_seqs: int) -> int:
    return int(_lib.dit_block_fp8_attn_workspace_bytes(ctypes.byref(desc), int(n_tokens),
                                                        int(n_seqs)))


def block_forward_fp8(desc: BlockDesc, x, modality, pos, cu_seqlens, max_seqlen: int, table,
                      w_qkv_codes, w_qkv_scales, w_o_codes, w_o_scales, b_qkv=None, b_o=None,
                      out=None, workspace=None, n_tokens=None, stream=None,
                      fp8_attention: bool = False):
    """The attention half with FP8 projections (libdit dit_block_forward_fp8),
    or with the attention in FP8 too (dit_block_forward_fp8_attn)."""
    torch = _torch()
    n = x.shape[0] if n_tokens is None else int(n_tokens)
    if out is None:
        out = torch.empty_like(x)
    if fp8_attention:
        need = block_fp8_attn_workspace_bytes(desc, n, cu_seqlens.numel() - 1)
        fn = _lib.dit_block_forward_fp8_attn
    else:
        need = block_fp8_workspace_bytes(desc, n)
        fn = _lib.dit_block_forward_fp8
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(fn(
        ctypes.byref(desc), x.data_ptr(), out.data_ptr(), modality.data_ptr(), pos.data_ptr(),
        cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, int(max_seqlen), n, table.data_ptr(),
        w_qkv_codes.data_ptr(), w_qkv_scales.data_ptr(), _ptr(b_qkv), w_o_codes.data_ptr(),
        w_o_scales.data_ptr(), _ptr(b_o), workspace.data_ptr(), workspace.numel(),
        _stream(stream)))
    return out


def ffn_fp8_workspace_bytes(desc: FfnDesc, n_tokens: int) -> int:
    return int(_lib.dit_ffn_fp8_workspace_bytes(ctypes.byref(desc), int(n_tokens)))


def ffn_forward_fp8(desc: FfnDesc, x, modality, table, w1_codes, w1_scales, w2_codes, w2_scales,
                    b1=None, b2=None, out=None, workspace=None, n_tokens=None, stream=None):
    """The feed-forward half with FP8 projections (libdit dit_ffn_forward_fp8)."""
    torch = _torch()
    n = x.shape[0] if n_tokens is None else int(n_tokens)
    if out is None:
        out = torch.empty_like(x)
    need = ffn_fp8_workspace_bytes(desc, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(_lib.dit_ffn_forward_fp8(
        ctypes.byref(desc), x.data_ptr(), out.data_ptr(), modality.data_ptr(), n,
        table.data_ptr(), w1_codes.data_ptr(), w1_scales.data_ptr(), _ptr(b1),
        w2_codes.data_ptr(), w2_scales.data_ptr(), _ptr(b2), workspace.data_ptr(),
        workspace.numel(), _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# Backward pass of the attention half
# ---------------------------------------------------------------------------

def block_backward_workspace_bytes(desc: BlockDesc, n_tokens: int) -> int:
    return int(_lib.dit_block_backward_workspace_bytes(ctypes.byref(desc), int(n_tokens)))


def block_backward(desc: BlockDesc, x, dout, modality, pos, cu_seqlens, max_seqlen: int, table,
                   w_qkv, w_o, b_qkv=None, b_o=None, bias_grads: bool = True, dx=None,
                   workspace=None, n_tokens=None, stream=None) -> dict:
    """Gradients of sum(dout * out) of the attention half (libdit dit_block_backward):
    dict(dx, dtable [3][3][D] float32, dw_qkv, dw_o, db_qkv, db_o (float32 or None))."""
    torch = _torch()
    n = x.shape[0] if n_tokens is None else int(n_tokens)
    d = x.shape[1]
    dev = x.device
    dx = torch.empty_like(x) if dx is None else dx
    dtable = torch.empty((3, 3, d), dtype=torch.float32, device=dev)
    dw_qkv = torch.empty((3 * d, d), dtype=x.dtype, device=dev)
    dw_o = torch.empty((d, d), dtype=x.dtype, device=dev)
    db_qkv = torch.empty(3 * d, dtype=torch.float32, device=dev) if bias_grads else None
    db_o = torch.empty(d, dtype=torch.float32, device=dev) if bias_grads else None
    if workspace is None:
        workspace = torch.empty(max(block_backward_workspace_bytes(desc, n), 1),
                                dtype=torch.uint8, device=dev)
    _check(_lib.dit_block_backward(
        ctypes.byref(desc), x.data_ptr(), dout.data_ptr(), modality.data_ptr(), pos.data_ptr(),
        cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, int(max_seqlen), n, table.data_ptr(),
        w_qkv.data_ptr(), _ptr(b_qkv), w_o.data_ptr(), _ptr(b_o), dx.data_ptr(),
        dtable.data_ptr(), dw_qkv.data_ptr(), _ptr(db_qkv), dw_o.data_ptr(), _ptr(db_o),
        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return dict(dx=dx, dtable=dtable, dw_qkv=dw_qkv, dw_o=dw_o, db_qkv=db_qkv, db_o=db_o)


def ffn_backward_workspace_bytes(desc: FfnDesc, n_tokens: int) -> int:
    return int(_lib.dit_ffn_backward_workspace_bytes(ctypes.byref(desc), int(n_tokens)))


def ffn_backward(desc: FfnDesc, x, dout, modality, table, w1, w2, b1=None, b2=None,
                 bias_grads: bool = True, dx=None, workspace=None, n_tokens=None,
                 stream=None) -> dict:
    """Gradients of sum(dout * out) of the feed-forward half (libdit dit_ffn_backward):
    dict(dx, dtable [3][3][D] float32, dw1, dw2, db1, db2 (float32 or None))."""
    torch = _torch()
    n = x.shape[0] if n_tokens is None else int(n_tokens)
    d, f = x.shape[1], w1.shape[0]
    dev = x.device
    dx = torch.empty_like(x) if dx is None else dx
    dtable = torch.empty((3, 3, d), dtype=torch.float32, device=dev)
    dw1 = torch.empty((f, d), dtype=x.dtype, device=dev)
    dw2 = torch.empty((d, f), dtype=x.dtype, device=dev)
    db1 = torch.empty(f, dtype=torch.float32, device=dev) if bias_grads else None
    db2 = torch.empty(d, dtype=torch.float32, device=dev) if bias_grads else None
    if workspace is None:
        workspace = torch.empty(max(ffn_backward_workspace_bytes(desc, n), 1), dtype=torch.uint8,
                                device=dev)
    _check(_lib.dit_ffn_backward(
        ctypes.byref(desc), x.data_ptr(), dout.data_ptr(), modality.data_ptr(), n,
        table.data_ptr(), w1.data_ptr(), _ptr(b1), w2.data_ptr(), _ptr(b2), dx.data_ptr(),
        dtable.data_ptr(), dw1.data_ptr(), _ptr(db1), dw2.data_ptr(), _ptr(db2),
        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return dict(dx=dx, dtable=dtable, dw1=dw1, dw2=dw2, db1=db1, db2=db2)
