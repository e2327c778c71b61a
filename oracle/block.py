"""Float64 stages of one DiT block: AdaLN, QKV, 3D RoPE, attention, gated output.

Test infrastructure only (see the package docstring).  Every function widens
its inputs to float64 and rounds nothing in between.  Arrays are row-major,
one token per row; a q/k/v/o row holds its heads side by side, head h in
columns [h*Dh, (h+1)*Dh).  Large inputs are processed in row chunks only to
bound memory; chunking does not change any result.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

_ROW_CHUNK = 2048


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _rows(rows, n):
    return np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)


def adaln_modulate(x, modality, table, eps: float = 1e-6, rows=None) -> np.ndarray:
    """Per-modality adaptive LayerNorm of each token.

    [H3-NFT], section on H3's architecture: the transformer has AdaLN branches
    per modality (not per-modality attention or feed-forward), and their
    modulation outputs can be computed once and cached; [VeRL-Omni] section 3
    (H3's unified generation) has all modalities share attention weights and
    AdaLN modulation.  So the block takes a cached table T[m][r][d] (m =
    modality 0 video / 1 audio / 2 text, r = 0 shift / 1 scale / 2 gate).

    Readings: LayerNorm over d_model without its own affine, biased variance,
    eps = 1e-6; y = xhat * (1 + scale) + shift (the DiT adaLN convention, so
    a zero table row is the identity modulation).
    """
    x = np.asarray(x)
    idx = _rows(rows, x.shape[0])
    mod = np.asarray(modality, dtype=np.int64)
    tab = _f64(table)
    out = np.empty((idx.size, x.shape[1]), dtype=np.float64)
    for s in range(0, idx.size, _ROW_CHUNK):
        r = idx[s:s + _ROW_CHUNK]
        xr = _f64(x[r])
        mu = xr.mean(axis=1, keepdims=True)
        var = ((xr - mu) ** 2).mean(axis=1, keepdims=True)
        xhat = (xr - mu) / np.sqrt(var + eps)
        m = mod[r]
        out[s:s + r.size] = xhat * (1.0 + tab[m, 1, :]) + tab[m, 0, :]
    return out


def qkv_project(y, w_qkv, b_qkv=None) -> np.ndarray:
    """Fused QKV projection qkv = y W_qkv^T (+ b).

    [VeRL-Omni] section 5.2: the rollout side packs the Q, K and V projections
    into one matrix; [H3-NFT] names them to_q, to_k, to_v.  Reading: W_qkv rows
    are to_q, then to_k, then to_v, each [D][D] in torch Linear layout
    ([out][in]), so qkv columns [0, D) are q, [D, 2D) k and [2D, 3D) v.
    """
    y = np.asarray(y)
    w = _f64(w_qkv)
    out = np.empty((y.shape[0], w.shape[0]), dtype=np.float64)
    for s in range(0, y.shape[0], _ROW_CHUNK):
        out[s:s + _ROW_CHUNK] = _f64(y[s:s + _ROW_CHUNK]) @ w.T
    if b_qkv is not None:
        out += _f64(b_qkv)
    return out


def rope_frequencies(section: int, theta: float) -> np.ndarray:
    """omega_j = theta^(-2j/s) for j in [0, s/2) of one section of size s."""
    j = np.arange(section // 2, dtype=np.float64)
    return theta ** (-2.0 * j / section)


def rope3d(x, pos, n_heads: int, head_dim: int, sections: Sequence[int],
           theta: float = 10000.0, rows=None) -> np.ndarray:
    """3D (time, height, width) rotary embedding of q or k, every head alike.

    [H3-NFT], section on H3's architecture: rotary position embedding over
    three axes, time, height and width.  [vLLM-Omni] section 3: each row
    carries its spatial/temporal position, and the modality tag steers RoPE's
    frequency selection so that modalities keep independent position spaces.

    Readings: head_dim splits into sections (s_t, s_h, s_w) at offsets 0,
    s_t, s_t + s_h; inside section a each adjacent pair (2j, 2j+1) is the
    complex number u + i w multiplied by exp(i pos_a omega_j) with
    omega_j = theta^(-2j / s_a) (RoFormer's rotary embedding, one 1-D RoPE
    per axis).  Audio and text rows have h = w = 0, so only their time
    section turns.  The pairing convention is parity unpinned by the pages:
    the tests pin the frequencies, the rotation and its relative-offset
    invariant, which hold for any pairing, so which dimensions pair up rests
    on this reading alone.

    x: [N][n_heads*head_dim]; pos: [N][3] ints.  Returns float64 [rows][H*Dh].
    """
    x = np.asarray(x)
    idx = _rows(rows, x.shape[0])
    p = np.asarray(pos, dtype=np.int64)[idx]
    if sum(sections) != head_dim or any(s % 2 for s in sections):
        raise ValueError("sections must be even and sum to head_dim")
    xr = _f64(x[idx]).reshape(idx.size, n_heads, head_dim)
    out = xr.copy()
    off = 0
    for axis, s in enumerate(sections):
        omega = rope_frequencies(s, theta)                        # [s/2]
        phi = p[:, axis].astype(np.float64)[:, None] * omega      # [n, s/2]
        c = np.cos(phi)[:, None, :]
        sn = np.sin(phi)[:, None, :]
        u = xr[:, :, off:off + s:2]
        w = xr[:, :, off + 1:off + s:2]
        out[:, :, off:off + s:2] = u * c - w * sn
        out[:, :, off + 1:off + s:2] = u * sn + w * c
        off += s
    return out.reshape(idx.size, n_heads * head_dim)


def _segment_of(cu, n_tokens):
    seg = np.empty(n_tokens, dtype=np.int64)
    for s in range(len(cu) - 1):
        seg[cu[s]:cu[s + 1]] = s
    return seg


def _probs(qh, kh, qi, seg_start, causal, scale):
    """Softmax weights of query rows qi (absolute indices) against keys kh of one segment."""
    s = (qh @ kh.T) * scale
    if causal:
        kj = seg_start + np.arange(kh.shape[0])
        s = np.where(kj[None, :] <= qi[:, None], s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def attention(q, k, v, cu_seqlens, n_heads: int, head_dim: int,
              causal: bool = False, scale: Optional[float] = None,
              rows=None) -> np.ndarray:
    """Softmax attention inside each cu_seqlens segment, per head.

    [vLLM-Omni] section 3: the attention kernel derives its mask from
    cu_seqlens, so a token normalises its softmax only over keys of its own
    sub-sequence, and other sub-sequences get exactly zero weight; section 1:
    audio and video share one attention context (full attention, [H3-NFT]
    "Limitations" section).  Reading: scale = 1/sqrt(head_dim), no q/k norm;
    causal means key j <= query i inside the segment ([VeRL-Omni] section 3
    mentions causal attention; kept as a variant).

    q, k, v: [N][H*Dh].  Returns float64 o [rows][H*Dh].
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    n = q.shape[0]
    cu = [int(c) for c in cu_seqlens]
    if cu[0] != 0 or cu[-1] != n or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("bad cu_seqlens")
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    idx = _rows(rows, n)
    seg = _segment_of(cu, n)
    out = np.empty((idx.size, n_heads * head_dim), dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        sel = np.nonzero(seg[idx] == s)[0]
        if sel.size == 0:
            continue
        qi = idx[sel]
        for h in range(n_heads):
            cols = slice(h * head_dim, (h + 1) * head_dim)
            kh = _f64(k[a:b, cols])
            vh = _f64(v[a:b, cols])
            for c in range(0, sel.size, 512):
                part = sel[c:c + 512]
                qh = _f64(q[idx[part], cols])
                p = _probs(qh, kh, idx[part], a, causal, scale)
                out[part, cols] = p @ vh
    return out


def attention_probs(q, k, cu_seqlens, n_heads: int, head_dim: int,
                    causal: bool = False, scale: Optional[float] = None) -> np.ndarray:
    """Full [H][N][N] softmax weight matrix for small N (zero across segments)."""
    q, k = np.asarray(q), np.asarray(k)
    n = q.shape[0]
    cu = [int(c) for c in cu_seqlens]
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    P = np.zeros((n_heads, n, n), dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b == a:
            continue
        for h in range(n_heads):
            cols = slice(h * head_dim, (h + 1) * head_dim)
            P[h, a:b, a:b] = _probs(_f64(q[a:b, cols]), _f64(k[a:b, cols]),
                                    np.arange(a, b), a, causal, scale)
    return P


def out_proj_gated(o, w_o, x, modality, table, b_o=None, rows=None) -> np.ndarray:
    """Output projection (to_out.0) and gated residual: x + gate[m] * (o W_o^T + b).

    [H3-NFT] names the attention output projection to_out.0; the gate row of
    the per-modality AdaLN table scales the branch before the residual add
    (DiT adaLN convention; a reading).  o: [rows][D] already restricted to
    ``rows`` when given; x: full [N][D].
    """
    o = np.asarray(o)
    x = np.asarray(x)
    idx = _rows(rows, x.shape[0])
    if o.shape[0] != idx.size:
        raise ValueError("o rows must match rows")
    w = _f64(w_o)
    mod = np.asarray(modality, dtype=np.int64)
    tab = _f64(table)
    out = np.empty((idx.size, w.shape[0]), dtype=np.float64)
    for s in range(0, idx.size, _ROW_CHUNK):
        r = idx[s:s + _ROW_CHUNK]
        z = _f64(o[s:s + r.size]) @ w.T
        if b_o is not None:
            z += _f64(b_o)
        out[s:s + r.size] = _f64(x[r]) + tab[mod[r], 2, :] * z
    return out


def block_forward(x, modality, pos, cu_seqlens, table, w_qkv, w_o, *,
                  n_heads: int, head_dim: int, sections: Sequence[int],
                  theta: float = 10000.0, eps: float = 1e-6,
                  causal: bool = False, scale: Optional[float] = None,
                  b_qkv=None, b_o=None, rows=None) -> Dict[str, np.ndarray]:
    """The attention half of one DiT block, from the original inputs.

    AdaLN(modality) -> fused QKV -> 3D RoPE on q and k -> attention inside
    cu_seqlens segments -> to_out.0 -> x + gate * branch.  Stage order as in
    [vLLM-Omni] section 3 (tags and RoPE before the blocks, attention bounded
    by cu_seqlens) and [H3-NFT] (AdaLN per modality, projection names).

    Returns every stage (float64): y, q, k, v (before RoPE), q_rot, k_rot, o
    and out.  With ``rows``, o and out hold only those rows, and q / q_rot are
    filled only at those rows (k and v are still computed for every token,
    since attention needs them).
    """
    x = np.asarray(x)
    n, d = x.shape
    w = np.asarray(w_qkv)
    bias = [None] * 3 if b_qkv is None else [np.asarray(b_qkv)[i * d:(i + 1) * d] for i in range(3)]
    y = adaln_modulate(x, modality, table, eps)
    k = qkv_project(y, w[d:2 * d], bias[1])
    v = qkv_project(y, w[2 * d:], bias[2])
    k_rot = rope3d(k, pos, n_heads, head_dim, sections, theta)
    if rows is None:
        q = qkv_project(y, w[:d], bias[0])
        q_rot = rope3d(q, pos, n_heads, head_dim, sections, theta)
    else:
        # queries are only needed for the requested rows; scatter them into a
        # full-size array so that attention() can index them by token
        idx = _rows(rows, n)
        q = np.zeros((n, d))
        q[idx] = qkv_project(y[idx], w[:d], bias[0])
        q_rot = np.zeros((n, d))
        q_rot[idx] = rope3d(q[idx], np.asarray(pos)[idx], n_heads, head_dim, sections, theta)
    o = attention(q_rot, k_rot, v, cu_seqlens, n_heads, head_dim, causal, scale, rows)
    out = out_proj_gated(o, w_o, x, modality, table, b_o, rows)
    return dict(y=y, q=q, k=k, v=v, q_rot=q_rot, k_rot=k_rot, o=o, out=out)


# ---------------------------------------------------------------------------
# Feed-forward half of the block
# ---------------------------------------------------------------------------

_GELU_C = math.sqrt(2.0 / math.pi)


def gelu_tanh(z) -> np.ndarray:
    """GELU in its tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).

    Reading.  [H3-NFT] (section "How VeRL-Omni's Adapter Architecture Keeps
    H3-Specific Logic Contained") names the feed-forward weights ff.net.0.proj
    and ff.net.2 but not the activation.  A projection called `proj` inside the
    first element of the feed-forward stack is the layout of a GELU module
    that owns its input projection, and the DiT family uses the tanh form of
    GELU; that is the reading.  The pages do not pin it.
    """
    z = _f64(z)
    return 0.5 * z * (1.0 + np.tanh(_GELU_C * (z + 0.044715 * z * z * z)))


def ffn_up(y, w1, b1=None) -> np.ndarray:
    """First feed-forward projection and activation: gelu_tanh(y W1^T + b1).

    W1 is ff.net.0.proj, [d_ff][d_model] ([out][in]).
    """
    y = np.asarray(y)
    w = _f64(w1)
    out = np.empty((y.shape[0], w.shape[0]), dtype=np.float64)
    for s in range(0, y.shape[0], _ROW_CHUNK):
        z = _f64(y[s:s + _ROW_CHUNK]) @ w.T
        if b1 is not None:
            z += _f64(b1)
        out[s:s + z.shape[0]] = gelu_tanh(z)
    return out


def ffn_forward(x, modality, table_mlp, w1, w2, b1=None, b2=None, eps: float = 1e-6,
                rows=None) -> np.ndarray:
    """Feed-forward half of one DiT block for every token (or the given rows).

    [vLLM-Omni] section 3 (the DiT stage of the packed data flow): every block
    runs attention and then an MLP over the packed rows.  [H3-NFT] (adapter
    section) names its weights ff.net.0.proj and ff.net.2.  The half mirrors
    the attention half (readings): AdaLN with the MLP rows of the cached
    per-modality table (shift, scale, gate), the two projections with the
    activation between, and the gated residual:

        out = x + gate_mlp[m] * (gelu_tanh(AdaLN_mlp(x) W1^T + b1) W2^T + b2)

    table_mlp is [3 modalities][shift, scale, gate][d_model]; W2 is [d_model][d_ff].
    """
    y = adaln_modulate(x, modality, table_mlp, eps, rows=rows)
    h = ffn_up(y, w1, b1)
    return out_proj_gated(h, w2, x, modality, table_mlp, b2, rows=rows)
