"""Float64 backward pass of the attention half of the block.

Test infrastructure only (see the package docstring).

[H3-NFT] section "DiffusionNFT: Skipping the Reverse Chain Entirely" (the
training objective is a flow-matching regression on the DiT's velocity) and
[VeRL-Omni] section 4 (the loss and its attraction / repulsion gradients)
need the gradients of the block's parameters and input; the pages print no
backward pass.  It is the chain rule through the forward definitions of
``oracle.block``, written out stage by stage:

    out = x + gate[m] * z,        z = o W_o^T + b_o
    o   = softmax(q' k'^T * scale) v   inside each segment (causal optional)
    q'  = R q,  k' = R k              (R: the 3D rotary rotation, orthogonal)
    [q | k | v] = y W_qkv^T + b_qkv
    y   = xhat (1 + scale[m]) + shift[m],   xhat = (x - mean) / sqrt(var + eps)

Given the upstream gradient g = dL/d(out), the functions return dL/d(every
input): x, the three table rows of every modality, W_qkv, b_qkv, W_o, b_o;
``ffn_backward`` does the same for the feed-forward half (W1, b1, W2, b2 and
the MLP table rows), through the tanh-form GELU of oracle.block.gelu_tanh.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .block import (_f64, _probs, adaln_modulate, attention, gelu_tanh, qkv_project, rope3d,
                    rope_frequencies)


def attention_backward(q, k, v, do, cu_seqlens, n_heads: int, head_dim: int,
                       causal: bool = False, scale: Optional[float] = None):
    """(dq, dk, dv) of o = softmax(q k^T scale) v per segment and head.

    With P the softmax weights: dv = P^T do, dP = do v^T,
    dS = P * (dP - rowsum(dP * P)), dq = scale dS k, dk = scale dS^T q.
    (rowsum(dP * P) equals rowsum(do * o).)
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    sc = 1.0 / np.sqrt(head_dim) if scale is None else float(scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    cu = [int(c) for c in cu_seqlens]
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b <= a:
            continue
        for h in range(n_heads):
            cols = slice(h * head_dim, (h + 1) * head_dim)
            qh, kh, vh, doh = q[a:b, cols], k[a:b, cols], v[a:b, cols], do[a:b, cols]
            P = _probs(qh, kh, np.arange(a, b), a, causal, sc)
            dv[a:b, cols] = P.T @ doh
            dP = doh @ vh.T
            dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
            dq[a:b, cols] = sc * (dS @ kh)
            dk[a:b, cols] = sc * (dS.T @ qh)
    return dq, dk, dv


def attention_lse(q, k, cu_seqlens, n_heads: int, head_dim: int, causal: bool = False,
                  scale: Optional[float] = None, rows=None) -> np.ndarray:
    """lse[h][i] = log sum_j exp(q_i k_j^T scale) over row i's keys (its segment, j <= i
    when causal), float64 [n_heads][len(rows)] (every row when rows is None)."""
    q, k = _f64(q), _f64(k)
    n = q.shape[0]
    sc = 1.0 / np.sqrt(head_dim) if scale is None else float(scale)
    idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    cu = [int(c) for c in cu_seqlens]
    seg = np.searchsorted(np.asarray(cu[1:]), idx, side="right")
    out = np.empty((n_heads, idx.size))
    for s in np.unique(seg):
        sel = np.flatnonzero(seg == s)
        a, b = cu[s], cu[s + 1]
        qi = idx[sel]
        for h in range(n_heads):
            cols = slice(h * head_dim, (h + 1) * head_dim)
            z = (q[qi, cols] @ k[a:b, cols].T) * sc
            if causal:
                z = np.where(np.arange(a, b)[None, :] <= qi[:, None], z, -np.inf)
            m = z.max(axis=1, keepdims=True)
            out[h, sel] = m[:, 0] + np.log(np.sum(np.exp(z - m), axis=1))
    return out


def attention_backward_rows(q, k, v, do, cu_seqlens, n_heads: int, head_dim: int, rows,
                            causal: bool = False, scale: Optional[float] = None) -> np.ndarray:
    """dq at the given query rows only (each needs its own softmax row, not the
    others'): dq_i = scale sum_j P_ij (do_i v_j - do_i o_i) k_j."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    sc = 1.0 / np.sqrt(head_dim) if scale is None else float(scale)
    idx = np.asarray(rows, dtype=np.int64)
    cu = [int(c) for c in cu_seqlens]
    seg = np.searchsorted(np.asarray(cu[1:]), idx, side="right")
    out = np.zeros((idx.size, q.shape[1]))
    for t, (i, sgi) in enumerate(zip(idx, seg)):
        a, b = cu[sgi], cu[sgi + 1]
        for h in range(n_heads):
            cols = slice(h * head_dim, (h + 1) * head_dim)
            P = _probs(q[i:i + 1, cols], k[a:b, cols], np.array([i]), a, causal, sc)[0]
            o_i = P @ v[a:b, cols]
            dP = v[a:b, cols] @ do[i, cols]
            dS = P * (dP - do[i, cols] @ o_i)
            out[t, cols] = sc * (dS @ k[a:b, cols])
    return out


def rope3d_backward(g, pos, n_heads: int, head_dim: int, sections: Sequence[int],
                    theta: float = 10000.0) -> np.ndarray:
    """Gradient through oracle.block.rope3d: the transposed rotation R^T g.

    Each pair (u, w) -> (u c - w s, u s + w c) has the transpose
    (gu, gw) -> (gu c + gw s, -gu s + gw c), the rotation by the negated angle.
    """
    g = _f64(g)
    n = g.shape[0]
    p = np.asarray(pos, dtype=np.int64)
    gr = g.reshape(n, n_heads, head_dim)
    out = gr.copy()
    off = 0
    for axis, s in enumerate(sections):
        phi = p[:, axis].astype(np.float64)[:, None] * rope_frequencies(s, theta)
        c = np.cos(phi)[:, None, :]
        sn = np.sin(phi)[:, None, :]
        gu = gr[:, :, off:off + s:2]
        gw = gr[:, :, off + 1:off + s:2]
        out[:, :, off:off + s:2] = gu * c + gw * sn
        out[:, :, off + 1:off + s:2] = -gu * sn + gw * c
        off += s
    return out.reshape(n, n_heads * head_dim)


def adaln_backward(x, modality, table, dy, eps: float = 1e-6):
    """(dx, dshift [3][D], dscale [3][D]) through y = xhat (1 + scale[m]) + shift[m].

    dshift[m] = sum of dy over rows of modality m, dscale[m] = sum of dy * xhat;
    with dxhat = dy (1 + scale[m]) and r = 1 / sqrt(var + eps),
    dx = r (dxhat - mean(dxhat) - xhat mean(dxhat * xhat)) (biased variance).
    """
    x, dy, tab = _f64(x), _f64(dy), _f64(table)
    mod = np.asarray(modality, dtype=np.int64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    r = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * r
    dxhat = dy * (1.0 + tab[mod, 1, :])
    dx = r * (dxhat - dxhat.mean(axis=1, keepdims=True)
              - xhat * (dxhat * xhat).mean(axis=1, keepdims=True))
    d = x.shape[1]
    dshift, dscale = np.zeros((3, d)), np.zeros((3, d))
    for m in range(3):
        sel = mod == m
        dshift[m] = dy[sel].sum(axis=0)
        dscale[m] = (dy[sel] * xhat[sel]).sum(axis=0)
    return dx, dshift, dscale


def block_backward(x, modality, pos, cu_seqlens, table, w_qkv, w_o, dout, *,
                   n_heads: int, head_dim: int, sections: Sequence[int],
                   theta: float = 10000.0, eps: float = 1e-6, causal: bool = False,
                   scale: Optional[float] = None, b_qkv=None, b_o=None) -> Dict[str, np.ndarray]:
    """Gradients of sum(dout * out) for the attention half (oracle.block.block_forward).

    Returns dx [N][D], dtable [3][3][D] (shift, scale, gate rows), dw_qkv [3D][D],
    db_qkv [3D], dw_o [D][D], db_o [D], and the intermediate gradients dz (of
    the branch before the gate), do, dq_rot, dk_rot, dv, dqkv and dy.
    """
    x, dout = _f64(x), _f64(dout)
    n, d = x.shape
    mod = np.asarray(modality, dtype=np.int64)
    tab = _f64(table)
    w, wo = _f64(w_qkv), _f64(w_o)
    # forward stages
    y = adaln_modulate(x, mod, tab, eps)
    qkv = qkv_project(y, w, b_qkv)
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    q_rot = rope3d(q, pos, n_heads, head_dim, sections, theta)
    k_rot = rope3d(k, pos, n_heads, head_dim, sections, theta)
    o = attention(q_rot, k_rot, v, cu_seqlens, n_heads, head_dim, causal, scale)
    z = o @ wo.T
    if b_o is not None:
        z = z + _f64(b_o)
    # backward, last stage first
    gate = tab[mod, 2, :]
    dgate = np.zeros((3, d))
    for m in range(3):
        sel = mod == m
        dgate[m] = (dout[sel] * z[sel]).sum(axis=0)
    dz = gate * dout
    dw_o = dz.T @ o
    db_o = dz.sum(axis=0)
    do = dz @ wo
    dq_rot, dk_rot, dv = attention_backward(q_rot, k_rot, v, do, cu_seqlens, n_heads, head_dim,
                                            causal, scale)
    dq = rope3d_backward(dq_rot, pos, n_heads, head_dim, sections, theta)
    dk = rope3d_backward(dk_rot, pos, n_heads, head_dim, sections, theta)
    dqkv = np.concatenate([dq, dk, dv], axis=1)
    dw_qkv = dqkv.T @ y
    db_qkv = dqkv.sum(axis=0)
    dy = dqkv @ w
    dx_ln, dshift, dscale = adaln_backward(x, mod, tab, dy, eps)
    dtable = np.stack([dshift, dscale, dgate], axis=1)
    return dict(dx=dout + dx_ln, dtable=dtable, dw_qkv=dw_qkv, db_qkv=db_qkv, dw_o=dw_o,
                db_o=db_o, dz=dz, do=do, dq_rot=dq_rot, dk_rot=dk_rot, dv=dv, dqkv=dqkv, dy=dy,
                o=o, q_rot=q_rot, k_rot=k_rot, v=v, y=y, z=z)


def gelu_tanh_grad(z) -> np.ndarray:
    """d/dz of oracle.block.gelu_tanh: with u = c (z + 0.044715 z^3), c = sqrt(2/pi),
    0.5 (1 + tanh u) + 0.5 z (1 - tanh^2 u) c (1 + 3 * 0.044715 z^2)."""
    z = _f64(z)
    c = np.sqrt(2.0 / np.pi)
    t = np.tanh(c * (z + 0.044715 * z ** 3))
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * z * z)


def ffn_backward(x, modality, table_mlp, w1, w2, dout, b1=None, b2=None,
                 eps: float = 1e-6) -> Dict[str, np.ndarray]:
    """Gradients of sum(dout * out) for the feed-forward half (oracle.block.ffn_forward):

        out = x + gate[m] * z,  z = h W2^T + b2,  h = gelu_tanh(a),  a = y W1^T + b1,
        y = AdaLN(x) with the MLP table rows.

    Returns dx, dtable [3][3][D], dw1 [F][D], db1 [F], dw2 [D][F], db2 [D] and the
    intermediate gradients dz, dh, da, dy.
    """
    x, dout = _f64(x), _f64(dout)
    d = x.shape[1]
    mod = np.asarray(modality, dtype=np.int64)
    tab = _f64(table_mlp)
    W1, W2 = _f64(w1), _f64(w2)
    y = adaln_modulate(x, mod, tab, eps)
    a = y @ W1.T
    if b1 is not None:
        a = a + _f64(b1)
    h = gelu_tanh(a)
    z = h @ W2.T
    if b2 is not None:
        z = z + _f64(b2)
    dgate = np.zeros((3, d))
    for m in range(3):
        sel = mod == m
        dgate[m] = (dout[sel] * z[sel]).sum(axis=0)
    dz = tab[mod, 2, :] * dout
    dw2 = dz.T @ h
    db2 = dz.sum(axis=0)
    dh = dz @ W2
    da = dh * gelu_tanh_grad(a)
    dw1 = da.T @ y
    db1 = da.sum(axis=0)
    dy = da @ W1
    dx_ln, dshift, dscale = adaln_backward(x, mod, tab, dy, eps)
    dtable = np.stack([dshift, dscale, dgate], axis=1)
    return dict(dx=dout + dx_ln, dtable=dtable, dw1=dw1, db1=db1, dw2=dw2, db2=db2, dz=dz,
                dh=dh, da=da, dy=dy)
