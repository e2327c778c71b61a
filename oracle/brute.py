"""Pure-Python loop versions of every floating-point stage, for tiny inputs.

Test infrastructure only.  Lists of Python floats, the math module and
explicit loops: no NumPy.  Used to check oracle.block on N <= 16, D <= 16.
"""
from __future__ import annotations

import math
from typing import List, Sequence


def adaln(x: List[List[float]], modality, table, eps: float = 1e-6):
    out = []
    for i, row in enumerate(x):
        d = len(row)
        mu = sum(row) / d
        var = sum((v - mu) ** 2 for v in row) / d
        inv = 1.0 / math.sqrt(var + eps)
        m = modality[i]
        out.append([(row[c] - mu) * inv * (1.0 + table[m][1][c]) + table[m][0][c]
                    for c in range(d)])
    return out


def linear(x, w, b=None):
    out = []
    for row in x:
        r = []
        for j, wr in enumerate(w):
            acc = 0.0
            for c in range(len(row)):
                acc += row[c] * wr[c]
            if b is not None:
                acc += b[j]
            r.append(acc)
        out.append(r)
    return out


def rope(x, pos, n_heads, head_dim, sections, theta=10000.0):
    out = [list(r) for r in x]
    for i in range(len(x)):
        for h in range(n_heads):
            base = h * head_dim
            off = 0
            for a, s in enumerate(sections):
                for j in range(s // 2):
                    omega = theta ** (-2.0 * j / s)
                    phi = pos[i][a] * omega
                    u = x[i][base + off + 2 * j]
                    w = x[i][base + off + 2 * j + 1]
                    out[i][base + off + 2 * j] = u * math.cos(phi) - w * math.sin(phi)
                    out[i][base + off + 2 * j + 1] = u * math.sin(phi) + w * math.cos(phi)
                off += s
    return out


def attention(q, k, v, cu_seqlens, n_heads, head_dim, causal=False, scale=None):
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    n = len(q)
    out = [[0.0] * (n_heads * head_dim) for _ in range(n)]
    for s in range(len(cu_seqlens) - 1):
        a, b = cu_seqlens[s], cu_seqlens[s + 1]
        for i in range(a, b):
            for h in range(n_heads):
                base = h * head_dim
                keys = [j for j in range(a, b) if (not causal or j <= i)]
                sc = []
                for j in keys:
                    dot = 0.0
                    for c in range(head_dim):
                        dot += q[i][base + c] * k[j][base + c]
                    sc.append(dot * scale)
                mx = max(sc)
                e = [math.exp(t - mx) for t in sc]
                tot = sum(e)
                for c in range(head_dim):
                    acc = 0.0
                    for jj, j in enumerate(keys):
                        acc += e[jj] / tot * v[j][base + c]
                    out[i][base + c] = acc
    return out


def block(x, modality, pos, cu_seqlens, table, w_qkv, w_o, n_heads, head_dim,
          sections: Sequence[int], theta=10000.0, eps=1e-6, causal=False,
          b_qkv=None, b_o=None):
    d = len(x[0])
    y = adaln(x, modality, table, eps)
    qkv = linear(y, w_qkv, b_qkv)
    q = [r[:d] for r in qkv]
    k = [r[d:2 * d] for r in qkv]
    v = [r[2 * d:] for r in qkv]
    q = rope(q, pos, n_heads, head_dim, sections, theta)
    k = rope(k, pos, n_heads, head_dim, sections, theta)
    o = attention(q, k, v, cu_seqlens, n_heads, head_dim, causal)
    z = linear(o, w_o, b_o)
    return [[x[i][c] + table[modality[i]][2][c] * z[i][c] for c in range(d)]
            for i in range(len(x))]


def gelu_tanh(z: float) -> float:
    """0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    return 0.5 * z * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def ffn(x, modality, table, w1, w2, b1=None, b2=None, eps: float = 1e-6):
    """x + gate[m] * (gelu(AdaLN(x) W1^T + b1) W2^T + b2), row by row."""
    y = adaln(x, modality, table, eps)
    h = [[gelu_tanh(v) for v in row] for row in linear(y, w1, b1)]
    z = linear(h, w2, b2)
    return [[x[i][j] + table[modality[i]][2][j] * z[i][j] for j in range(len(x[i]))]
            for i in range(len(x))]


def denoise_step(z, v, modality, sigmas, anchor=None, anchor_vals=None, velocity_sign=1.0):
    """Loop version of oracle.denoise.denoise_step (None where a row is not advanced)."""
    z_next, x0 = [], []
    for i, row in enumerate(z):
        m = modality[i]
        if m not in (0, 1):
            z_next.append(list(row))
            x0.append([None] * len(row))
            continue
        if anchor is not None and anchor[i]:
            z_next.append(list(anchor_vals[i]))
            x0.append(list(anchor_vals[i]))
            continue
        s, s_next = sigmas[m]
        zr, xr = [], []
        for c in range(len(row)):
            vs = velocity_sign * v[i][c]
            xr.append(row[c] - s * vs)
            zr.append(row[c] + (s_next - s) * vs)
        z_next.append(zr)
        x0.append(xr)
    return z_next, x0


def nft_loss(v_theta, v_old, v_target, cu, reward, beta, loss_mask=None, velocity_sign=1.0,
             grad_scale=None):
    """Loop version of oracle.nft.nft_loss: (loss, mse_pos, mse_neg, grad) as lists."""
    n_s = len(cu) - 1
    scale = 1.0 / n_s if grad_scale is None else grad_scale
    n, c = len(v_theta), len(v_theta[0])
    grad = [[0.0] * c for _ in range(n)]
    loss, mp, mn = [], [], []
    for s in range(n_s):
        rows = [i for i in range(cu[s], cu[s + 1]) if loss_mask is None or loss_mask[i]]
        if not rows:
            loss.append(0.0), mp.append(0.0), mn.append(0.0)
            continue
        cnt = len(rows) * c
        sp = sn = 0.0
        for i in rows:
            for j in range(c):
                vt = velocity_sign * v_theta[i][j]
                vo = velocity_sign * v_old[i][j]
                ep = beta * vt + (1.0 - beta) * vo - v_target[i][j]
                en = (1.0 + beta) * vo - beta * vt - v_target[i][j]
                sp += ep * ep
                sn += en * en
                g = 2.0 / cnt * (reward[s] * beta * ep - (1.0 - reward[s]) * beta * en)
                grad[i][j] = scale * velocity_sign * g
        mp.append(sp / cnt)
        mn.append(sn / cnt)
        loss.append(reward[s] * mp[-1] + (1.0 - reward[s]) * mn[-1])
    return loss, mp, mn, grad
