"""FP8 (e4m3, OCP "fn" variant) quantization and FP8 projections in float64.

Test infrastructure only (see the package docstring).

[vLLM-Omni] section 5 ("Distributed Layerwise Offload") runs the active DiT
layers in FP8; the pages give no scaling recipe.  Readings:

* Format: e4m3 with 1 sign, 4 exponent (bias 7) and 3 mantissa bits,
  subnormals, no infinities, codes 0x7F / 0xFF for NaN, largest finite 448.
* Rounding: to the nearest representable value, ties to the even code
  (mantissa LSB 0); finite values beyond +-448 saturate to +-448 (beyond the
  rounding midpoint 464 the e4m3fn format has no code, so a saturating
  conversion is the plainest choice for a quantizer).
* Scaling: one float32 scale per row (per token for activations, per output
  channel for weights), scale = amax(|row|) / 448 computed in float32; a zero
  row has scale 1.  Codes are e4m3(fp32(x) * inv) with inv = 1 / scale, one
  IEEE float32 division per row and one float32 product per value: the
  precision in which the GPU takes the same decision (a multiply by the
  reciprocal, not a division per value, which would dominate the
  quantization pass).
* A projection C = (dequant(A) dequant(B)^T) with dequant(q) = decode(q) *
  scale of its row, evaluated here in float64.
* The FP8 block: the attention half and the feed-forward half of the block
  with every projection in FP8.  The operand of each projection (the AdaLN
  output, the attention output, the activated hidden state) is quantized per
  row from its float32 value; rotary embedding, attention, the activation
  and the gated residual stay in the plain oracle's float64 arithmetic.
* FP8 attention (the softmax products in FP8): q is quantized per (token,
  head) row as above; k and v with one scale per (segment, head), amax / 448
  over the segment's tokens of that head (one scale factors out of both
  products: out of s = q k^T for k, out of o = P v for v, whose sum runs over
  the keys of one segment; a request's operands do not depend on the other
  requests of its pack).  The
  scores and o = softmax(s) v are then evaluated here in float64 from the
  dequantized operands with exact probabilities; the GPU also rounds the
  probabilities to e4m3 (2^8 times their value relative to a running row
  maximum, so at most 448), which this function does not model: it moves
  each o element by at most 2^-4 sum_k P_k |v_k| / sum_k P_k (relative
  half-step of a normal e4m3 value) plus 2^-18 max_k |v_k| per key for
  probabilities in the subnormal range.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .block import (adaln_modulate, attention, ffn_up, out_proj_gated, qkv_project, rope3d)

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_decode(code: int) -> float:
    """Value of one e4m3fn code, from the format definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3_table() -> np.ndarray:
    """float64 [256]: the value of every code (NaN for the two NaN codes)."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


_POS = e4m3_table()[:0x7F]          # codes 0x00..0x7E: 0 and the positive finite values


def _apply_sign(v, code: int) -> int:
    return code | 0x80 if (v < 0 or (v == 0 and np.signbit(v))) else code


def e4m3_encode_bruteforce(x) -> np.ndarray:
    """uint8 codes of float values: nearest finite e4m3 value, ties to the even
    code, saturating beyond +-448; NaN -> 0x7F.  A search over the 127
    non-negative finite values, one value at a time (for tiny inputs)."""
    a = np.asarray(x, dtype=np.float64)
    flat = a.ravel()
    out = np.empty(flat.size, dtype=np.uint8)
    for i, v in enumerate(flat):
        if np.isnan(v):
            out[i] = E4M3_NAN
            continue
        mag = min(abs(v), E4M3_MAX)
        d = np.abs(_POS - mag)
        best = np.flatnonzero(d == d.min())
        code = int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])
        out[i] = _apply_sign(v, code)
    return out.reshape(a.shape)


def e4m3_encode(x) -> np.ndarray:
    """The same rounding as e4m3_encode_bruteforce, vectorised: the two finite
    neighbours of |x| (clamped to 448) in the sorted value table, the nearer
    one, the even code on a tie."""
    a = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(a), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, mag, side="left"), 0, _POS.size - 1)
    lo = np.clip(hi - 1, 0, _POS.size - 1)
    d_lo, d_hi = mag - _POS[lo], _POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = (a < 0) | ((a == 0) & np.signbit(a))
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(a), np.uint8(E4M3_NAN), code).astype(np.uint8)


def row_scales(x) -> np.ndarray:
    """float32 per-row scales amax / 448 (1 for an all-zero row), computed in float32."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s[amax == 0] = np.float32(1.0)
    return s


def quantize_rows(x):
    """Per-row e4m3 quantization: (codes uint8 [N][D], scales float32 [N])."""
    x32 = np.asarray(x, dtype=np.float32)
    s = row_scales(x32)
    inv = (np.float32(1.0) / s).astype(np.float32)   # IEEE float32 division, once per row
    q = (x32 * inv[:, None]).astype(np.float32)      # one float32 rounding per value
    return e4m3_encode(q), s


def dequantize_rows(codes, scales) -> np.ndarray:
    """float64 decode(code) * scale of the row."""
    return e4m3_table()[np.asarray(codes, dtype=np.uint8)] * np.asarray(scales, np.float64)[:, None]


def linear_fp8(a_codes, a_scales, w_codes, w_scales, bias=None) -> np.ndarray:
    """float64 C = dequant(A) dequant(W)^T (+ bias): A [N][K], W [F][K] ([out][in])."""
    c = dequantize_rows(a_codes, a_scales) @ dequantize_rows(w_codes, w_scales).T
    if bias is not None:
        c = c + np.asarray(bias, np.float64)[None, :]
    return c


# ---------------------------------------------------------------------------
# FP8 block
# ---------------------------------------------------------------------------

def adaln_modulate_fp8(x, modality, table, eps: float = 1e-6, rows=None):
    """AdaLN (oracle.block.adaln_modulate) quantized per row: (codes, scales)
    of the float32 value of its output."""
    return quantize_rows(adaln_modulate(x, modality, table, eps, rows=rows))


def block_forward_fp8(x, modality, pos, cu_seqlens, table, wq_codes, wq_scales, wo_codes,
                      wo_scales, *, n_heads: int, head_dim: int, sections: Sequence[int],
                      theta: float = 10000.0, eps: float = 1e-6, causal: bool = False,
                      scale: Optional[float] = None, b_qkv=None, b_o=None,
                      rows=None, fp8_attention: bool = False) -> Dict[str, np.ndarray]:
    """The attention half of the block (oracle.block.block_forward) with both
    projections in FP8: the AdaLN output and the attention output are
    quantized per row, W_qkv [3D][D] and W_o [D][D] are given as per-row codes
    and scales.  With ``fp8_attention`` the attention is attention_fp8 of the
    rotated q, k and v.  Returns y_codes, y_scales, q, k, v, q_rot, k_rot, o,
    o_codes, o_scales and out (float64); with ``rows``, o, its codes and out
    hold those rows only, and q, q_rot are filled only at those rows.
    """
    x = np.asarray(x)
    n, d = x.shape
    yc, ys = adaln_modulate_fp8(x, modality, table, eps)
    y = dequantize_rows(yc, ys)
    w = dequantize_rows(wq_codes, wq_scales)
    bias = [None] * 3 if b_qkv is None else [np.asarray(b_qkv)[i * d:(i + 1) * d] for i in range(3)]
    k = qkv_project(y, w[d:2 * d], bias[1])
    v = qkv_project(y, w[2 * d:], bias[2])
    k_rot = rope3d(k, pos, n_heads, head_dim, sections, theta)
    idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    q = np.zeros((n, d))
    q[idx] = qkv_project(y[idx], w[:d], bias[0])
    q_rot = np.zeros((n, d))
    q_rot[idx] = rope3d(q[idx], np.asarray(pos)[idx], n_heads, head_dim, sections, theta)
    if fp8_attention:
        o = attention_fp8(q_rot, k_rot, v, cu_seqlens, n_heads, head_dim, causal, scale, rows)["o"]
    else:
        o = attention(q_rot, k_rot, v, cu_seqlens, n_heads, head_dim, causal, scale, rows)
    oc, os_ = quantize_rows(o)
    out = out_proj_gated(dequantize_rows(oc, os_), dequantize_rows(wo_codes, wo_scales), x,
                         modality, table, b_o, rows)
    return dict(y_codes=yc, y_scales=ys, q=q, k=k, v=v, q_rot=q_rot, k_rot=k_rot, o=o,
                o_codes=oc, o_scales=os_, out=out)


def ffn_forward_fp8(x, modality, table_mlp, w1_codes, w1_scales, w2_codes, w2_scales,
                    b1=None, b2=None, eps: float = 1e-6, rows=None) -> Dict[str, np.ndarray]:
    """The feed-forward half (oracle.block.ffn_forward) with both projections
    in FP8: the AdaLN output and the activated hidden state h are quantized
    per row.  Returns y_codes, y_scales, h, h_codes, h_scales and out."""
    yc, ys = adaln_modulate_fp8(x, modality, table_mlp, eps, rows=rows)
    h = ffn_up(dequantize_rows(yc, ys), dequantize_rows(w1_codes, w1_scales), b1)
    hc, hs = quantize_rows(h)
    out = out_proj_gated(dequantize_rows(hc, hs), dequantize_rows(w2_codes, w2_scales), x,
                         modality, table_mlp, b2, rows=rows)
    return dict(y_codes=yc, y_scales=ys, h=h, h_codes=hc, h_scales=hs, out=out)


# ---------------------------------------------------------------------------
# FP8 attention
# ---------------------------------------------------------------------------

def quantize_tensor(x):
    """One float32 scale for the whole array (amax / 448, 1 for an all-zero
    array) and the e4m3 codes of every value: the per-row recipe applied to
    the array as one row."""
    x32 = np.asarray(x, dtype=np.float32)
    codes, s = quantize_rows(x32.reshape(1, -1))
    return codes.reshape(x32.shape), np.float32(s[0])


def attention_fp8_operands(q, k, v, n_heads: int, head_dim: int,
                           cu_seqlens=None) -> Dict[str, np.ndarray]:
    """Codes and scales of the FP8 attention operands (q, k, v: [N][H*Dh]):
    q_codes [N][H*Dh] with q_scales [N][H] (one per token and head), k_codes /
    v_codes [N][H*Dh] with k_scales / v_scales [S][H], one per (cu_seqlens
    segment, head), the segment's rows of the head quantized as one tensor
    (quantize_tensor; an empty segment keeps scale 1).  Reading: the requests
    of a pack are independent ([vLLM-Omni] section 3: every sub-sequence
    normalises over its own keys only), so a request's quantization depends on
    its own values, not on what else was packed with it.  Without cu_seqlens
    the rows form one segment.  The dict also carries the segments."""
    q = np.asarray(q, dtype=np.float32)
    n = q.shape[0]
    cu = [0, n] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    qc, qs = quantize_rows(q.reshape(n * n_heads, head_dim))
    out = dict(q_codes=qc.reshape(n, n_heads * head_dim), q_scales=qs.reshape(n, n_heads),
               cu_seqlens=np.asarray(cu, dtype=np.int64))
    for name, t in (("k", k), ("v", v)):
        t = np.asarray(t, dtype=np.float32)
        codes = np.zeros(t.shape, dtype=np.uint8)
        scales = np.ones((len(cu) - 1, n_heads), dtype=np.float32)
        for s, (a, b) in enumerate(zip(cu, cu[1:])):
            if b <= a:
                continue
            for h in range(n_heads):
                cols = slice(h * head_dim, (h + 1) * head_dim)
                codes[a:b, cols], scales[s, h] = quantize_tensor(t[a:b, cols])
        out[name + "_codes"], out[name + "_scales"] = codes, scales
    return out


def dequantize_attention_operands(ops: Dict[str, np.ndarray], n_heads: int, head_dim: int):
    """float64 q, k, v [N][H*Dh] from attention_fp8_operands' codes and scales
    (k's and v's scale taken from each row's segment)."""
    tab = e4m3_table()
    qs = np.repeat(np.asarray(ops["q_scales"], np.float64), head_dim, axis=1)
    q = tab[ops["q_codes"]] * qs
    cu = [int(c) for c in ops["cu_seqlens"]]
    n = q.shape[0]
    seg = np.zeros(n, dtype=np.int64)
    for s, (a, b) in enumerate(zip(cu, cu[1:])):
        seg[a:b] = s
    ks = np.repeat(np.asarray(ops["k_scales"], np.float64), head_dim, axis=1)[seg]
    vs = np.repeat(np.asarray(ops["v_scales"], np.float64), head_dim, axis=1)[seg]
    return q, tab[ops["k_codes"]] * ks, tab[ops["v_codes"]] * vs


def attention_fp8(q, k, v, cu_seqlens, n_heads: int, head_dim: int, causal: bool = False,
                  scale: Optional[float] = None, rows=None) -> Dict[str, np.ndarray]:
    """Softmax attention (oracle.block.attention) of the dequantized FP8
    operands with exact probabilities.  Returns the operands' codes and
    scales, o (float64 [rows][H*Dh]) and o_abs, the same attention of |v|
    (sum_k P_k |v_k| / sum_k P_k, the weight of the probability-rounding bound)."""
    ops = attention_fp8_operands(q, k, v, n_heads, head_dim, cu_seqlens)
    qd, kd, vd = dequantize_attention_operands(ops, n_heads, head_dim)
    o = attention(qd, kd, vd, cu_seqlens, n_heads, head_dim, causal, scale, rows)
    o_abs = attention(qd, kd, np.abs(vd), cu_seqlens, n_heads, head_dim, causal, scale, rows)
    return dict(o=o, o_abs=o_abs, **ops)
