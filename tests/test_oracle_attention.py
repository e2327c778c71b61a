"""Pins of the oracle's packed softmax attention (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import brute
import synth

H, DH = 2, 8


def _qkv(n, seed, std=1.0):
    return tuple(synth.normal_array((n, H * DH), seed + i, std).astype(np.float64)
                 for i in range(3))


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one_and_zero_off_mask(causal):
    cu = [0, 5, 13, 20]
    q, k, _ = _qkv(20, 1, 2.0)
    P = oracle.attention_probs(q, k, cu, H, DH, causal)
    np.testing.assert_allclose(P.sum(axis=2), 1.0, rtol=0, atol=1e-12)
    for h in range(H):
        for i in range(20):
            for j in range(20):
                same = any(a <= i < b and a <= j < b for a, b in zip(cu, cu[1:]))
                if not same or (causal and j > i):
                    assert P[h, i, j] == 0.0


def test_page_cu_seqlens_example():
    with open(os.path.join(os.path.dirname(__file__), "golden", "cu_seqlens_example.json")) as f:
        g = json.load(f)
    for cu in (g["cu_two"], g["cu_three"]):
        n = cu[-1]
        q, k, _ = _qkv(n, 7)
        P = oracle.attention_probs(q, k, cu, H, DH)
        lo, hi = g["visible_keys"]
        row = P[:, g["query"], :]
        assert np.all(row[:, lo:hi + 1] > 0)
        assert np.all(row[:, :lo] == 0) and np.all(row[:, hi + 1:] == 0)


def test_constant_value_column_gives_one():
    cu = [0, 9, 16]
    q, k, v = _qkv(16, 3)
    v[:, 5] = 1.0
    o = oracle.attention(q, k, v, cu, H, DH)
    np.testing.assert_allclose(o[:, 5], 1.0, rtol=0, atol=1e-13)


def test_single_visible_key_returns_its_value():
    cu = [0, 6, 11]
    q, k, v = _qkv(11, 4)
    o = oracle.attention(q, k, v, cu, H, DH, causal=True)
    for a in cu[:-1]:
        np.testing.assert_allclose(o[a], v[a], rtol=0, atol=1e-14)


def test_equal_keys_give_mean_of_values():
    cu = [0, 7, 12]
    q, k, v = _qkv(12, 5)
    k[:] = k[0]
    o = oracle.attention(q, k, v, cu, H, DH)
    for a, b in zip(cu, cu[1:]):
        np.testing.assert_allclose(o[a:b], np.broadcast_to(v[a:b].mean(0), (b - a, H * DH)),
                                   rtol=0, atol=1e-13)


def test_packed_equals_per_segment_runs():
    cu = [0, 4, 15, 23]
    q, k, v = _qkv(23, 6)
    o = oracle.attention(q, k, v, cu, H, DH)
    for a, b in zip(cu, cu[1:]):
        seg = oracle.attention(q[a:b], k[a:b], v[a:b], [0, b - a], H, DH)
        np.testing.assert_allclose(o[a:b], seg, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    cu = [0, 13, 30, 31, 40]
    q, k, v = _qkv(40, 8, 1.5)
    o = oracle.attention(q, k, v, cu, H, DH, causal)
    for a, b in zip(cu, cu[1:]):
        def heads(t):
            return torch.from_numpy(t[a:b]).reshape(b - a, H, DH).transpose(0, 1)
        ref = F.scaled_dot_product_attention(heads(q), heads(k), heads(v), is_causal=causal)
        ref = ref.transpose(0, 1).reshape(b - a, H * DH).numpy()
        np.testing.assert_allclose(o[a:b], ref, rtol=0, atol=1e-12)


def test_custom_scale_matches_sdpa():
    q, k, v = _qkv(10, 9)
    o = oracle.attention(q, k, v, [0, 10], H, DH, scale=0.37)
    def heads(t):
        return torch.from_numpy(t).reshape(10, H, DH).transpose(0, 1)
    ref = F.scaled_dot_product_attention(heads(q), heads(k), heads(v), scale=0.37)
    np.testing.assert_allclose(o, ref.transpose(0, 1).reshape(10, H * DH).numpy(), atol=1e-12)


def test_rows_subset_matches_full():
    cu = [0, 8, 19]
    q, k, v = _qkv(19, 10)
    rows = [18, 0, 7, 8]
    for causal in (False, True):
        np.testing.assert_array_equal(oracle.attention(q, k, v, cu, H, DH, causal, rows=rows),
                                      oracle.attention(q, k, v, cu, H, DH, causal)[rows])


def test_empty_segment_allowed():
    cu = [0, 5, 5, 9]
    q, k, v = _qkv(9, 11)
    o = oracle.attention(q, k, v, cu, H, DH)
    np.testing.assert_allclose(o[5:], oracle.attention(q[5:], k[5:], v[5:], [0, 4], H, DH),
                               atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_agreement(causal):
    cu = [0, 3, 8]
    q, k, v = _qkv(8, 12, 2.0)
    o = oracle.attention(q, k, v, cu, H, DH, causal)
    ob = brute.attention(q.tolist(), k.tolist(), v.tolist(), cu, H, DH, causal)
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
