"""Pins of the oracle's feed-forward half (CPU only).

The activation (tanh GELU) and the half's composition are readings; these
tests pin the oracle to them with independent implementations: torch's own
tanh-approximated GELU and layer/linear routines in float64, the pure-Python
loop version, and closed-form properties.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle import brute


def _inputs(n=10, d=16, f=48, seed=60, with_bias=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((n, d))
    table = rng.standard_normal((3, 3, d)) * 0.3
    w1 = rng.standard_normal((f, d)) * 0.3
    w2 = rng.standard_normal((d, f)) * 0.3
    b1 = rng.standard_normal(f) * 0.1 if with_bias else None
    b2 = rng.standard_normal(d) * 0.1 if with_bias else None
    mod = rng.integers(0, 3, n)
    return x, mod, table, w1, w2, b1, b2


def test_gelu_matches_torch_tanh_form():
    z = np.concatenate([np.linspace(-12.0, 12.0, 2001), [0.0, 1e-8, -1e-8, 40.0, -40.0]])
    ref = F.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(z), ref, rtol=1e-14, atol=1e-15)


def test_gelu_closed_forms():
    z = np.linspace(-6.0, 6.0, 121)
    g = oracle.gelu_tanh(z)
    # the gate 0.5 (1 + tanh(u(z))) of an odd u sums to one with its mirror
    np.testing.assert_allclose(g - oracle.gelu_tanh(-z), z, rtol=0, atol=1e-14)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    # far tails: identity on the right, zero on the left
    np.testing.assert_allclose(oracle.gelu_tanh(np.array([30.0, -30.0])), [30.0, 0.0], atol=1e-12)
    # one value by hand: z = 1 -> 0.5 (1 + tanh(sqrt(2/pi) * 1.044715))
    assert math.isclose(oracle.gelu_tanh(np.array([1.0]))[0],
                        0.5 * (1.0 + math.tanh(0.7978845608028654 * 1.044715)), rel_tol=1e-15)


def test_ffn_is_torch_composition():
    x, mod, table, w1, w2, b1, b2 = _inputs()
    t = torch.from_numpy
    ln = F.layer_norm(t(x), (x.shape[1],), eps=1e-6)
    tab = t(table)[t(mod)]
    y = ln * (1.0 + tab[:, 1]) + tab[:, 0]
    h = F.gelu(F.linear(y, t(w1), t(b1)), approximate="tanh")
    ref = t(x) + tab[:, 2] * F.linear(h, t(w2), t(b2))
    got = oracle.ffn_forward(x, mod, table, w1, w2, b1, b2)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_ffn_matches_loops():
    x, mod, table, w1, w2, b1, b2 = _inputs(n=4, d=6, f=10, seed=61)
    got = oracle.ffn_forward(x, mod, table, w1, w2, b1, b2)
    ref = brute.ffn(x.tolist(), mod.tolist(), table.tolist(), w1.tolist(), w2.tolist(),
                    b1.tolist(), b2.tolist())
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-12, atol=1e-12)


def test_ffn_zero_gate_is_identity_and_rows_select():
    x, mod, table, w1, w2, b1, b2 = _inputs(seed=62)
    table[:, 2, :] = 0.0
    np.testing.assert_array_equal(oracle.ffn_forward(x, mod, table, w1, w2, b1, b2), x)
    x, mod, table, w1, w2, b1, b2 = _inputs(seed=63)
    full = oracle.ffn_forward(x, mod, table, w1, w2, b1, b2)
    rows = np.array([7, 0, 3, 9])
    np.testing.assert_allclose(oracle.ffn_forward(x, mod, table, w1, w2, b1, b2, rows=rows),
                               full[rows], rtol=1e-13, atol=1e-13)


def test_ffn_up_sign_and_bias():
    """A single unit: h = gelu(y . w + b) picks the right sign and adds the bias once."""
    y = np.array([[1.0, -2.0, 0.5]])
    w1 = np.array([[0.5, 0.25, -1.0], [-0.5, -0.25, 1.0]])
    b1 = np.array([0.75, 0.0])
    got = oracle.ffn_up(y, w1, b1)[0]
    z0 = 1.0 * 0.5 + (-2.0) * 0.25 + 0.5 * (-1.0) + 0.75   # = 0.25
    assert math.isclose(got[0], brute.gelu_tanh(z0), rel_tol=1e-15)
    z1 = 1.0 * (-0.5) + (-2.0) * (-0.25) + 0.5 * 1.0        # = 0.5
    assert math.isclose(got[1], brute.gelu_tanh(z1), rel_tol=1e-15)
