"""Pins of the oracle's backward pass of the attention half (CPU only).

The backward pass is the chain rule through the forward definitions; it is
pinned by (a) central differences of the oracle's own float64 forward along
random directions (no derivative is retyped), (b) torch autograd in float64
(a library) through torch's layer norm and scaled-dot-product attention, (c)
the adjoint and inverse identities of the rotation, and (d) special cases.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def _setup(n=14, d=16, h=2, seed=80, bias=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((n, d)) * 1.5 + 0.3
    table = rng.standard_normal((3, 3, d)) * 0.3
    w_qkv = rng.standard_normal((3 * d, d)) * 0.4
    w_o = rng.standard_normal((d, d)) * 0.4
    b_qkv = rng.standard_normal(3 * d) * 0.1 if bias else None
    b_o = rng.standard_normal(d) * 0.1 if bias else None
    mod = rng.integers(0, 3, n)
    pos = rng.integers(0, 7, (n, 3))
    dout = rng.standard_normal((n, d))
    return x, table, w_qkv, w_o, b_qkv, b_o, mod, pos, dout


KW = dict(n_heads=2, head_dim=8, sections=(2, 2, 4), theta=50.0)


def _objective(x, table, w_qkv, w_o, b_qkv, b_o, mod, pos, dout, cu, causal):
    out = oracle.block_forward(x, mod, pos, cu, table, w_qkv, w_o, b_qkv=b_qkv, b_o=b_o,
                               causal=causal, **KW)["out"]
    return float(np.sum(dout * out))


@pytest.mark.parametrize("causal", [False, True])
def test_block_backward_directional_derivatives(causal):
    """<grad, delta> equals the central difference of sum(dout * out) along delta for every
    input group (x, table, W_qkv, b_qkv, W_o, b_o)."""
    x, table, w_qkv, w_o, b_qkv, b_o, mod, pos, dout = _setup()
    cu = [0, 6, 14]
    g = oracle.block_backward(x, mod, pos, cu, table, w_qkv, w_o, dout, b_qkv=b_qkv, b_o=b_o,
                              causal=causal, **KW)
    args = dict(x=x, table=table, w_qkv=w_qkv, w_o=w_o, b_qkv=b_qkv, b_o=b_o)
    grads = dict(x=g["dx"], table=g["dtable"], w_qkv=g["dw_qkv"], w_o=g["dw_o"],
                 b_qkv=g["db_qkv"], b_o=g["db_o"])
    rng = np.random.Generator(np.random.PCG64(81))
    eps = 1e-5
    for name, val in args.items():
        delta = rng.standard_normal(val.shape)
        plus = dict(args, **{name: val + eps * delta})
        minus = dict(args, **{name: val - eps * delta})
        fd = (_objective(**plus, mod=mod, pos=pos, dout=dout, cu=cu, causal=causal)
              - _objective(**minus, mod=mod, pos=pos, dout=dout, cu=cu, causal=causal)) / (2 * eps)
        an = float(np.sum(grads[name] * delta))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_attention_backward_matches_torch_autograd():
    """torch's scaled_dot_product_attention (float64, block-diagonal / causal masks)
    differentiated by autograd gives the same dq, dk, dv."""
    rng = np.random.Generator(np.random.PCG64(82))
    n, H, Dh = 23, 3, 8
    q, k, v, do = (rng.standard_normal((n, H * Dh)) for _ in range(4))
    cu = [0, 9, 9, 23]
    for causal in (False, True):
        dq, dk, dv = oracle.attention_backward(q, k, v, do, cu, H, Dh, causal=causal, scale=0.4)
        tq, tk, tv = (torch.tensor(a.reshape(n, H, Dh).transpose(1, 0, 2), requires_grad=True)
                      for a in (q, k, v))
        seg = np.searchsorted(np.asarray(cu[1:]), np.arange(n), side="right")
        mask = seg[:, None] == seg[None, :]
        if causal:
            mask &= np.arange(n)[None, :] <= np.arange(n)[:, None]
        o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(mask), scale=0.4)
        o.backward(torch.tensor(do.reshape(n, H, Dh).transpose(1, 0, 2).copy()))
        for got, t in ((dq, tq), (dk, tk), (dv, tv)):
            ref = t.grad.numpy().transpose(1, 0, 2).reshape(n, H * Dh)
            np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_adaln_backward_matches_torch_autograd():
    x, table, *_ , mod, _, dout = _setup(n=11, d=24, seed=83)
    dx, dsh, dsc = oracle.adaln_backward(x, mod, table, dout, eps=1e-6)
    tx = torch.tensor(x, requires_grad=True)
    tt = torch.tensor(table, requires_grad=True)
    m = torch.tensor(mod)
    y = F.layer_norm(tx, (x.shape[1],), eps=1e-6) * (1 + tt[m, 1]) + tt[m, 0]
    y.backward(torch.tensor(dout))
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dsh, tt.grad[:, 0].numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dsc, tt.grad[:, 1].numpy(), rtol=1e-10, atol=1e-12)
    assert np.all(tt.grad[:, 2].numpy() == 0)


def test_rope_backward_is_the_adjoint_and_the_inverse():
    rng = np.random.Generator(np.random.PCG64(84))
    n, H, Dh, sec = 9, 2, 16, (4, 6, 6)
    pos = rng.integers(0, 50, (n, 3))
    a, b = rng.standard_normal((n, H * Dh)), rng.standard_normal((n, H * Dh))
    ra = oracle.rope3d(a, pos, H, Dh, sec, 100.0)
    rb_t = oracle.rope3d_backward(b, pos, H, Dh, sec, 100.0)
    assert abs(np.sum(ra * b) - np.sum(a * rb_t)) <= 1e-10 * np.abs(ra * b).sum()
    np.testing.assert_allclose(oracle.rope3d(rb_t, pos, H, Dh, sec, 100.0), b, atol=1e-12)
    # position 0 leaves the gradient as it is
    np.testing.assert_array_equal(oracle.rope3d_backward(b, np.zeros((n, 3), int), H, Dh, sec),
                                  b)


def test_zero_gate_passes_the_gradient_straight_through():
    """A zero gate cuts the branch: dx = dout exactly, every weight gradient and the shift
    and scale rows vanish, and the gate row collects dout * z per modality."""
    x, table, w_qkv, w_o, b_qkv, b_o, mod, pos, dout = _setup(seed=85)
    table[:, 2, :] = 0.0
    g = oracle.block_backward(x, mod, pos, [0, 14], table, w_qkv, w_o, dout, b_qkv=b_qkv,
                              b_o=b_o, **KW)
    np.testing.assert_array_equal(g["dx"], dout)
    for key in ("dw_qkv", "db_qkv", "dw_o", "db_o"):
        assert not np.any(g[key]), key
    assert not np.any(g["dtable"][:, :2, :])
    for m in range(3):
        np.testing.assert_allclose(g["dtable"][m, 2], (dout * g["z"])[mod == m].sum(0))


def test_value_gradient_of_a_single_key_segment():
    """A one-token segment attends only to itself: o = v, so dv = do and dq = dk = 0."""
    rng = np.random.Generator(np.random.PCG64(86))
    q, k, v, do = (rng.standard_normal((5, 16)) for _ in range(4))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, [0, 1, 5], 2, 8)
    np.testing.assert_allclose(dv[0], do[0], atol=1e-15)
    assert not np.any(dq[0]) and not np.any(dk[0])


def test_attention_lse_matches_torch_logsumexp_and_closed_form():
    rng = np.random.Generator(np.random.PCG64(87))
    n, H, Dh = 17, 2, 8
    q, k = rng.standard_normal((n, H * Dh)), rng.standard_normal((n, H * Dh))
    cu = [0, 7, 17]
    for causal in (False, True):
        lse = oracle.attention_lse(q, k, cu, H, Dh, causal=causal, scale=0.3)
        for i in range(n):
            a = 0 if i < 7 else 7
            b = i + 1 if causal else (7 if i < 7 else 17)
            for h in range(H):
                c = slice(h * Dh, (h + 1) * Dh)
                ref = torch.logsumexp(torch.tensor(k[a:b, c] @ q[i, c] * 0.3), 0).item()
                assert abs(lse[h, i] - ref) <= 1e-12 * max(1, abs(ref))
    # equal keys: every score is the same, lse = s + log(segment length)
    kk = np.tile(k[:1], (n, 1))
    lse = oracle.attention_lse(q, kk, [0, n], H, Dh)
    s0 = np.array([[q[i, h * Dh:(h + 1) * Dh] @ k[0, h * Dh:(h + 1) * Dh] / np.sqrt(Dh)
                    for i in range(n)] for h in range(H)])
    np.testing.assert_allclose(lse, s0 + np.log(n), rtol=1e-12, atol=1e-12)
    # a subset of rows equals those rows of the whole
    np.testing.assert_allclose(oracle.attention_lse(q, k, cu, H, Dh, rows=[3, 16]),
                               oracle.attention_lse(q, k, cu, H, Dh)[:, [3, 16]])


def test_attention_backward_rows_equals_the_full_backward():
    rng = np.random.Generator(np.random.PCG64(88))
    q, k, v, do = (rng.standard_normal((19, 16)) for _ in range(4))
    for causal in (False, True):
        dq, _, _ = oracle.attention_backward(q, k, v, do, [0, 8, 19], 2, 8, causal=causal)
        rows = [0, 7, 8, 18]
        got = oracle.attention_backward_rows(q, k, v, do, [0, 8, 19], 2, 8, rows, causal=causal)
        np.testing.assert_allclose(got, dq[rows], rtol=1e-12, atol=1e-13)


def test_attention_gradient_column_sums():
    """Shift invariance of the softmax over keys: the key gradients of a segment sum
    to zero per head and dimension; the value gradients sum to the output gradients."""
    rng = np.random.Generator(np.random.PCG64(89))
    q, k, v, do = (rng.standard_normal((21, 16)) for _ in range(4))
    for causal in (False, True):
        _, dk, dv = oracle.attention_backward(q, k, v, do, [0, 9, 21], 2, 8, causal=causal)
        for a, b in ((0, 9), (9, 21)):
            np.testing.assert_allclose(dk[a:b].sum(0), 0.0, atol=1e-12)
            np.testing.assert_allclose(dv[a:b].sum(0), do[a:b].sum(0), rtol=1e-12, atol=1e-12)


def test_gelu_grad_matches_torch_autograd_and_central_differences():
    z = np.linspace(-9.0, 9.0, 1201)
    tz = torch.tensor(z, requires_grad=True)
    F.gelu(tz, approximate="tanh").sum().backward()
    np.testing.assert_allclose(oracle.gelu_tanh_grad(z), tz.grad.numpy(), rtol=1e-12, atol=1e-14)
    e = 1e-6
    fd = (oracle.gelu_tanh(z + e) - oracle.gelu_tanh(z - e)) / (2 * e)
    np.testing.assert_allclose(oracle.gelu_tanh_grad(z), fd, rtol=1e-7, atol=1e-9)
    assert oracle.gelu_tanh_grad(0.0) == 0.5          # GELU'(0) = 1/2


def _ffn_setup(n=13, d=16, f=40, seed=90):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((n, d)) * 1.3 - 0.2
    table = rng.standard_normal((3, 3, d)) * 0.3
    w1 = rng.standard_normal((f, d)) * 0.4
    w2 = rng.standard_normal((d, f)) * 0.3
    b1, b2 = rng.standard_normal(f) * 0.1, rng.standard_normal(d) * 0.1
    mod = rng.integers(0, 3, n)
    dout = rng.standard_normal((n, d))
    return x, table, w1, w2, b1, b2, mod, dout


def test_ffn_backward_directional_derivatives():
    x, table, w1, w2, b1, b2, mod, dout = _ffn_setup()
    g = oracle.ffn_backward(x, mod, table, w1, w2, dout, b1, b2)
    args = dict(x=x, table_mlp=table, w1=w1, w2=w2, b1=b1, b2=b2)
    grads = dict(x=g["dx"], table_mlp=g["dtable"], w1=g["dw1"], w2=g["dw2"], b1=g["db1"],
                 b2=g["db2"])

    def obj(**kw):
        return float(np.sum(dout * oracle.ffn_forward(modality=mod, **kw)))

    rng = np.random.Generator(np.random.PCG64(91))
    eps = 1e-5
    for name, val in args.items():
        delta = rng.standard_normal(val.shape)
        fd = (obj(**dict(args, **{name: val + eps * delta}))
              - obj(**dict(args, **{name: val - eps * delta}))) / (2 * eps)
        an = float(np.sum(grads[name] * delta))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_ffn_backward_matches_torch_autograd():
    x, table, w1, w2, b1, b2, mod, dout = _ffn_setup(seed=92)
    g = oracle.ffn_backward(x, mod, table, w1, w2, dout, b1, b2)
    t = {k: torch.tensor(v, requires_grad=True) for k, v in
         dict(x=x, table=table, w1=w1, w2=w2, b1=b1, b2=b2).items()}
    m = torch.tensor(mod)
    y = F.layer_norm(t["x"], (x.shape[1],), eps=1e-6) * (1 + t["table"][m, 1]) + t["table"][m, 0]
    h = F.gelu(F.linear(y, t["w1"], t["b1"]), approximate="tanh")
    out = t["x"] + t["table"][m, 2] * F.linear(h, t["w2"], t["b2"])
    out.backward(torch.tensor(dout))
    for key, tk in (("dx", "x"), ("dtable", "table"), ("dw1", "w1"), ("dw2", "w2"),
                    ("db1", "b1"), ("db2", "b2")):
        np.testing.assert_allclose(g[key], t[tk].grad.numpy(), rtol=1e-10, atol=1e-12)


def test_stored_medium_backward_belongs_to_the_current_inputs():
    """tests/golden/block_backward_medium.npz (written by the oracle through
    make_block_backward_medium.py) matches the medium workload's current inputs:
    its db_o equals the closed form sum_i gate[m_i] * dout_i, its gate-row table
    gradients are zero nowhere the modality is present, and it holds every
    array the GPU test reads."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "block_backward_medium.npz")
    gold = np.load(path)
    wl = synth.WORKLOADS["medium"]
    inp = synth.block_inputs(wl)
    lay = oracle.pack_layout([r.grid for r in wl.requests])
    n, d = wl.n_tokens, wl.d_model
    dout = synth.normal_array((n, d), seed=1500 + n, dtype="bf16")
    gate = np.asarray(inp.table, np.float64)[np.asarray(lay["modality"]), 2, :]
    db_o = (gate * dout).sum(axis=0)
    np.testing.assert_allclose(gold["db_o"], db_o, rtol=1e-5, atol=1e-4)
    assert np.all(np.abs(gold["dtable"][:, 2, :]).max(axis=1) > 0)
    for key in ("dx", "dw_qkv", "dw_o"):
        for part in ("pos", "val", "rownorm", "norm", "maxabs", "sketch"):
            assert f"{key}_{part}" in gold.files, (key, part)
