"""Pins of the oracle's whole block (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import brute
import synth


def _tiny(n=12, d=16, h=2, seed=50, with_bias=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((n, d))
    table = rng.standard_normal((3, 3, d)) * 0.3
    w_qkv = rng.standard_normal((3 * d, d)) * 0.3
    w_o = rng.standard_normal((d, d)) * 0.3
    b_qkv = rng.standard_normal(3 * d) * 0.1 if with_bias else None
    b_o = rng.standard_normal(d) * 0.1 if with_bias else None
    mod = rng.integers(0, 3, n)
    pos = rng.integers(0, 9, (n, 3))
    return x, table, w_qkv, w_o, b_qkv, b_o, mod, pos


def test_identity_modulation_zero_positions_is_torch_composition():
    """Zero shift, unit scale, unit gate, all positions 0:
    out = x + linear(SDPA(LN(x)Wq, LN(x)Wk, LN(x)Wv), W_o), from torch float64 calls."""
    d, h = 16, 2
    x, table, w_qkv, w_o, _, _, mod, pos = _tiny(d=d, h=h)
    table[:] = 0.0
    table[:, 2, :] = 1.0
    pos[:] = 0
    cu = [0, 7, 12]
    res = oracle.block_forward(x, mod, pos, cu, table, w_qkv, w_o,
                               n_heads=h, head_dim=d // h, sections=(2, 2, 4))
    xt = torch.from_numpy(x)
    ln = F.layer_norm(xt, (d,), eps=1e-6)
    qkv = F.linear(ln, torch.from_numpy(w_qkv))
    outs = []
    for a, b in zip(cu, cu[1:]):
        q, k, v = (qkv[a:b, i * d:(i + 1) * d].reshape(b - a, h, d // h).transpose(0, 1)
                   for i in range(3))
        o = F.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(b - a, d)
        outs.append(o)
    o = torch.cat(outs)
    ref = xt + F.linear(o, torch.from_numpy(w_o))
    np.testing.assert_allclose(res["out"], ref.numpy(), rtol=0, atol=1e-12)


def test_zero_gate_returns_input_exactly():
    x, table, w_qkv, w_o, _, _, mod, pos = _tiny()
    table[:, 2, :] = 0.0
    res = oracle.block_forward(x, mod, pos, [0, 12], table, w_qkv, w_o,
                               n_heads=2, head_dim=8, sections=(2, 2, 4))
    np.testing.assert_array_equal(res["out"], x)


def test_gate_row_scales_branch_linearly():
    x, table, w_qkv, w_o, _, _, mod, pos = _tiny(seed=51)
    kw = dict(n_heads=2, head_dim=8, sections=(2, 2, 4))
    r1 = oracle.block_forward(x, mod, pos, [0, 12], table, w_qkv, w_o, **kw)
    t2 = table.copy()
    t2[:, 2, :] *= 3.0
    r2 = oracle.block_forward(x, mod, pos, [0, 12], t2, w_qkv, w_o, **kw)
    np.testing.assert_allclose(r2["out"] - x, 3.0 * (r1["out"] - x), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal,with_bias", [(False, False), (True, True)])
def test_brute_force_block(causal, with_bias):
    x, table, w_qkv, w_o, b_qkv, b_o, mod, pos = _tiny(n=10, seed=52, with_bias=with_bias)
    cu = [0, 4, 10]
    res = oracle.block_forward(x, mod, pos, cu, table, w_qkv, w_o, n_heads=2, head_dim=8,
                               sections=(2, 2, 4), causal=causal, b_qkv=b_qkv, b_o=b_o)
    ob = brute.block(x.tolist(), mod.tolist(), pos.tolist(), cu, table.tolist(),
                     w_qkv.tolist(), w_o.tolist(), 2, 8, (2, 2, 4), causal=causal,
                     b_qkv=None if b_qkv is None else b_qkv.tolist(),
                     b_o=None if b_o is None else b_o.tolist())
    np.testing.assert_allclose(res["out"], np.array(ob), rtol=0, atol=1e-11)


def test_rows_mode_matches_full():
    x, table, w_qkv, w_o, _, _, mod, pos = _tiny(seed=53)
    kw = dict(n_heads=2, head_dim=8, sections=(2, 2, 4))
    full = oracle.block_forward(x, mod, pos, [0, 5, 12], table, w_qkv, w_o, **kw)
    rows = [11, 0, 5]
    part = oracle.block_forward(x, mod, pos, [0, 5, 12], table, w_qkv, w_o, rows=rows, **kw)
    # BLAS may block a row subset differently: equal up to rounding order
    np.testing.assert_allclose(part["out"], full["out"][rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(part["o"], full["o"][rows], rtol=0, atol=1e-13)


def test_tiny_workload_runs_and_is_finite():
    wl = synth.WORKLOADS["tiny"]
    inp = synth.block_inputs(wl)
    lay = oracle.pack_layout([r.grid for r in wl.requests])
    res = oracle.block_forward(inp.x, lay["modality"], lay["pos"], lay["cu_seqlens"],
                               inp.table, inp.w_qkv, inp.w_o, n_heads=wl.n_heads,
                               head_dim=wl.head_dim, sections=wl.sections)
    assert res["out"].shape == (328, 256)
    assert np.isfinite(res["out"]).all()


def test_intermediates_catch_wiring_mistakes_that_out_does_not():
    """Why the block's GPU parity compares q', o and the other intermediates, not
    only out: the residual x dominates out (the branch is a gate ~ N(0, 0.1)
    times a projection of a softmax average), so a block without RoPE (every
    position 0) or with the mask split into four segments stays within the bf16
    tolerance on out, while q' and o move far past it.  The mistakes are planted
    in the oracle itself, on a 640-token pack with the bf16 workloads' value
    distributions."""
    wl = synth.WORKLOADS["small"]
    grid = (4, 8, 15, 40, 40)                       # 480 video + 2 x 40 audio + 40 text
    lay = oracle.pack_layout([grid])
    n, d, h, dh = lay["n_tokens"], 512, 4, 128
    x = synth.normal_array((n, d), seed=61, dtype="bf16")
    table = synth.normal_array((3, 3, d), seed=62, std=0.1)
    w_qkv = synth.normal_array((3 * d, d), seed=63, std=0.02, dtype="bf16")
    w_o = synth.normal_array((d, d), seed=64, std=0.02, dtype="bf16")

    def run(pos, cu):
        return oracle.block_forward(x, lay["modality"], pos, cu, table, w_qkv, w_o,
                                    n_heads=h, head_dim=dh, sections=wl.sections)

    def rel(a, b):
        return np.linalg.norm(a - b) / np.linalg.norm(b)

    good = run(lay["pos"], lay["cu_seqlens"])
    no_rope = run(np.zeros_like(lay["pos"]), lay["cu_seqlens"])
    split = run(lay["pos"], [0, n // 4, n // 2, 3 * n // 4, n])
    tol = 1e-2                                             # the bf16 rel-L2 bound
    for bad in (no_rope, split):
        assert rel(bad["out"], good["out"]) < tol          # out alone would pass
    assert rel(no_rope["q_rot"], good["q_rot"]) > 5 * tol
    assert rel(no_rope["o"], good["o"]) > 5 * tol
    assert rel(split["o"], good["o"]) > 5 * tol
