"""Parity of the backward entry points against the float64 oracle (MI355X only).

Gradients are bf16 and compared at rel-L2 <= 1e-2 with max-abs <= 3e-2 times
max(1, max |reference|) (the bf16 output bound, relative to the gradient's own
scale: weight gradients sum over every token and grow with the pack).  The
log-sum-exp is float32 and compared at 1e-5 relative.  At the full shape the
key and value gradients (whose oracle needs every softmax row) are checked
through two invariants of the softmax: per segment the key gradients sum to
zero and the value gradients sum to the output gradients.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, dev_int, host, rel_l2, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jav():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import joint_audio_video_amd as m
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


def check_grad(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref))) if got.size else 0.0
    bound = 3e-2 * max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)
    print(f"  {what}: rel_l2={r:.3e} max_abs={m:.3e} (bound {bound:.2e})", flush=True)
    assert r <= 1e-2 and m <= bound, (what, r, m)


def _qkvo(n, H, seed, q_scale=1.0):
    q = synth.normal_array((n, H * 128), seed, dtype="bf16") * np.float32(q_scale)
    q = synth.round_to_bf16(q)
    k = synth.normal_array((n, H * 128), seed + 1, dtype="bf16")
    v = synth.normal_array((n, H * 128), seed + 2, dtype="bf16")
    do = synth.normal_array((n, H * 128), seed + 3, dtype="bf16")
    return q, k, v, do


CASES = [
    # (name, n, heads, cu, causal, q_scale)
    ("one_segment", 4096, 12, [0, 4096], False, 1.0),
    ("ragged", 1000, 4, [0, 1, 64, 128, 129, 259, 559, 560, 1000], False, 1.0),
    ("ragged_causal", 1000, 4, [0, 1, 64, 128, 129, 259, 559, 560, 1000], True, 1.0),
    ("peaky", 700, 3, [0, 300, 700], False, 3.0),
    ("peaky_causal", 700, 3, [0, 700], True, 3.0),
]


@pytest.mark.parametrize("name,n,H,cu,causal,qs", CASES)
def test_attention_lse_and_backward(jav, name, n, H, cu, causal, qs):
    import torch
    q, k, v, do = _qkvo(n, H, 1200 + n, qs)
    cu_d = dev_int(np.asarray(cu), torch.int32)
    ms = max(b - a for a, b in zip(cu, cu[1:]))
    print(f"attn backward {name} n={n} H={H} causal={causal}", flush=True)
    qd, kd, vd, dod = (dev(a, "bf16") for a in (q, k, v, do))
    o, lse = jav.attn_packed_lse(qd, kd, vd, cu_d, ms, H, 128, causal=causal)
    o_plain = jav.attn_packed(qd, kd, vd, cu_d, ms, H, 128, causal=causal)
    dq, dk, dv = jav.attn_packed_backward(qd, kd, vd, o, dod, lse, cu_d, ms, H, 128,
                                          causal=causal)
    dq2, dk2, dv2 = jav.attn_packed_backward(qd, kd, vd, o, dod, lse, cu_d, ms, H, 128,
                                             causal=causal)
    _sync()
    assert torch.equal(o, o_plain)                     # the lse output changes nothing else
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    ref_lse = oracle.attention_lse(q, k, cu, H, 128, causal=causal)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=1e-5)
    # the oracle's backward takes the library's bf16 o only through delta = rowsum(do o);
    # it recomputes its own o from q, k, v
    rq, rk, rv = oracle.attention_backward(q, k, v, do, cu, H, 128, causal=causal)
    check_grad(host(dq), rq, f"{name}.dq")
    check_grad(host(dk), rk, f"{name}.dk")
    check_grad(host(dv), rv, f"{name}.dv")


def test_attention_backward_leaves_rows_outside_segments_alone(jav):
    """cu_seqlens ending before the buffer: trailing rows of dq, dk, dv keep their contents
    and NaN in the trailing input rows does not leak."""
    import torch
    n, H = 600, 2
    q, k, v, do = _qkvo(n, H, 1300)
    for a in (q, k, v, do):
        a[520:] = np.nan
    cu = [0, 200, 520]
    cu_d = dev_int(np.asarray(cu), torch.int32)
    qd, kd, vd, dod = (dev(a, "bf16") for a in (q, k, v, do))
    o, lse = jav.attn_packed_lse(qd, kd, vd, cu_d, 320, H, 128, n_tokens=520)
    dq, dk, dv = (torch.full((n, H * 128), 7.0, dtype=torch.bfloat16, device="cuda")
                  for _ in range(3))
    jav.attn_packed_backward(qd, kd, vd, o, dod, lse, cu_d, 320, H, 128, dq=dq, dk=dk, dv=dv,
                             n_tokens=520)
    _sync()
    for t in (dq, dk, dv):
        assert torch.isfinite(t[:520].float()).all()
        assert bool((t[520:] == 7.0).all())
    rq, rk, rv = oracle.attention_backward(q[:520], k[:520], v[:520], do[:520], cu, H, 128)
    check_grad(host(dq)[:520], rq, "tail.dq")
    check_grad(host(dk)[:520], rk, "tail.dk")
    check_grad(host(dv)[:520], rv, "tail.dv")


def test_attention_backward_full_shape(jav):
    """58,758 tokens, 40 heads: dq on sampled rows against the oracle; dk and dv through
    the softmax's invariants per head (sum of dk = 0, sum of dv = sum of dout)."""
    import torch
    wl = synth.WORKLOADS["full"]
    n, H = wl.n_tokens, wl.n_heads
    q, k, v, do = _qkvo(n, H, 1400)
    cu = [0, n]
    cu_d = dev_int(np.asarray(cu), torch.int32)
    print(f"attn backward full n={n} H={H}", flush=True)
    qd, kd, vd, dod = (dev(a, "bf16") for a in (q, k, v, do))
    o, lse = jav.attn_packed_lse(qd, kd, vd, cu_d, n, H, 128)
    dq, dk, dv = jav.attn_packed_backward(qd, kd, vd, o, dod, lse, cu_d, n, H, 128)
    _sync()
    rows = sample_rows(cu, n, extra_every=4999, edge=2, limit=24)
    rq = oracle.attention_backward_rows(q, k, v, do, cu, H, 128, rows)
    check_grad(host(dq[torch.from_numpy(rows).cuda()]), rq, "full.dq")
    ref_lse = oracle.attention_lse(q, k, cu, H, 128, rows=rows[:6])
    np.testing.assert_allclose(lse[:, torch.from_numpy(rows[:6]).cuda()].cpu().numpy(), ref_lse,
                               rtol=1e-5, atol=1e-5)
    dk_sum = dk.float().sum(0).cpu().numpy().astype(np.float64)
    dv_sum = dv.float().sum(0).cpu().numpy().astype(np.float64)
    do_sum = do.astype(np.float64).sum(0)
    dk_abs = dk.float().abs().sum(0).cpu().numpy().astype(np.float64)
    print(f"  full: |sum dk| / sum |dk| max {np.max(np.abs(dk_sum) / dk_abs):.2e}", flush=True)
    assert np.all(np.abs(dk_sum) <= 1e-2 * dk_abs)
    r = rel_l2(dv_sum, do_sum)
    print(f"  full: sum dv vs sum dout rel_l2={r:.2e}", flush=True)
    assert r <= 1e-2


@pytest.mark.parametrize("causal", [False, True])
def test_attention_backward_varlen_pack(jav, causal):
    """The 4-request pack (58,758 tokens in segments of 14,690 / 14,690 / 14,689 /
    14,689, 40 heads): dq on rows at every segment's edges and spread through it against
    the oracle; dk and dv through the softmax's invariants per segment and head (the
    sum of dk over a segment's keys is 0, the sum of dv equals the sum of dout over its
    queries); a second call gives the same bits."""
    import torch
    wl = synth.WORKLOADS["varlen"]
    n, H = wl.n_tokens, wl.n_heads
    cu = [int(c) for c in oracle.pack_layout([r.grid for r in wl.requests])["cu_seqlens"]]
    ms = max(b - a for a, b in zip(cu, cu[1:]))
    q, k, v, do = _qkvo(n, H, 1600 + int(causal))
    cu_d = dev_int(np.asarray(cu), torch.int32)
    print(f"attn backward varlen n={n} H={H} segs={len(cu) - 1} causal={causal}", flush=True)
    qd, kd, vd, dod = (dev(a, "bf16") for a in (q, k, v, do))
    o, lse = jav.attn_packed_lse(qd, kd, vd, cu_d, ms, H, 128, causal=causal)
    dq, dk, dv = jav.attn_packed_backward(qd, kd, vd, o, dod, lse, cu_d, ms, H, 128,
                                          causal=causal)
    dq2, dk2, dv2 = jav.attn_packed_backward(qd, kd, vd, o, dod, lse, cu_d, ms, H, 128,
                                             causal=causal)
    _sync()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    edges = {r for a, b in zip(cu, cu[1:]) for r in (a, a + 1, b - 2, b - 1)}
    rows = np.array(sorted(edges | set(range(0, n, 2999))), dtype=np.int64)
    rq = oracle.attention_backward_rows(q, k, v, do, cu, H, 128, rows, causal=causal)
    check_grad(host(dq[torch.from_numpy(rows).cuda()]), rq, f"varlen.c{int(causal)}.dq")
    dk_h = dk.float().cpu().numpy().astype(np.float64)
    dv_h = dv.float().cpu().numpy().astype(np.float64)
    do_h = do.astype(np.float64)
    for a, b in zip(cu, cu[1:]):
        dk_sum, dk_abs = dk_h[a:b].sum(0), np.abs(dk_h[a:b]).sum(0)
        assert np.all(np.abs(dk_sum) <= 1e-2 * dk_abs), (a, b)
        r = rel_l2(dv_h[a:b].sum(0), do_h[a:b].sum(0))
        print(f"  segment [{a}, {b}): max |sum dk| / sum |dk| "
              f"{np.max(np.abs(dk_sum) / dk_abs):.2e}, sum dv vs sum dout rel_l2={r:.2e}", flush=True)
        assert r <= 1e-2, (a, b, r)


# ---------------------------------------------------------------------------
# The attention half's backward
# ---------------------------------------------------------------------------

def _layout(jav, name, n, cu):
    import torch
    wl = synth.WORKLOADS[name]
    grids = [r.grid for r in wl.requests]
    lay_d, lay = jav.pack_layout(grids), oracle.pack_layout(grids)
    cu = list(lay["cu_seqlens"]) if cu is None else list(cu)
    mod, pos = np.asarray(lay["modality"])[:n], np.asarray(lay["pos"])[:n]
    dev_lay = (dev_int(np.asarray(lay_d["modality"])[:n], torch.uint8),
               dev_int(np.asarray(lay_d["pos"])[:n], torch.int32),
               dev_int(np.asarray(cu), torch.int32), int(max(b - a for a, b in zip(cu, cu[1:]))))
    return mod, pos, cu, dev_lay


def _block_backward(jav, name, n=None, cu=None, causal=False, with_bias=False, inplace=False):
    import torch
    wl = synth.WORKLOADS[name]
    inp = synth.block_inputs(wl, n_tokens=n, with_bias=with_bias)
    n, d = inp.x.shape
    mod, pos, cu, (mod_d, pos_d, cu_d, ms) = _layout(jav, name, n, cu)
    dout = synth.normal_array((n, d), seed=1500 + n, dtype="bf16")
    desc = jav.block_desc(jav.DIT_BF16, d, wl.n_heads, wl.head_dim, wl.sections, wl.theta,
                          wl.eps, causal=causal)
    print(f"block backward {name} n={n} segs={len(cu) - 1} causal={causal} bias={with_bias} "
          f"inplace={inplace}", flush=True)
    x_d, dout_d = dev(inp.x, "bf16"), dev(dout, "bf16")
    args = (desc, x_d, dout_d, mod_d, pos_d, cu_d, ms, dev(inp.table, "f32"),
            dev(inp.w_qkv, "bf16"), dev(inp.w_o, "bf16"))
    kw = dict(b_qkv=dev(inp.b_qkv, "bf16") if with_bias else None,
              b_o=dev(inp.b_o, "bf16") if with_bias else None)
    again = jav.block_backward(*args, **kw)
    got = jav.block_backward(*args, dx=dout_d if inplace else None, **kw)
    _sync()
    for key in ("dtable", "dw_qkv", "dw_o", "db_qkv", "db_o"):
        assert torch.equal(got[key], again[key]), key          # deterministic
    assert torch.equal(got["dx"], again["dx"])
    ref = oracle.block_backward(inp.x, mod, pos, cu, inp.table, inp.w_qkv, inp.w_o, dout,
                                n_heads=wl.n_heads, head_dim=wl.head_dim, sections=wl.sections,
                                theta=wl.theta, eps=wl.eps, causal=causal,
                                b_qkv=inp.b_qkv if with_bias else None,
                                b_o=inp.b_o if with_bias else None)
    check_grad(host(got["dx"]), ref["dx"], f"{name}.dx")
    check_grad(host(got["dw_o"]), ref["dw_o"], f"{name}.dw_o")
    check_grad(host(got["dw_qkv"]), ref["dw_qkv"], f"{name}.dw_qkv")
    check_grad(host(got["db_o"]), ref["db_o"], f"{name}.db_o")
    check_grad(host(got["db_qkv"]), ref["db_qkv"], f"{name}.db_qkv")
    present = np.unique(mod)
    for r, row in enumerate(("shift", "scale", "gate")):
        check_grad(host(got["dtable"])[present, r], ref["dtable"][present, r],
                   f"{name}.dtable.{row}")
    absent = np.setdiff1d(np.arange(3), present)
    assert not host(got["dtable"])[absent].any()


def test_block_backward_small(jav):
    _block_backward(jav, "small")


def test_block_backward_ragged_causal_bias_inplace(jav):
    _block_backward(jav, "small", n=1000, cu=[0, 617, 1000], causal=True, with_bias=True,
                    inplace=True)


def _golden_module():
    import importlib.util
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "make_block_backward_medium.py")
    spec = importlib.util.spec_from_file_location("_make_block_backward_medium", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_block_backward_medium_against_stored_oracle(jav):
    """dit_block_backward at the medium workload (16,384 tokens, d_model 3072, 24
    heads) against the float64 oracle's gradients, which
    tests/golden/make_block_backward_medium.py stored (the oracle needs minutes
    there).  db_qkv, db_o and every table row are compared whole; dx, dW_qkv and
    dW_o on 16,384 sampled elements each, through every row's norm, the
    Frobenius norm, and a two-sided Gaussian sketch A G B whose relative
    distance estimates the whole tensor's (2e-2: the estimate of a 1e-2-scale
    error varies by a small factor with the error's shape)."""
    import torch
    gm = _golden_module()
    gold = np.load(gm.OUT)
    wl = synth.WORKLOADS["medium"]
    inp = synth.block_inputs(wl)
    n, d = inp.x.shape
    mod, _, _, (mod_d, pos_d, cu_d, ms) = _layout(jav, "medium", n, None)
    dout = synth.normal_array((n, d), seed=1500 + n, dtype="bf16")
    desc = jav.block_desc(jav.DIT_BF16, d, wl.n_heads, wl.head_dim, wl.sections, wl.theta,
                          wl.eps)
    print(f"block backward medium n={n} (stored oracle)", flush=True)
    got = jav.block_backward(desc, dev(inp.x, "bf16"), dev(dout, "bf16"), mod_d, pos_d, cu_d, ms,
                             dev(inp.table, "f32"), dev(inp.w_qkv, "bf16"), dev(inp.w_o, "bf16"))
    _sync()
    check_grad(host(got["db_qkv"]), gold["db_qkv"], "medium.db_qkv")
    check_grad(host(got["db_o"]), gold["db_o"], "medium.db_o")
    present = np.unique(mod)
    for r, row in enumerate(("shift", "scale", "gate")):
        check_grad(host(got["dtable"])[present, r], gold["dtable"][present, r],
                   f"medium.dtable.{row}")
    for key, seed in gm.BIG.items():
        g = host(got[key])
        pos = gold[f"{key}_pos"]
        vals = g.reshape(-1)[pos]
        ref = gold[f"{key}_val"].astype(np.float64)
        r = rel_l2(vals, ref)
        m = float(np.max(np.abs(vals - ref)))
        bound = 3e-2 * max(1.0, float(gold[f"{key}_maxabs"]))
        rn = rel_l2(np.linalg.norm(g, axis=1), gold[f"{key}_rownorm"])
        nr = abs(float(np.linalg.norm(g)) - float(gold[f"{key}_norm"])) / float(gold[f"{key}_norm"])
        a, b = gm.sketch_mats(g.shape[0], g.shape[1], seed)
        sk = rel_l2(a @ g @ b, gold[f"{key}_sketch"])
        print(f"  medium.{key}: sampled rel_l2={r:.3e} max_abs={m:.3e} (bound {bound:.2e}) "
              f"row norms {rn:.3e} norm {nr:.3e} sketch {sk:.3e}", flush=True)
        assert np.isfinite(g).all(), key
        assert r <= 1e-2 and m <= bound, (key, r, m)
        assert rn <= 1e-2 and nr <= 1e-2 and sk <= 2e-2, (key, rn, nr, sk)


def test_block_backward_full_shape(jav):
    """58,758 tokens: finite and deterministic; db_o against the sum of gate * dout from the
    inputs alone; absent modalities get zero table rows (the full pack has all three)."""
    import torch
    wl = synth.WORKLOADS["full"]
    inp = synth.block_inputs(wl)
    n, d = inp.x.shape
    mod, _, cu, (mod_d, pos_d, cu_d, ms) = _layout(jav, "full", n, None)
    dout = synth.normal_array((n, d), seed=1600, dtype="bf16")
    desc = jav.block_desc(jav.DIT_BF16, d, wl.n_heads, wl.head_dim, wl.sections, wl.theta,
                          wl.eps)
    print(f"block backward full n={n}", flush=True)
    args = (desc, dev(inp.x, "bf16"), dev(dout, "bf16"), mod_d, pos_d, cu_d, ms,
            dev(inp.table, "f32"), dev(inp.w_qkv, "bf16"), dev(inp.w_o, "bf16"))
    a = jav.block_backward(*args)
    b = jav.block_backward(*args)
    _sync()
    for key in ("dx", "dtable", "dw_qkv", "dw_o", "db_qkv", "db_o"):
        assert torch.isfinite(a[key].float()).all(), key
        assert torch.equal(a[key], b[key]), key
    gate = inp.table[mod, 2, :].astype(np.float64)
    want = (gate * dout.astype(np.float64)).sum(0)
    r = rel_l2(host(a["db_o"]), want)
    print(f"  full.db_o: rel_l2={r:.2e}", flush=True)
    assert r <= 1e-2


# ---------------------------------------------------------------------------
# The feed-forward half's backward
# ---------------------------------------------------------------------------

def _ffn_backward(jav, name, n=None, with_bias=False, inplace=False):
    import torch
    wl = synth.WORKLOADS[name]
    f = synth.ffn_inputs(wl, with_bias=with_bias)
    x = synth.normal_array((wl.n_tokens, wl.d_model), seed=500 + wl.seed, dtype="bf16")
    if n is not None:
        x = x[:n]
    n, d = x.shape
    mod, _, _, (mod_d, _, _, _) = _layout(jav, name, n, [0, n])
    dout = synth.normal_array((n, d), seed=1700 + n, dtype="bf16")
    desc = jav.ffn_desc(jav.DIT_BF16, d, wl.d_ff, wl.eps)
    print(f"ffn backward {name} n={n} bias={with_bias} inplace={inplace}", flush=True)
    dout_d = dev(dout, "bf16")
    args = (desc, dev(x, "bf16"), dout_d, mod_d, dev(f.table, "f32"), dev(f.w1, "bf16"),
            dev(f.w2, "bf16"))
    kw = dict(b1=dev(f.b1, "bf16") if with_bias else None,
              b2=dev(f.b2, "bf16") if with_bias else None)
    again = jav.ffn_backward(*args, **kw)
    got = jav.ffn_backward(*args, dx=dout_d if inplace else None, **kw)
    _sync()
    for key in ("dx", "dtable", "dw1", "dw2", "db1", "db2"):
        assert torch.equal(got[key], again[key]), key
    ref = oracle.ffn_backward(x, mod, f.table, f.w1, f.w2, dout, f.b1 if with_bias else None,
                              f.b2 if with_bias else None, wl.eps)
    for key in ("dx", "dw1", "dw2", "db1", "db2"):
        check_grad(host(got[key]), ref[key], f"ffn.{name}.{key}")
    present = np.unique(mod)
    for r, row in enumerate(("shift", "scale", "gate")):
        check_grad(host(got["dtable"])[present, r], ref["dtable"][present, r],
                   f"ffn.{name}.dtable.{row}")


def test_ffn_backward_small(jav):
    _ffn_backward(jav, "small")


def test_ffn_backward_ragged_bias_inplace(jav):
    _ffn_backward(jav, "small", n=1000, with_bias=True, inplace=True)


def test_ffn_backward_full_shape(jav):
    """58,758 tokens, d_ff 20,480: finite, deterministic, and db2 against the sum of
    gate * dout from the inputs alone."""
    import torch
    wl = synth.WORKLOADS["full"]
    f = synth.ffn_inputs(wl)
    n, d = wl.n_tokens, wl.d_model
    mod, _, _, (mod_d, _, _, _) = _layout(jav, "full", n, [0, n])
    x = synth.normal_array((n, d), seed=1800, dtype="bf16")
    dout = synth.normal_array((n, d), seed=1801, dtype="bf16")
    desc = jav.ffn_desc(jav.DIT_BF16, d, wl.d_ff, wl.eps)
    print(f"ffn backward full n={n}", flush=True)
    args = (desc, dev(x, "bf16"), dev(dout, "bf16"), mod_d, dev(f.table, "f32"),
            dev(f.w1, "bf16"), dev(f.w2, "bf16"))
    a = jav.ffn_backward(*args)
    b = jav.ffn_backward(*args)
    _sync()
    for key in ("dx", "dtable", "dw1", "dw2", "db1", "db2"):
        assert torch.isfinite(a[key].float()).all(), key
        assert torch.equal(a[key], b[key]), key
    want = (f.table[mod, 2, :].astype(np.float64) * dout.astype(np.float64)).sum(0)
    r = rel_l2(host(a["db2"]), want)
    print(f"  ffn.full.db2: rel_l2={r:.2e}", flush=True)
    assert r <= 1e-2


def test_backward_workspaces_poisoned_with_nan(jav):
    """Workspaces filled with NaN give gradients bit-identical to a zero-filled workspace:
    no stage reads scratch it has not written (the transposes' zero padding included)."""
    import torch
    wl = synth.WORKLOADS["small"]
    n = 700                                  # not a multiple of 64: padded transposes
    inp = synth.block_inputs(wl, n_tokens=n, with_bias=True)
    f = synth.ffn_inputs(wl, with_bias=True)
    d = wl.d_model
    _, _, cu, (mod_d, pos_d, cu_d, ms) = _layout(jav, "small", n, [0, 300, n])
    dout = dev(synth.normal_array((n, d), seed=1900, dtype="bf16"), "bf16")
    x = dev(inp.x, "bf16")
    desc = jav.block_desc(jav.DIT_BF16, d, wl.n_heads, wl.head_dim, wl.sections, wl.theta, wl.eps)
    fdesc = jav.ffn_desc(jav.DIT_BF16, d, wl.d_ff, wl.eps)
    print(f"backward poison n={n}", flush=True)
    outs = []
    for fill in (0.0, float("nan")):
        bws = torch.empty(jav.block_backward_workspace_bytes(desc, n), dtype=torch.uint8,
                          device="cuda")
        fws = torch.empty(jav.ffn_backward_workspace_bytes(fdesc, n), dtype=torch.uint8,
                          device="cuda")
        for w in (bws, fws):                 # sizes are multiples of 256 bytes
            w.view(torch.float32).fill_(fill)
        a = jav.block_backward(desc, x, dout, mod_d, pos_d, cu_d, ms, dev(inp.table, "f32"),
                               dev(inp.w_qkv, "bf16"), dev(inp.w_o, "bf16"),
                               b_qkv=dev(inp.b_qkv, "bf16"), b_o=dev(inp.b_o, "bf16"),
                               workspace=bws)
        b = jav.ffn_backward(fdesc, x, dout, mod_d, dev(f.table, "f32"), dev(f.w1, "bf16"),
                             dev(f.w2, "bf16"), b1=dev(f.b1, "bf16"), b2=dev(f.b2, "bf16"),
                             workspace=fws)
        _sync()
        outs.append((a, b))
    for key in ("dx", "dtable", "dw_qkv", "dw_o", "db_qkv", "db_o"):
        assert torch.isfinite(outs[1][0][key].float()).all(), key
        assert torch.equal(outs[0][0][key], outs[1][0][key]), key
    for key in ("dx", "dtable", "dw1", "dw2", "db1", "db2"):
        assert torch.isfinite(outs[1][1][key].float()).all(), key
        assert torch.equal(outs[0][1][key], outs[1][1][key]), key


def test_backward_segment_longer_than_max_seqlen_becomes_nan(jav):
    """cu_seqlens breaking its contract (a 400-row segment against max_seqlen 300,
    inside the buffers): that segment's dq, dk and dv rows come out NaN, and the
    other segment's gradients are bit-identical to a call with the right max_seqlen."""
    import torch
    n, H = 700, 2
    q, k, v, do = (dev(a, "bf16") for a in _qkvo(n, H, 1400))
    cu_d = dev_int(np.array([0, 300, 700], np.int32), torch.int32)
    o, lse = jav.attn_packed_lse(q, k, v, cu_d, 400, H, 128)
    good = jav.attn_packed_backward(q, k, v, o, do, lse, cu_d, 400, H, 128)
    bad = jav.attn_packed_backward(q, k, v, o, do, lse, cu_d, 300, H, 128)
    _sync()
    for name, g, b in zip(("dq", "dk", "dv"), good, bad):
        assert torch.equal(b[:300].view(torch.int16), g[:300].view(torch.int16)), name
        assert torch.isnan(b[300:].float()).all(), name
