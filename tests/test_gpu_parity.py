"""Parity of every libdit entry point against the float64 oracle (MI355X only).

Each stage is checked on its own seeded inputs (so errors do not compound),
and the whole block end to end from the original inputs.  Inputs come from
``synth``; the library's own host layout feeds the device, the oracle's own
layout feeds the oracle (the two are bit-identical, see test_abi_host.py).
Large workloads are compared on sampled rows that include the first and last
rows of every segment and the ragged tail.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import check, ci_sample_rows, dev, dev_f32, dev_int, host, rel_l2, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jav():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import joint_audio_video_amd as m
    return m


@functools.lru_cache(maxsize=2)
def _inputs(name):
    return synth.block_inputs(synth.WORKLOADS[name])


@functools.lru_cache(maxsize=4)
def _layout(name):
    wl = synth.WORKLOADS[name]
    return oracle.pack_layout([r.grid for r in wl.requests])


def _dev_layout(jav, name):
    import torch
    wl = synth.WORKLOADS[name]
    lay = jav.pack_layout([r.grid for r in wl.requests])
    return (dev_int(lay["modality"], torch.uint8), dev_int(lay["pos"], torch.int32),
            dev_int(lay["cu_seqlens"], torch.int32), lay["max_seqlen"])


def _sync():
    import torch
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# adaln_modulate
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "small", "medium", "full"])
def test_adaln_parity(jav, name):
    import torch
    wl = synth.WORKLOADS[name]
    inp = _inputs(name)
    lay = _layout(name)
    mod_d, _, _, _ = _dev_layout(jav, name)
    print(f"adaln {name} N={wl.n_tokens} D={wl.d_model}", flush=True)
    x = dev(inp.x, wl.dtype)
    y = jav.adaln_modulate(x, mod_d, dev_f32(inp.table), eps=wl.eps)
    _sync()
    rows = None if name != "full" else sample_rows(lay["cu_seqlens"], wl.n_tokens, limit=4000)
    ref = oracle.adaln_modulate(inp.x, lay["modality"], inp.table, wl.eps, rows=rows)
    got = host(y) if rows is None else host(y[torch.from_numpy(rows).cuda()])
    check(got, ref, wl.dtype, f"adaln[{name}]")


@pytest.mark.parametrize("n", [1000, 999])
def test_adaln_strided_rows_and_trim(jav, n):
    """Rows inside wider buffers; only n_tokens rows are touched.  Modalities are
    drawn per row, so neighbouring rows (one wave's pair) often differ; an odd
    n leaves the last wave a single row."""
    import torch
    d, rows_alloc = 1536, 1040
    x_full = synth.normal_array((rows_alloc, d + 64), seed=70, dtype="bf16")
    table = synth.normal_array((3, 3, d), seed=71, std=0.1)
    mod = synth.uniform_ints((rows_alloc,), 0, 3, seed=72).astype(np.uint8)
    x = dev(x_full, "bf16")
    y = torch.full((rows_alloc, d + 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    jav.adaln_modulate(x[:, :d], dev_int(mod, torch.uint8), dev_f32(table), out=y[:, :d],
                       n_tokens=n)
    _sync()
    ref = oracle.adaln_modulate(x_full[:n, :d], mod[:n], table)
    check(host(y[:n, :d]), ref, "bf16", "adaln strided")
    assert torch.isnan(y[n:]).all() and torch.isnan(y[:, d:]).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_adaln_wide_rows(jav, dtype):
    """d_model 8192: rows longer than the two-rows-per-wave register budget (one
    row per wave), with per-row modalities and an odd row count."""
    import torch
    d, n = 8192, 37
    x_h = synth.normal_array((n, d), seed=73, dtype=dtype)
    table = synth.normal_array((3, 3, d), seed=74, std=0.1)
    mod = synth.uniform_ints((n,), 0, 3, seed=75).astype(np.uint8)
    y = jav.adaln_modulate(dev(x_h, dtype), dev_int(mod, torch.uint8), dev_f32(table))
    _sync()
    check(host(y), oracle.adaln_modulate(x_h, mod, table), dtype, f"adaln wide {dtype}")


# ---------------------------------------------------------------------------
# rope3d_apply
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "small", "medium", "full"])
def test_rope_parity_on_fused_qkv(jav, name):
    import torch
    wl = synth.WORKLOADS[name]
    d, H, Dh = wl.d_model, wl.n_heads, wl.head_dim
    lay = _layout(name)
    _, pos_d, _, _ = _dev_layout(jav, name)
    n = wl.n_tokens
    print(f"rope {name} N={n}", flush=True)
    qkv_h = synth.normal_array((n, 3 * d), seed=100 + wl.seed, dtype=wl.dtype)
    qkv = dev(qkv_h, wl.dtype)
    before = qkv.clone()
    jav.rope3d_apply(qkv[:, :d], qkv[:, d:2 * d], pos_d, H, Dh, wl.sections, wl.theta)
    _sync()
    rows = None if n < 20000 else sample_rows(lay["cu_seqlens"], n, limit=3000)
    for which, sl in (("q", slice(0, d)), ("k", slice(d, 2 * d))):
        ref = oracle.rope3d(qkv_h[:, sl], lay["pos"], H, Dh, wl.sections, wl.theta, rows=rows)
        got = host(qkv[:, sl]) if rows is None else host(qkv[:, sl][torch.from_numpy(rows).cuda()])
        check(got, ref, wl.dtype, f"rope[{name}].{which}")
    # v untouched; audio/text rows keep their h and w sections bit for bit
    assert torch.equal(qkv[:, 2 * d:], before[:, 2 * d:])
    mod = np.asarray(lay["modality"])
    at = torch.from_numpy(np.nonzero(mod != 0)[0]).cuda()
    s_t = wl.sections[0]
    for sl in (slice(0, d), slice(d, 2 * d)):
        a = qkv[:, sl].view(n, H, Dh)[at][:, :, s_t:]
        b = before[:, sl].view(n, H, Dh)[at][:, :, s_t:]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("name", ["tiny", "small", "full"])
def test_rope_apply_to_out_of_place_and_crossed(jav, name):
    """rope3d_apply_to: separate outputs (inputs untouched), and the block's own
    arrangement, rotated q into a spare plane and rotated k over q's plane, with the
    same bits as the in-place entry point."""
    import torch
    wl = synth.WORKLOADS[name]
    d, H, Dh = wl.d_model, wl.n_heads, wl.head_dim
    lay = _layout(name)
    _, pos_d, _, _ = _dev_layout(jav, name)
    n = wl.n_tokens
    print(f"rope_to {name} N={n}", flush=True)
    qh = synth.normal_array((n, d), seed=120 + wl.seed, dtype=wl.dtype)
    kh = synth.normal_array((n, d), seed=121 + wl.seed, dtype=wl.dtype)
    q, k = dev(qh, wl.dtype), dev(kh, wl.dtype)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    jav.rope3d_apply_to(q, k, qo, ko, pos_d, H, Dh, wl.sections, wl.theta)
    _sync()
    assert torch.equal(q, dev(qh, wl.dtype)) and torch.equal(k, dev(kh, wl.dtype))
    rows = None if n < 20000 else sample_rows(lay["cu_seqlens"], n, limit=3000)
    for which, src, out in (("q", qh, qo), ("k", kh, ko)):
        ref = oracle.rope3d(src, lay["pos"], H, Dh, wl.sections, wl.theta, rows=rows)
        got = host(out) if rows is None else host(out[torch.from_numpy(rows).cuda()])
        check(got, ref, wl.dtype, f"rope_to[{name}].{which}")
    # in place, for the bit comparison
    qi, ki = q.clone(), k.clone()
    jav.rope3d_apply(qi, ki, pos_d, H, Dh, wl.sections, wl.theta)
    # the block's arrangement: q -> spare plane, k -> over q's plane
    spare = torch.empty_like(q)
    q2, k2 = q.clone(), k.clone()
    jav.rope3d_apply_to(q2, k2, spare, q2, pos_d, H, Dh, wl.sections, wl.theta)
    _sync()
    assert torch.equal(qo, qi) and torch.equal(ko, ki)
    assert torch.equal(spare, qi) and torch.equal(q2, ki) and torch.equal(k2, k)


def test_rope_wide_rows_in_chunks(jav):
    """56 heads x 128 (896 vectors per row): rows wider than one pass of the
    kernel, walked in chunks; 37 tokens (not a multiple of the 4 per
    workgroup), positions drawn at random with zeros included."""
    import torch
    n, H, Dh, sections = 37, 56, 128, (32, 48, 48)
    d = H * Dh
    qkv_h = synth.normal_array((n, 3 * d), seed=111, dtype="bf16")
    pos = synth.uniform_ints((n, 3), 0, 40, seed=112).astype(np.int32)
    pos[::5] = 0
    qkv = dev(qkv_h, "bf16")
    before = qkv.clone()
    jav.rope3d_apply(qkv[:, :d], qkv[:, d:2 * d], dev_int(pos, torch.int32), H, Dh, sections)
    _sync()
    for which, sl in (("q", slice(0, d)), ("k", slice(d, 2 * d))):
        ref = oracle.rope3d(qkv_h[:, sl], pos, H, Dh, sections, 1e4)
        check(host(qkv[:, sl]), ref, "bf16", f"rope wide.{which}")
    assert torch.equal(qkv[:, 2 * d:], before[:, 2 * d:])


def test_rope_q_only_and_zero_positions(jav):
    import torch
    n, H, Dh = 300, 4, 128
    x_h = synth.normal_array((n, H * Dh), seed=110, dtype="bf16")
    x = dev(x_h, "bf16")
    jav.rope3d_apply(x, None, dev_int(np.zeros((n, 3), np.int32), torch.int32), H, Dh, (32, 48, 48))
    _sync()
    assert torch.equal(x.view(torch.int16), dev(x_h, "bf16").view(torch.int16))


# ---------------------------------------------------------------------------
# attn_packed
# ---------------------------------------------------------------------------

def _attn_case(jav, n, H, Dh, cu, dtype, causal, seed, std=1.0, rows=None, max_seqlen=None,
               label=""):
    import torch
    print(f"attn {label} N={n} H={H} cu_len={len(cu) - 1} causal={causal}", flush=True)
    q_h = synth.normal_array((n, H * Dh), seed=seed, std=std, dtype=dtype)
    k_h = synth.normal_array((n, H * Dh), seed=seed + 1, std=std, dtype=dtype)
    v_h = synth.normal_array((n, H * Dh), seed=seed + 2, dtype=dtype)
    cu_d = dev_int(np.array(cu, np.int32), torch.int32)
    ms = max_seqlen or max(b - a for a, b in zip(cu, cu[1:]))
    o = jav.attn_packed(dev(q_h, dtype), dev(k_h, dtype), dev(v_h, dtype), cu_d, ms, H, Dh,
                        causal=causal)
    _sync()
    ref = oracle.attention(q_h, k_h, v_h, cu, H, Dh, causal, rows=rows)
    got = host(o) if rows is None else host(o[torch.from_numpy(rows).cuda()])
    check(got, ref, dtype, f"attn[{label}]")
    return o


def test_attention_tiny_f32(jav):
    wl = synth.WORKLOADS["tiny"]
    _attn_case(jav, wl.n_tokens, wl.n_heads, wl.head_dim, [0, wl.n_tokens], "f32", False, 200,
               label="tiny f32")
    _attn_case(jav, wl.n_tokens, wl.n_heads, wl.head_dim, [0, 100, 101, 328], "f32", True, 201,
               label="tiny f32 causal varlen")


def test_attention_f32_head_dim_128(jav):
    _attn_case(jav, 200, 2, 128, [0, 77, 200], "f32", False, 205, label="f32 dh128")


@pytest.mark.parametrize("causal", [False, True])
def test_attention_ragged_segments(jav, causal):
    """Segments of 1, 63, 64, 65, 127, 128, 129 and 300 tokens plus an empty one."""
    lens = [1, 63, 64, 65, 0, 127, 128, 129, 300]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    _attn_case(jav, cu[-1], 3, 128, cu, "bf16", causal, 210 + causal, label=f"ragged c={causal}")


def test_attention_peaky_scores(jav):
    _attn_case(jav, 700, 2, 128, [0, 700], "bf16", False, 220, std=2.0, label="peaky std2")
    _attn_case(jav, 700, 2, 128, [0, 333, 700], "bf16", True, 223, std=2.0, label="peaky causal")


def test_attention_small(jav):
    wl = synth.WORKLOADS["small"]
    rows = sample_rows([0, wl.n_tokens], wl.n_tokens, limit=512)
    _attn_case(jav, wl.n_tokens, wl.n_heads, 128, [0, wl.n_tokens], "bf16", False, 230, rows=rows,
               label="small")


@pytest.mark.parametrize("causal", [False, True])
def test_attention_medium(jav, causal):
    """The 16,384-token pack with 24 heads, on the CI sample of its layout."""
    wl = synth.WORKLOADS["medium"]
    rows = ci_sample_rows(_layout("medium"))
    _attn_case(jav, wl.n_tokens, wl.n_heads, 128, [0, wl.n_tokens], "bf16", causal, 235,
               rows=rows, label=f"medium c={causal}")


@pytest.mark.parametrize("variant", ["full", "modality_isolated", "varlen", "varlen_causal"])
def test_attention_full_shape(jav, variant):
    """58,758 tokens x 40 heads on the CI sample of the pack's layout (segment
    edges, every text row, the audio ends of both channels, the modality
    boundaries, every 97th row); the modality-isolated variant cuts segments at
    the modality boundaries of the full pack."""
    name = "varlen" if variant.startswith("varlen") else "full"
    wl = synth.WORKLOADS[name]
    n, H = wl.n_tokens, wl.n_heads
    if variant == "modality_isolated":
        cu = [0, 57040, 58640, 58758]
        lay = dict(_layout(name), cu_seqlens=cu)
    else:
        cu = list(wl.expected_cu_seqlens)
        lay = _layout(name)
    rows = ci_sample_rows(lay)
    _attn_case(jav, n, H, 128, cu, "bf16", variant == "varlen_causal", 240, rows=rows,
               label=variant)


# ---------------------------------------------------------------------------
# qkv_project / out_proj_gated
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,bias", [("tiny", False), ("tiny", True), ("small", True),
                                       ("medium", False), ("full", False)])
def test_qkv_project_parity(jav, name, bias):
    import torch
    wl = synth.WORKLOADS[name]
    inp = synth.block_inputs(wl, with_bias=True) if bias else _inputs(name)
    n, d = wl.n_tokens, wl.d_model
    print(f"qkv {name} bias={bias}", flush=True)
    y_h = synth.normal_array((n, d), seed=300 + wl.seed, dtype=wl.dtype)
    out = jav.qkv_project(dev(y_h, wl.dtype), dev(inp.w_qkv, wl.dtype),
                          dev(inp.b_qkv, wl.dtype) if bias else None)
    _sync()
    rows = None if n <= 4096 else sample_rows([0, n], n, limit=700)
    ref = oracle.qkv_project(y_h if rows is None else y_h[rows], inp.w_qkv,
                             inp.b_qkv if bias else None)
    got = host(out) if rows is None else host(out[torch.from_numpy(rows).cuda()])
    check(got, ref, wl.dtype, f"qkv[{name}]")


@pytest.mark.parametrize("d,n", [(64, 300), (1600, 777)])
def test_gemm_odd_depths_and_ragged_tiles(jav, d, n):
    """d_model 64 (a single k-step) and 1600 (25 k-steps, an odd count); token
    and feature counts that leave partial 256-wide tiles; bias and the gated
    residual with per-row modalities."""
    import torch
    print(f"gemm d={d} n={n}", flush=True)
    y_h = synth.normal_array((n, d), seed=310 + d, dtype="bf16")
    w_qkv = synth.normal_array((3 * d, d), seed=311 + d, std=0.02, dtype="bf16")
    b_qkv = synth.normal_array((3 * d,), seed=312 + d, std=0.1, dtype="bf16")
    out = jav.qkv_project(dev(y_h, "bf16"), dev(w_qkv, "bf16"), dev(b_qkv, "bf16"))
    _sync()
    check(host(out), oracle.qkv_project(y_h, w_qkv, b_qkv), "bf16", f"qkv d={d}")
    w_o = synth.normal_array((d, d), seed=313 + d, std=0.02, dtype="bf16")
    x_h = synth.normal_array((n, d), seed=314 + d, dtype="bf16")
    table = synth.normal_array((3, 3, d), seed=315 + d, std=0.1)
    mod = synth.uniform_ints((n,), 0, 3, seed=316 + d).astype(np.uint8)
    res = jav.out_proj_gated(dev(y_h, "bf16"), dev(w_o, "bf16"), dev(x_h, "bf16"),
                             dev_int(mod, torch.uint8), dev_f32(table))
    _sync()
    check(host(res), oracle.out_proj_gated(y_h, w_o, x_h, mod, table), "bf16", f"out d={d}")


@pytest.mark.parametrize("name,bias,inplace", [("tiny", True, False), ("small", False, False),
                                               ("small", True, True), ("medium", False, False),
                                               ("full", False, True)])
def test_out_proj_gated_parity(jav, name, bias, inplace):
    import torch
    wl = synth.WORKLOADS[name]
    inp = synth.block_inputs(wl, with_bias=True) if bias else _inputs(name)
    lay = _layout(name)
    mod_d, _, _, _ = _dev_layout(jav, name)
    n, d = wl.n_tokens, wl.d_model
    print(f"out_proj {name} bias={bias} inplace={inplace}", flush=True)
    o_h = synth.normal_array((n, d), seed=400 + wl.seed, dtype=wl.dtype)
    x_h = inp.x
    x = dev(x_h, wl.dtype)
    out = jav.out_proj_gated(dev(o_h, wl.dtype), dev(inp.w_o, wl.dtype), x, mod_d,
                             dev_f32(inp.table), dev(inp.b_o, wl.dtype) if bias else None,
                             out=x if inplace else None)
    _sync()
    rows = None if n <= 4096 else ci_sample_rows(lay)
    ref = oracle.out_proj_gated(o_h if rows is None else o_h[rows], inp.w_o, x_h,
                                lay["modality"], inp.table, inp.b_o if bias else None, rows=rows)
    got = host(out) if rows is None else host(out[torch.from_numpy(rows).cuda()])
    check(got, ref, wl.dtype, f"out_proj[{name}]")
    # the branch alone (out - x), where the residual does not hide errors
    if rows is None and wl.dtype == "f32":
        check(got - np.asarray(x_h, np.float64)[: n], ref - x_h, wl.dtype, "branch")


# ---------------------------------------------------------------------------
# dit_block_forward
# ---------------------------------------------------------------------------

_REF_CACHE = {}


def _oracle_block(name, causal, with_bias, rows):
    """The oracle's block from the original inputs.  The bidirectional run is
    kept for the workload (y, k, v, k' and the sampled q' do not depend on the
    mask), and the causal form reuses its stages: attention with the causal
    mask, then the gated output projection."""
    wl = synth.WORKLOADS[name]
    inp = synth.block_inputs(wl, with_bias=True) if with_bias else _inputs(name)
    lay = _layout(name)
    key = (name, with_bias, None if rows is None else rows.tobytes())
    base = _REF_CACHE.get(key)
    if base is None:
        _REF_CACHE.clear()
        base = oracle.block_forward(inp.x, lay["modality"], lay["pos"], lay["cu_seqlens"],
                                    inp.table, inp.w_qkv, inp.w_o, n_heads=wl.n_heads,
                                    head_dim=wl.head_dim, sections=wl.sections, theta=wl.theta,
                                    eps=wl.eps, causal=False,
                                    b_qkv=inp.b_qkv if with_bias else None,
                                    b_o=inp.b_o if with_bias else None, rows=rows)
        _REF_CACHE[key] = base
    if not causal:
        return base
    o = oracle.attention(base["q_rot"], base["k_rot"], base["v"], lay["cu_seqlens"], wl.n_heads,
                         wl.head_dim, True, rows=rows)
    out = oracle.out_proj_gated(o, inp.w_o, inp.x, lay["modality"], inp.table,
                                inp.b_o if with_bias else None, rows=rows)
    return dict(base, o=o, out=out)


def _block(jav, name, causal=False, with_bias=False, rows=None):
    """dit_block_forward against the oracle, every stage checked twice (on every
    row, or on `rows`):

    * per stage, from the GPU's own input to that stage, so roundings do not
      compound: y = AdaLN(x); q', k', v = RoPE(QKV(y)); o = attention(q', k',
      v) inside the cu_seqlens segments; out = x + gate * to_out.0(o);
    * end to end, the block's output against the oracle run from the original
      inputs.

    The output alone is dominated by the residual x: a block without RoPE or with
    a wrong mask still comes within tolerance on out (test_oracle_block.py), so
    the per-stage q', k' and o checks are the sensitive ones."""
    import torch
    wl = synth.WORKLOADS[name]
    inp = synth.block_inputs(wl, with_bias=True) if with_bias else _inputs(name)
    lay = _layout(name)
    mod_d, pos_d, cu_d, ms = _dev_layout(jav, name)
    n, d, H, Dh = wl.n_tokens, wl.d_model, wl.n_heads, wl.head_dim
    code = jav.DIT_BF16 if wl.dtype == "bf16" else jav.DIT_F32
    desc = jav.block_desc(code, d, H, Dh, wl.sections, wl.theta, wl.eps, causal=causal)
    nrows = n if rows is None else len(rows)
    print(f"block {name} causal={causal} bias={with_bias} rows={nrows}", flush=True)
    x = dev(inp.x, wl.dtype)
    ws = torch.empty(jav.block_workspace_bytes(desc, n), dtype=torch.uint8, device="cuda")
    out = jav.block_forward(desc, x, mod_d, pos_d, cu_d, ms, dev_f32(inp.table),
                            dev(inp.w_qkv, wl.dtype), dev(inp.w_o, wl.dtype),
                            b_qkv=dev(inp.b_qkv, wl.dtype) if with_bias else None,
                            b_o=dev(inp.b_o, wl.dtype) if with_bias else None, workspace=ws)
    _sync()
    planes = jav.block_planes(desc, ws, n)
    idx = None if rows is None else torch.from_numpy(rows).cuda()
    sel = np.arange(n) if rows is None else rows

    def got(t):
        return host(t) if idx is None else host(t[idx])

    tag = f"block[{name}{' causal' if causal else ''}]"
    b_qkv = inp.b_qkv if with_bias else None
    b_o = inp.b_o if with_bias else None
    # per stage
    check(got(planes["y"]), oracle.adaln_modulate(inp.x, lay["modality"], inp.table, wl.eps,
                                                  rows=rows), wl.dtype, f"{tag}.y")
    qkv = oracle.qkv_project(got(planes["y"]), inp.w_qkv, b_qkv)
    pos = np.asarray(lay["pos"])[sel]
    check(got(planes["q_rot"]), oracle.rope3d(qkv[:, :d], pos, H, Dh, wl.sections, wl.theta),
          wl.dtype, f"{tag}.q'")
    check(got(planes["k_rot"]), oracle.rope3d(qkv[:, d:2 * d], pos, H, Dh, wl.sections, wl.theta),
          wl.dtype, f"{tag}.k'")
    check(got(planes["v"]), qkv[:, 2 * d:], wl.dtype, f"{tag}.v")
    del qkv
    o_ref = oracle.attention(host(planes["q_rot"]), host(planes["k_rot"]), host(planes["v"]),
                             lay["cu_seqlens"], H, Dh, causal, rows=rows)
    o_got = got(planes["o"])
    check(o_got, o_ref, wl.dtype, f"{tag}.o")
    check(got(out), oracle.out_proj_gated(o_got, inp.w_o, inp.x, lay["modality"], inp.table, b_o,
                                          rows=rows), wl.dtype, f"{tag}.out (stage)")
    # end to end
    ref = _oracle_block(name, causal, with_bias, rows)
    check(got(out), ref["out"], wl.dtype, f"{tag}.out")
    if wl.dtype == "f32":
        # The branch alone, out - x = gate * (o W_o^T + b), where x does not hide
        # errors.  It is read back from the stored out, whose float32 rounding
        # (at most 2^-24 |out| per element) is large against a branch about
        # 1e-3 of |out|: the bound is 1e-5 plus that rounding's norm relative
        # to the branch's.
        gb = got(out) - np.asarray(inp.x, np.float64)[sel]
        rb = ref["out"] - np.asarray(inp.x, np.float64)[sel]
        bound = 1e-5 + np.linalg.norm(2.0 ** -24 * np.abs(ref["out"])) / np.linalg.norm(rb)
        r = rel_l2(gb, rb)
        print(f"  {tag}.branch: rel_l2={r:.3e} (bound {bound:.2e})", flush=True)
        assert r <= bound, (tag, r, bound)
    return out, planes, ws, desc


def _assert_unrotated_bits(jav, name, planes, ws, desc, with_bias=False):
    """The rotation leaves what it must not touch bit for bit: v, and the h and w
    sections of q and k on audio and text rows (their h = w = 0).  Reference: the
    standalone QKV projection of the AdaLN output y the block left in its
    workspace (the same GEMM, so the same bits before any rotation)."""
    import torch
    wl = synth.WORKLOADS[name]
    n, d, H, Dh = wl.n_tokens, wl.d_model, wl.n_heads, wl.head_dim
    inp = synth.block_inputs(wl, with_bias=True) if with_bias else _inputs(name)
    qkv = jav.qkv_project(planes["y"], dev(inp.w_qkv, wl.dtype),
                          dev(inp.b_qkv, wl.dtype) if with_bias else None)
    _sync()
    ibits = torch.int16 if wl.dtype == "bf16" else torch.int32
    assert torch.equal(planes["v"].view(ibits), qkv[:, 2 * d:].contiguous().view(ibits))
    mod = np.asarray(_layout(name)["modality"])
    at = torch.from_numpy(np.nonzero(mod != 0)[0]).cuda()
    s_t = wl.sections[0]
    for plane, lo in (("q_rot", 0), ("k_rot", d)):
        a = planes[plane].view(n, H, Dh)[at][:, :, s_t:].contiguous()
        b = qkv[:, lo:lo + d].reshape(n, H, Dh)[at][:, :, s_t:].contiguous()
        assert torch.equal(a.view(ibits), b.view(ibits)), plane


def test_block_tiny_f32(jav):
    _block(jav, "tiny")
    _block(jav, "tiny", causal=True, with_bias=True)


def test_block_small_bf16(jav):
    rows = ci_sample_rows(_layout("small"))
    _, planes, ws, desc = _block(jav, "small", rows=rows)
    _assert_unrotated_bits(jav, "small", planes, ws, desc)


def test_block_small_bias_causal(jav):
    rows = ci_sample_rows(_layout("small"))
    _, planes, ws, desc = _block(jav, "small", causal=True, with_bias=True, rows=rows)
    _assert_unrotated_bits(jav, "small", planes, ws, desc, with_bias=True)


def test_block_medium_sampled(jav):
    _block(jav, "medium", rows=ci_sample_rows(_layout("medium")))


@pytest.mark.parametrize("causal", [False, True])
def test_block_varlen_pack_sampled(jav, causal):
    """The 4-request pack (14,690 / 14,690 / 14,689 / 14,689 tokens), each
    request attending only inside its own cu_seqlens segment."""
    _block(jav, "varlen", causal=causal, rows=ci_sample_rows(_layout("varlen")))


def test_block_full_shape_sampled(jav):
    """58,758 tokens on the CI sample: segment edges, every text row, the first and
    last audio frame of both channels, the modality boundaries, every 97th row."""
    rows = ci_sample_rows(_layout("full"))
    _, planes, ws, desc = _block(jav, "full", rows=rows)
    _assert_unrotated_bits(jav, "full", planes, ws, desc)


def test_block_poison_tail_and_determinism(jav):
    """Buffers of 58,816 rows whose last 58 rows are NaN give finite outputs that are
    bit-identical to the unpadded run, leave the tail untouched, and repeat exactly."""
    import torch
    wl = synth.WORKLOADS["full"]
    n, d = wl.n_tokens, wl.d_model
    inp = _inputs("full")
    mod_d, pos_d, cu_d, ms = _dev_layout(jav, "full")
    desc = jav.block_desc(jav.DIT_BF16, d, wl.n_heads, wl.head_dim, wl.sections)
    x = dev(inp.x, "bf16")
    tab, wq, wo = dev_f32(inp.table), dev(inp.w_qkv, "bf16"), dev(inp.w_o, "bf16")
    print("block poison", flush=True)
    out_ref = jav.block_forward(desc, x, mod_d, pos_d, cu_d, ms, tab, wq, wo)
    out_rep = jav.block_forward(desc, x, mod_d, pos_d, cu_d, ms, tab, wq, wo)
    pad = synth.FULL_ALIGNED_TOKENS
    xp = torch.full((pad, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    xp[:n] = x
    modp = torch.zeros(pad, dtype=torch.uint8, device="cuda")
    modp[:n] = mod_d
    modp[n:] = 7                      # invalid ids in the padding must never be read
    posp = torch.full((pad, 3), -1, dtype=torch.int32, device="cuda")
    posp[:n] = pos_d
    outp = torch.full((pad, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(jav.block_workspace_bytes(desc, pad), dtype=torch.uint8, device="cuda")
    ws.view(torch.bfloat16)[:].fill_(float("nan"))
    jav.block_forward(desc, xp, modp, posp, cu_d, ms, tab, wq, wo, out=outp, workspace=ws,
                      n_tokens=n)
    _sync()
    assert torch.isfinite(outp[:n].float()).all()
    assert torch.equal(outp[:n].view(torch.int16), out_ref.view(torch.int16))
    assert torch.isnan(outp[n:].float()).all()
    assert torch.equal(out_rep.view(torch.int16), out_ref.view(torch.int16))


def test_validate_env_rejects_broken_device_arrays(jav):
    """DIT_VALIDATE=1: broken cu_seqlens or modality ids come back as DIT_EINVAL before any
    launch; valid arrays pass.  (The broken cases here are memory-safe even unchecked: the
    buffers cover every row a kernel could touch and the table is the front of a larger
    allocation.)"""
    import os
    import torch
    n, H = 512, 2
    q = torch.zeros((n, H * 128), dtype=torch.bfloat16, device="cuda")
    tab_big = torch.zeros((2, 3, 3, H * 128), dtype=torch.float32, device="cuda")
    cases = [([0, 300, 200, 400], 300, "decreases"), ([0, 200, 480], 280, "ends at"),
             ([0, 100, 400], 200, "max_seqlen"), ([5, 400], 395, "not 0")]
    old = os.environ.get("DIT_VALIDATE")
    os.environ["DIT_VALIDATE"] = "1"
    try:
        for cu, ms, msg in cases:
            cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
            with pytest.raises(jav.DitError) as ei:
                jav.attn_packed(q, q, q, cu_d, ms, H, 128, n_tokens=400)
            assert ei.value.status == jav.DIT_EINVAL and msg in str(ei.value), (cu, str(ei.value))
        jav.attn_packed(q, q, q, torch.tensor([0, 150, 400], dtype=torch.int32, device="cuda"),
                        250, H, 128, n_tokens=400)
        mod = torch.zeros(n, dtype=torch.uint8, device="cuda")
        mod[77] = 3
        with pytest.raises(jav.DitError) as ei:
            jav.adaln_modulate(q, mod, tab_big[0], n_tokens=400)
        assert "modality[77] = 3" in str(ei.value)
        mod[77] = 2
        jav.adaln_modulate(q, mod, tab_big[0], n_tokens=400)
        torch.cuda.synchronize()
    finally:
        if old is None:
            os.environ.pop("DIT_VALIDATE", None)
        else:
            os.environ["DIT_VALIDATE"] = old


def test_segment_longer_than_max_seqlen_becomes_nan(jav):
    """cu_seqlens breaking its contract (the second segment, 400 rows, is longer than
    the max_seqlen of 300 the grid is sized for; the rows lie inside the buffers, so
    the call is memory-safe): that segment's output rows and log-sum-exps come out NaN
    instead of partly unwritten, and the first segment is bit-identical to a call
    with the right max_seqlen."""
    import torch
    n, H = 700, 2
    cu = [0, 300, 700]
    q, k, v = (dev(synth.normal_array((n, H * 128), seed=260 + i, dtype="bf16"), "bf16")
               for i in range(3))
    cu_d = dev_int(np.array(cu, np.int32), torch.int32)
    good, lse_good = jav.attn_packed_lse(q, k, v, cu_d, 400, H, 128)
    bad = torch.zeros_like(good)
    bad, lse_bad = jav.attn_packed_lse(q, k, v, cu_d, 300, H, 128, out=bad)
    _sync()
    assert torch.equal(bad[:300].view(torch.int16), good[:300].view(torch.int16))
    assert torch.isnan(bad[300:].float()).all()
    assert torch.equal(lse_bad[:, :300], lse_good[:, :300])
    assert torch.isnan(lse_bad[:, 300:]).all()
