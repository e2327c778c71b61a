"""Parity of the FP8 entry points against the float64 oracle (MI355X only).

quantize_rows_fp8 must give the oracle's e4m3 codes and float32 scales bit for
bit (both take the rounding decision on the same float32 values).
linear_fp8 is compared with the oracle's product of the same codes and
scales: a bf16 output, so max-abs <= 3e-2 and rel-L2 <= 1e-2.  Shapes: the
workloads' QKV, out-proj and feed-forward projections (the full shape on
sampled rows), an odd number of k-steps with ragged tiles, biases, the gated
epilogue in place and the GELU epilogue.
"""
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


def _sync():
    import torch
    torch.cuda.synchronize()


def _codes_dev(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda()


@pytest.mark.parametrize("shape,dtype", [((328, 256), "f32"), ((4096, 1536), "bf16"),
                                         ((1000, 20480), "bf16"), ((37, 5120), "bf16")])
def test_quantize_rows_bit_exact(jav, shape, dtype):
    import torch
    n, d = shape
    x = synth.normal_array(shape, 700 + d, dtype=dtype) * np.float32(4.0)   # stays bf16-exact
    x[0] = 0.0                                   # an all-zero row: scale 1, codes 0
    x[1, :8] = np.float32(2.0 ** -12)            # tiny values: subnormal codes and zeros
    x[2, 8:16] = np.float32(0.0)                 # zeros inside a row
    codes, scales = jav.quantize_rows_fp8(dev(x, dtype))
    _sync()
    ref_codes, ref_scales = oracle.quantize_rows(x)
    np.testing.assert_array_equal(scales.cpu().numpy(), ref_scales)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_codes)


def _codes(shape, seed):
    """e4m3 codes of N(0, 1) values scaled so the row maxima sit near 448, drawn from
    a pool of one million encoded values (the full-shape operands have 3e8 codes)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pool = oracle.e4m3_encode(synth.normal_array((1 << 20,), seed) * np.float32(448.0 / 4.5))
    return pool[rng.integers(0, pool.size, size=shape)]


def _inputs(n, k, f, seed, bias=False):
    """Codes and scales as a per-row quantization of the workloads' values would give
    them: activation rows N(0, 1) (scale about 4.5 / 448), weight rows N(0, 0.02^2)."""
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    ac = _codes((n, k), seed)
    wc = _codes((f, k), seed + 1)
    asc = (rng.uniform(0.95, 1.05, n) * 4.5 / 448).astype(np.float32)
    wsc = (rng.uniform(0.95, 1.05, f) * 0.02 * 4.5 / 448).astype(np.float32)
    b = synth.normal_array((f,), seed + 2, std=0.02, dtype="bf16") if bias else None
    return ac, asc, wc, wsc, b


@pytest.mark.parametrize("n,k,f,bias", [(328, 256, 768, True), (4096, 1536, 4608, False),
                                        (1000, 1664, 1000, True), (58758, 5120, 15360, False)])
def test_linear_fp8_plain(jav, n, k, f, bias):
    import torch
    print(f"linear_fp8 plain n={n} k={k} f={f}", flush=True)
    ac, asc, wc, wsc, b = _inputs(n, k, f, 710 + f, bias)
    out = jav.linear_fp8(_codes_dev(ac), dev_f32(asc), _codes_dev(wc), dev_f32(wsc),
                         None if b is None else dev(b, "bf16"))
    _sync()
    rows = None if n <= 4096 else sample_rows([0, n], n, limit=400)
    ra = ac if rows is None else ac[rows]
    rs = asc if rows is None else asc[rows]
    ref = oracle.linear_fp8(ra, rs, wc, wsc, b)
    got = host(out) if rows is None else host(out[torch.from_numpy(rows).cuda()])
    check(got, ref, "bf16", f"linear_fp8 {n}x{k}x{f}")


@pytest.mark.parametrize("name", ["small", "medium"])
def test_linear_fp8_gated_in_place_and_gelu(jav, name):
    import torch
    wl = synth.WORKLOADS[name]
    n, d = wl.n_tokens, wl.d_model
    lay = oracle.pack_layout([r.grid for r in wl.requests])
    mod = np.asarray(lay["modality"], dtype=np.uint8)
    table = synth.normal_array((3, 3, d), 720, std=0.1)
    x = synth.normal_array((n, d), 721, dtype="bf16")
    # gated: out = x + gate[m] * (o W^T), written over x
    ac, asc, wc, wsc, b = _inputs(n, d, d, 722, bias=True)
    xd = dev(x, "bf16")
    jav.linear_fp8(_codes_dev(ac), dev_f32(asc), _codes_dev(wc), dev_f32(wsc), dev(b, "bf16"),
                   epilogue="gated", x=xd, modality=dev_int(mod, torch.uint8),
                   table=dev_f32(table), out=xd)
    _sync()
    prod = oracle.linear_fp8(ac, asc, wc, wsc, b)
    ref = x.astype(np.float64) + table[mod, 2, :] * prod
    check(host(xd), ref, "bf16", f"linear_fp8 gated {name}")
    # GELU (tanh form) of the product, a 4 d_model wide output
    ac, asc, wc, wsc, b = _inputs(n, d, 4 * d, 723, bias=False)
    out = jav.linear_fp8(_codes_dev(ac), dev_f32(asc), _codes_dev(wc), dev_f32(wsc),
                         epilogue="gelu")
    _sync()
    rows = sample_rows([0, n], n, limit=500)
    ref = oracle.gelu_tanh(oracle.linear_fp8(ac[rows], asc[rows], wc, wsc))
    check(host(out[torch.from_numpy(rows).cuda()]), ref, "bf16", f"linear_fp8 gelu {name}")


def test_fp8_projection_error_against_bf16(jav):
    """The FP8 path as a whole (GPU quantization of bf16 rows, then the FP8 product)
    against the unquantized float64 product: the error that e4m3's 3-bit mantissa
    costs, bounded by the derived tolerance rel-L2 <= 5e-2 (per-value relative error
    at most 1/16, about 1/(16 sqrt(3)) in RMS for each operand)."""
    import torch
    n, k, f = 2048, 1536, 1536
    a = synth.normal_array((n, k), 730, dtype="bf16")
    w = synth.normal_array((f, k), 731, std=0.02, dtype="bf16")
    ac, asc = jav.quantize_rows_fp8(dev(a, "bf16"))
    wc, wsc = jav.quantize_rows_fp8(dev(w, "bf16"))
    out = jav.linear_fp8(ac, asc, wc, wsc)
    _sync()
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    got = host(out)
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"  fp8 vs exact bf16 product: rel_l2={rel:.3e}", flush=True)
    assert rel <= 5e-2


# ---------------------------------------------------------------------------
# FP8 block halves
# ---------------------------------------------------------------------------

def _round256(b):
    return (b + 255) // 256 * 256


def _spacing(v):
    """e4m3 spacing at |v| (code units, before scaling)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
    return 2.0 ** (e - 3)


def _check_codes(got, ref, what, max_frac):
    """Codes equal, except where the two sides' float32 values straddle a rounding
    boundary: there the codes must be neighbours (one e4m3 step apart)."""
    tab = oracle.e4m3_table()
    got = np.asarray(got, np.uint8)
    ref = np.asarray(ref, np.uint8)
    bad = got != ref
    frac = float(bad.mean()) if bad.size else 0.0
    print(f"  {what}: code mismatches {frac:.2e}", flush=True)
    if bad.any():
        vg, vr = tab[got[bad]], tab[ref[bad]]
        assert np.all(np.isfinite(vg))
        assert np.all(np.abs(vg - vr) <= _spacing(np.maximum(np.abs(vg), np.abs(vr))) * (1 + 1e-9))
    assert frac <= max_frac, (what, frac)


# Output tolerance of an FP8 half against the oracle's FP8 half: the two sides
# quantize intermediates (o, h) that differ by their bf16 error, so about 2% of
# the codes sit one e4m3 step (2^-3 relative) apart.  Over K = 20480 operands
# that gives the branch an RMS error of sqrt(0.02 K) 2^-3 rms(h) rms(w) ~ 0.05,
# times |gate| <= 0.4 and 4.5 sigma over the sampled outputs: max-abs 0.1.  The
# rel-L2 bound stays the bf16 one.
FP8_HALF_MAX_ABS = 1e-1


def _check_fp8_out(got, ref, what):
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(np.asarray(got) - np.asarray(ref))))
    print(f"  {what}: rel_l2={r:.3e} max_abs={m:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert r <= 1e-2 and m <= FP8_HALF_MAX_ABS, (what, r, m)


def _check_quantized(codes, scales, vals, ref_codes, what, max_frac):
    """Codes and scales the library wrote for its own bf16 values: each scale is the
    row's float32 amax / 448 and each code a nearest rounding of value / scale (within
    half an e4m3 step).  Against the oracle's codes of its float64 values, only the
    fraction that differs is bounded: the two sides round values that differ by the
    bf16 error of the attention (or projection) output, often across a rounding
    boundary near zero, where the e4m3 steps are finest."""
    tab = oracle.e4m3_table()
    vals = np.asarray(vals, np.float32)
    amax = np.abs(vals).max(axis=1)
    want = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
    np.testing.assert_array_equal(scales, want)
    s = scales.astype(np.float64)[:, None]
    u = vals.astype(np.float64) / s
    assert np.all(np.abs(tab[codes] - u) <= 0.5 * _spacing(u) * (1 + 1e-6) + 1e-12), what
    frac = float(np.mean(codes != ref_codes))
    print(f"  {what}: codes differing from the oracle's {frac:.2e}", flush=True)
    assert frac <= max_frac, (what, frac)


def _fp8_layout(jav, name, n=None, cu=None):
    """Device and oracle layouts of a workload, optionally cut to the first n rows with
    the segment offsets cu."""
    import torch
    wl = synth.WORKLOADS[name]
    grids = [r.grid for r in wl.requests]
    lay_d = jav.pack_layout(grids)
    lay = oracle.pack_layout(grids)
    n = wl.n_tokens if n is None else n
    cu = list(lay["cu_seqlens"]) if cu is None else list(cu)
    mod, pos = np.asarray(lay["modality"])[:n], np.asarray(lay["pos"])[:n]
    dev_lay = (dev_int(np.asarray(lay_d["modality"])[:n], torch.uint8),
               dev_int(np.asarray(lay_d["pos"])[:n], torch.int32),
               dev_int(np.asarray(cu), torch.int32), int(max(b - a for a, b in zip(cu, cu[1:]))))
    return mod, pos, cu, dev_lay


@pytest.mark.parametrize("name,n", [("tiny", None), ("small", 1000), ("full", None)])
def test_adaln_fp8_codes_and_scales(jav, name, n):
    import torch
    wl = synth.WORKLOADS[name]
    inp = synth.block_inputs(wl, n_tokens=n)
    mod, _, _, (mod_d, _, _, _) = _fp8_layout(jav, name, n=inp.x.shape[0],
                                              cu=[0, inp.x.shape[0]])
    print(f"adaln_fp8 {name} n={inp.x.shape[0]}", flush=True)
    codes, scales = jav.adaln_modulate_fp8(dev(inp.x, wl.dtype), mod_d, dev_f32(inp.table),
                                           eps=wl.eps)
    _sync()
    rows = None if inp.x.shape[0] <= 4096 else sample_rows([0, inp.x.shape[0]], inp.x.shape[0],
                                                           limit=3000)
    ref_c, ref_s = oracle.adaln_modulate_fp8(inp.x, mod, inp.table, wl.eps, rows=rows)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    if rows is not None:
        got_c, got_s = got_c[rows], got_s[rows]
    np.testing.assert_allclose(got_s, ref_s, rtol=1e-5)
    _check_codes(got_c, ref_c, f"adaln_fp8[{name}]", 1e-3)


# With the attention in FP8 the GPU rounds the probabilities to e4m3, which
# the oracle (exact probabilities) does not: o's relative L2 error is then
# about 0.026-0.036 (the bound of the FP8 attention tests is 0.05), plus the
# operands' own rounding (bf16 q, k, v on the GPU, float64 in the oracle) at
# code boundaries: o within 0.06, its row scales within 10%, and its codes are
# checked against the GPU's own o values only.
FP8_ATTN_O_REL_L2 = 6e-2


_FP8_REF = {}


def _oracle_block_fp8(name, inp, mod, pos, cu, wq, wo, wl, causal, with_bias, rows,
                      fp8_attention):
    """oracle.block_forward_fp8; at the full shape the run with bf16 attention is
    kept, and the FP8-attention form reuses its stages (the FP8 AdaLN, both
    projections' operands, q', k', v) and applies the rest of the definition:
    attention_fp8, o's per-row quantization, to_out.0 in FP8 and the gate."""
    b_qkv = inp.b_qkv if with_bias else None
    b_o = inp.b_o if with_bias else None
    if name != "full":
        return oracle.block_forward_fp8(inp.x, mod, pos, cu, inp.table, *wq, *wo,
                                        n_heads=wl.n_heads, head_dim=wl.head_dim,
                                        sections=wl.sections, theta=wl.theta, eps=wl.eps,
                                        causal=causal, b_qkv=b_qkv, b_o=b_o, rows=rows,
                                        fp8_attention=fp8_attention)
    key = (name, tuple(cu), causal, with_bias, None if rows is None else rows.tobytes())
    base = _FP8_REF.get(key)
    if base is None:
        _FP8_REF.clear()
        base = oracle.block_forward_fp8(inp.x, mod, pos, cu, inp.table, *wq, *wo,
                                        n_heads=wl.n_heads, head_dim=wl.head_dim,
                                        sections=wl.sections, theta=wl.theta, eps=wl.eps,
                                        causal=causal, b_qkv=b_qkv, b_o=b_o, rows=rows)
        _FP8_REF[key] = base
    if not fp8_attention:
        return base
    o = oracle.attention_fp8(base["q_rot"], base["k_rot"], base["v"], cu, wl.n_heads,
                             wl.head_dim, causal, rows=rows)["o"]
    oc, os_ = oracle.quantize_rows(o)
    out = oracle.out_proj_gated(oracle.dequantize_rows(oc, os_), oracle.dequantize_rows(*wo),
                                inp.x, mod, inp.table, b_o, rows)
    return dict(base, o=o, o_codes=oc, o_scales=os_, out=out)


def _check_o_scales(o_scales, o_h, ref, what):
    """o's row scales: exactly amax / 448 of the GPU's own o rows (float32, R33),
    and within the oracle's by what o's own error allows: a row maximum moves by
    at most the row's largest element error (it is 1-Lipschitz in the max norm),
    so |s - s_ref| <= max_j |o_j - o_ref_j| / 448, plus three float32 roundings
    (o to float32 in the oracle, and each side's division by 448), within
    2^-21 |s_ref|."""
    np.testing.assert_array_equal(o_scales, oracle.row_scales(o_h))
    err = np.max(np.abs(o_h - ref["o"]), axis=1) / oracle.E4M3_MAX
    gap = np.abs(o_scales.astype(np.float64) - ref["o_scales"].astype(np.float64))
    slack = 2.0 ** -21 * np.abs(ref["o_scales"].astype(np.float64))
    worst = float(np.max(gap - err - slack))
    print(f"  {what}.o_scales: max gap {float(gap.max()):.3e} (worst margin {worst:.3e})", flush=True)
    assert worst <= 0.0, (what, worst)


def _block_fp8(jav, name, n=None, cu=None, rows=None, with_bias=False, causal=False,
               inplace=False, fp8_attention=False):
    import torch
    wl = synth.WORKLOADS[name]
    inp = synth.block_inputs(wl, n_tokens=n, with_bias=with_bias)
    n = inp.x.shape[0]
    mod, pos, cu, (mod_d, pos_d, cu_d, ms) = _fp8_layout(jav, name, n=n, cu=cu)
    wq = oracle.quantize_rows(inp.w_qkv)
    wo = oracle.quantize_rows(inp.w_o)
    desc = jav.block_desc(jav.DIT_BF16, wl.d_model, wl.n_heads, wl.head_dim, wl.sections,
                          wl.theta, wl.eps, causal=causal)
    need = (jav.block_fp8_attn_workspace_bytes(desc, n, len(cu) - 1) if fp8_attention
            else jav.block_fp8_workspace_bytes(desc, n))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    print(f"block_fp8 {name} n={n} segs={len(cu) - 1} bias={with_bias} causal={causal} "
          f"inplace={inplace} fp8_attention={fp8_attention}", flush=True)
    x = dev(inp.x, "bf16")
    out = jav.block_forward_fp8(desc, x, mod_d, pos_d, cu_d, ms, dev_f32(inp.table),
                                _codes_dev(wq[0]), dev_f32(wq[1]), _codes_dev(wo[0]),
                                dev_f32(wo[1]),
                                b_qkv=dev(inp.b_qkv, "bf16") if with_bias else None,
                                b_o=dev(inp.b_o, "bf16") if with_bias else None,
                                out=x if inplace else None, workspace=ws,
                                fp8_attention=fp8_attention)
    _sync()
    ref = _oracle_block_fp8(name, inp, mod, pos, cu, wq, wo, wl, causal, with_bias, rows,
                            fp8_attention)
    idx = np.arange(n) if rows is None else rows
    d = wl.d_model
    plane = _round256(n * d * 2)
    # after the call the workspace holds o (plane 4), o's codes (plane 0) and o's scales
    o = ws[4 * plane:4 * plane + n * d * 2].view(torch.bfloat16).view(n, d)
    o_codes = ws[:n * d].view(n, d).cpu().numpy()[idx]
    o_scales = ws[5 * plane:5 * plane + 4 * n].view(torch.float32).cpu().numpy()[idx]
    o_h = host(o)[idx]
    if fp8_attention:
        r = rel_l2(o_h, ref["o"])
        print(f"  block_fp8[{name}].o (fp8 attention): rel_l2={r:.3e}", flush=True)
        assert np.isfinite(o_h).all() and r <= FP8_ATTN_O_REL_L2, r
        _check_o_scales(o_scales, o_h, ref, f"block_fp8[{name}]")
        _check_quantized(o_codes, o_scales, o_h, ref["o_codes"], f"block_fp8[{name}].o_codes", 1.0)
    else:
        check(o_h, ref["o"], "bf16", f"block_fp8[{name}].o")
        _check_o_scales(o_scales, o_h, ref, f"block_fp8[{name}]")
        _check_quantized(o_codes, o_scales, o_h, ref["o_codes"], f"block_fp8[{name}].o_codes", 0.1)
    _check_fp8_out(host(out)[idx], ref["out"], f"block_fp8[{name}].out")
    return out


def test_block_fp8_small(jav):
    _block_fp8(jav, "small")


def test_block_fp8_ragged_segments_bias_causal_inplace(jav):
    _block_fp8(jav, "small", n=1000, cu=[0, 617, 1000], with_bias=True, causal=True,
               inplace=True)


@pytest.mark.parametrize("case", ["small", "ragged_bias_causal_inplace"])
def test_block_fp8_with_fp8_attention(jav, case):
    if case == "small":
        _block_fp8(jav, "small", fp8_attention=True)
    else:
        _block_fp8(jav, "small", n=1000, cu=[0, 617, 1000], with_bias=True, causal=True,
                   inplace=True, fp8_attention=True)


@pytest.mark.parametrize("fp8_attention", [False, True])
def test_block_fp8_full_shape_sampled(jav, fp8_attention):
    """The attention half with FP8 projections (and FP8 attention) at 58,758 tokens
    against the oracle on the CI row sample: o, its codes and scales, and out."""
    layout = oracle.pack_layout([r.grid for r in synth.WORKLOADS["full"].requests])
    _block_fp8(jav, "full", rows=ci_sample_rows(layout), fp8_attention=fp8_attention)


def _weights(f, k, seed):
    """Weight codes and scales of a per-row quantization of N(0, 0.02^2) rows."""
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    return _codes((f, k), seed), (rng.uniform(0.95, 1.05, f) * 0.02 * 4.5 / 448).astype(np.float32)


@pytest.mark.parametrize("fp8_attention", [False, True])
def test_block_fp8_full_shape_equals_its_stages(jav, fp8_attention):
    """At the full shape (a 3 GB workspace) the fused entry point gives bit for bit
    what its stages give when called one by one on separate buffers; each stage
    has its own full-shape parity test against the oracle.  (The oracle needs
    every row's keys and values for one query, minutes of float64 work here.)"""
    import torch
    wl = synth.WORKLOADS["full"]
    n, d, H, Dh = wl.n_tokens, wl.d_model, wl.n_heads, wl.head_dim
    _, _, cu, (mod_d, pos_d, cu_d, ms) = _fp8_layout(jav, "full")
    print(f"block_fp8 full n={n} fp8_attention={fp8_attention}: fused vs stages", flush=True)
    x = dev(synth.normal_array((n, d), seed=900, dtype="bf16"), "bf16")
    table = dev_f32(synth.normal_array((3, 3, d), seed=901, std=0.1))
    wqc, wqs = _weights(3 * d, d, 902)
    woc, wos = _weights(d, d, 903)
    b_qkv = dev(synth.normal_array((3 * d,), seed=904, std=0.02, dtype="bf16"), "bf16")
    b_o = dev(synth.normal_array((d,), seed=905, std=0.02, dtype="bf16"), "bf16")
    wqc, wqs, woc, wos = _codes_dev(wqc), dev_f32(wqs), _codes_dev(woc), dev_f32(wos)
    desc = jav.block_desc(jav.DIT_BF16, d, H, Dh, wl.sections, wl.theta, wl.eps)
    fused = jav.block_forward_fp8(desc, x, mod_d, pos_d, cu_d, ms, table, wqc, wqs, woc, wos,
                                  b_qkv=b_qkv, b_o=b_o, fp8_attention=fp8_attention)
    _sync()
    yc, ys = jav.adaln_modulate_fp8(x, mod_d, table, eps=wl.eps)
    qkv = jav.linear_fp8(yc, ys, wqc, wqs, bias=b_qkv)
    q_r = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    k_r = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    jav.rope3d_apply_to(qkv[:, :d], qkv[:, d:2 * d], q_r, k_r, pos_d, H, Dh, wl.sections,
                        wl.theta)
    if fp8_attention:
        aws = jav.attn_fp8_prepare(q_r, k_r, qkv[:, 2 * d:], cu_d, ms, H)
        o = jav.attn_packed_fp8(aws, cu_d, ms, n, H)
    else:
        o = jav.attn_packed(q_r, k_r, qkv[:, 2 * d:], cu_d, ms, H, Dh)
    oc, os_ = jav.quantize_rows_fp8(o)
    staged = jav.linear_fp8(oc, os_, woc, wos, bias=b_o, epilogue="gated", x=x, modality=mod_d,
                            table=table)
    _sync()
    assert torch.isfinite(fused.float()).all()
    assert torch.equal(fused, staged)


def _ffn_fp8(jav, name, n=None, rows=None, with_bias=False, pool_weights=False):
    import torch
    wl = synth.WORKLOADS[name]
    f = synth.ffn_inputs(wl, with_bias=with_bias)
    x_h = synth.normal_array((wl.n_tokens, wl.d_model), seed=500 + wl.seed, dtype=wl.dtype)
    if n is not None:
        x_h = x_h[:n]
    n = x_h.shape[0]
    mod, _, _, (mod_d, _, _, _) = _fp8_layout(jav, name, n=n, cu=[0, n])
    if pool_weights:
        w1, w2 = _weights(wl.d_ff, wl.d_model, 906), _weights(wl.d_model, wl.d_ff, 907)
    else:
        w1, w2 = oracle.quantize_rows(f.w1), oracle.quantize_rows(f.w2)
    desc = jav.ffn_desc(jav.DIT_BF16, wl.d_model, wl.d_ff, wl.eps)
    ws = torch.empty(jav.ffn_fp8_workspace_bytes(desc, n), dtype=torch.uint8, device="cuda")
    print(f"ffn_fp8 {name} n={n} bias={with_bias}", flush=True)
    out = jav.ffn_forward_fp8(desc, dev(x_h, "bf16"), mod_d, dev_f32(f.table), _codes_dev(w1[0]),
                              dev_f32(w1[1]), _codes_dev(w2[0]), dev_f32(w2[1]),
                              b1=dev(f.b1, "bf16") if with_bias else None,
                              b2=dev(f.b2, "bf16") if with_bias else None, workspace=ws)
    _sync()
    ref = oracle.ffn_forward_fp8(x_h, mod, f.table, *w1, *w2, b1=f.b1 if with_bias else None,
                                 b2=f.b2 if with_bias else None, eps=wl.eps, rows=rows)
    idx = np.arange(n) if rows is None else rows
    F = wl.d_ff
    c0 = _round256(n * max(F, wl.d_model))
    # after the call the workspace holds h's codes, h and h's scales
    h = ws[c0:c0 + n * F * 2].view(torch.bfloat16).view(n, F)
    h_h = host(h)[idx]
    check(h_h, ref["h"], "bf16", f"ffn_fp8[{name}].h")
    sc0 = c0 + _round256(n * F * 2)
    h_scales = ws[sc0:sc0 + 4 * n].view(torch.float32).cpu().numpy()[idx]
    np.testing.assert_allclose(h_scales, ref["h_scales"], rtol=1e-2)
    _check_quantized(ws[:n * F].view(n, F).cpu().numpy()[idx], h_scales, h_h, ref["h_codes"],
                     f"ffn_fp8[{name}].h_codes", 0.1)
    _check_fp8_out(host(out)[idx], ref["out"], f"ffn_fp8[{name}].out")


def test_ffn_fp8_small_ragged_bias(jav):
    _ffn_fp8(jav, "small", n=1000, with_bias=True)


def test_ffn_fp8_full_shape_sampled(jav):
    """The half is row-local, so sampled rows of the oracle are cheap; the weights
    come as codes of a per-row quantization drawn from a pool (3e8 codes)."""
    wl = synth.WORKLOADS["full"]
    _ffn_fp8(jav, "full", rows=sample_rows([0, wl.n_tokens], wl.n_tokens, limit=200),
             pool_weights=True)


def test_ffn_fp8_equals_its_stages(jav):
    """The fused feed-forward half gives bit for bit what its stages give when called
    one by one (ragged rows, biases)."""
    import torch
    wl = synth.WORKLOADS["small"]
    n, d, F = 1000, wl.d_model, wl.d_ff
    f = synth.ffn_inputs(wl, with_bias=True)
    _, _, _, (mod_d, _, _, _) = _fp8_layout(jav, "small", n=n, cu=[0, n])
    print(f"ffn_fp8 small n={n}: fused vs stages", flush=True)
    x = dev(synth.normal_array((n, d), seed=910, dtype="bf16"), "bf16")
    table = dev_f32(f.table)
    w1c, w1s = oracle.quantize_rows(f.w1)
    w2c, w2s = oracle.quantize_rows(f.w2)
    w1c, w1s, w2c, w2s = _codes_dev(w1c), dev_f32(w1s), _codes_dev(w2c), dev_f32(w2s)
    b1, b2 = dev(f.b1, "bf16"), dev(f.b2, "bf16")
    desc = jav.ffn_desc(jav.DIT_BF16, d, F, wl.eps)
    fused = jav.ffn_forward_fp8(desc, x, mod_d, table, w1c, w1s, w2c, w2s, b1=b1, b2=b2)
    yc, ys = jav.adaln_modulate_fp8(x, mod_d, table, eps=wl.eps)
    h = jav.linear_fp8(yc, ys, w1c, w1s, bias=b1, epilogue="gelu")
    hc, hs = jav.quantize_rows_fp8(h)
    staged = jav.linear_fp8(hc, hs, w2c, w2s, bias=b2, epilogue="gated", x=x, modality=mod_d,
                            table=table)
    _sync()
    assert torch.isfinite(fused.float()).all()
    assert torch.equal(fused, staged)
