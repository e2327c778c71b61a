"""Parity of the FP8 attention (attn_fp8_prepare, attn_packed_fp8) with
oracle.attention_fp8 (MI355X only).

The operands must match bit for bit: q codes with their per-row scales, k and
v codes with the per-head scales, v's codes in the transposed layout (and
zero codes in each segment's padding).  Both sides take every rounding
decision on the same float32 values.

o is compared with the oracle's attention of the same dequantized operands
with exact probabilities.  The GPU rounds p' = 2^8 p (relative to the running
row maximum, at most 2^8.75) to e4m3, which moves a term by at most 2^-4 of
itself in the normal range and by 2^-18 of the largest |v| per key below it,
and stores o in bf16 (2^-9 relative); float32 accumulation over L keys adds a
relative error of about L 2^-24 at worst.  Hence, per element,
  |o - ref| <= (2^-4 + 1e-3) o_abs + L 2^-18 max|v| + 2^-8 |ref| + 1e-5,
with o_abs = sum_k P_k |v_k| / sum_k P_k from the oracle.  Over many elements
the rounding errors are independent: for zero-mean v the relative L2 error
is about 2^-4 / sqrt(3) times the RMS of 1 / mantissa, 0.026 to 0.036, and the
test bounds it by 0.05.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, dev_int, host, rel_l2, sample_rows

pytestmark = pytest.mark.gpu

FP8_ATTN_REL_L2 = 5e-2


@pytest.fixture(scope="module")
def jav():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import joint_audio_video_amd as m
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


def _cu(lens):
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    return cu


def _views(jav, ws, n, n_seqs, H):
    """Device views of the operand parts of an attn_fp8_prepare workspace."""
    import torch
    lay = jav.attn_fp8_layout(n, n_seqs, H)
    ld8, ld_vt = lay["ld8"], lay["ld_vt"]
    q8 = ws[lay["q8"]:lay["q8"] + n * ld8].view(n, ld8)
    k8 = ws[lay["k8"]:lay["k8"] + n * ld8].view(n, ld8)
    vt = ws[lay["vt"]:lay["vt"] + H * 128 * ld_vt].view(H * 128, ld_vt)
    sq = ws[lay["sq"]:lay["sq"] + 4 * H * n].view(torch.float32).view(H, n)
    sk = ws[lay["sk"]:lay["sk"] + 4 * H * n_seqs].view(torch.float32).view(n_seqs, H)
    sv = ws[lay["sv"]:lay["sv"] + 4 * H * n_seqs].view(torch.float32).view(n_seqs, H)
    return dict(q8=q8, k8=k8, vt=vt, sq=sq, sk=sk, sv=sv)


def _col0(cu, s):
    return (cu[s] + 63) // 64 * 64 + 128 * s


def _check_o(got, r, vmax, max_len, what):
    ref, o_abs = r["o"], r["o_abs"]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = (2.0 ** -4 + 1e-3) * o_abs + max_len * 2.0 ** -18 * vmax + 2.0 ** -8 * np.abs(ref) + 1e-5
    rl = rel_l2(got, ref)
    worst = float(np.max(err / bound)) if err.size else 0.0
    print(f"  {what}: rel_l2={rl:.3e} max_abs={float(err.max()):.3e} worst err/bound={worst:.3f}",
          flush=True)
    assert np.all(err <= bound), (what, worst)
    assert rl <= FP8_ATTN_REL_L2, (what, rl)


def _run(jav, q_h, k_h, v_h, cu, H, causal, rows=None, heads=None, label="", check_ops=True):
    """Prepare + attention on the GPU, the oracle on `heads` (all by default)
    and `rows` (all by default); checks operands and o."""
    import torch
    n = q_h.shape[0]
    n_seqs = len(cu) - 1
    ms = max(max(b - a for a, b in zip(cu, cu[1:])), 1)
    print(f"fp8 attn {label} N={n} H={H} segs={n_seqs} causal={causal}", flush=True)
    cu_d = dev_int(np.array(cu, np.int32), torch.int32)
    ws = jav.attn_fp8_prepare(dev(q_h, "bf16"), dev(k_h, "bf16"), dev(v_h, "bf16"), cu_d, ms, H)
    o = jav.attn_packed_fp8(ws, cu_d, ms, n, H, causal=causal)
    _sync()
    heads = list(range(H)) if heads is None else list(heads)
    cols = np.concatenate([np.arange(h * 128, (h + 1) * 128) for h in heads])
    r = oracle.attention_fp8(q_h[:, cols], k_h[:, cols], v_h[:, cols], cu, len(heads), 128,
                             causal=causal, rows=rows)
    if check_ops:
        views = _views(jav, ws, n, n_seqs, H)
        qrows = np.arange(n) if rows is None else np.asarray(rows)
        qr = torch.from_numpy(qrows).cuda()
        ct = torch.from_numpy(cols).cuda()
        np.testing.assert_array_equal(views["q8"][qr][:, ct].cpu().numpy(), r["q_codes"][qrows])
        np.testing.assert_array_equal(views["k8"][:, ct].cpu().numpy(), r["k_codes"])
        sq = views["sq"].cpu().numpy()[heads][:, qrows].T
        np.testing.assert_array_equal(sq, r["q_scales"][qrows])
        np.testing.assert_array_equal(views["sk"].cpu().numpy()[:, heads], r["k_scales"])
        np.testing.assert_array_equal(views["sv"].cpu().numpy()[:, heads], r["v_scales"])
        vt = views["vt"].cpu().numpy()
        for i, h in enumerate(heads):
            for s in range(n_seqs):
                a, b = cu[s], cu[s + 1]
                if b == a:
                    continue
                c0 = _col0(cu, s)
                blk = vt[h * 128:(h + 1) * 128, c0:c0 + (b - a + 63) // 64 * 64]
                np.testing.assert_array_equal(blk[:, :b - a], r["v_codes"][a:b, i * 128:(i + 1) * 128].T)
                assert not blk[:, b - a:].any(), (label, h, s, "padding codes not zero")
    _, _, vd = oracle.dequantize_attention_operands(r, len(heads), 128)
    got = host(o)[:, cols] if rows is None else host(o[torch.from_numpy(np.asarray(rows)).cuda()])[:, cols]
    _check_o(got, r, float(np.max(np.abs(vd))), ms, f"fp8 attn[{label}]")
    return ws, o


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attention_ragged_segments(jav, causal):
    """Segments of 1, 63, 64, 65, 127, 128, 129 and 300 tokens plus an empty one."""
    cu = _cu([1, 63, 64, 65, 0, 127, 128, 129, 300])
    n, H = cu[-1], 3
    q = synth.normal_array((n, H * 128), seed=610 + causal, dtype="bf16")
    k = synth.normal_array((n, H * 128), seed=612 + causal, dtype="bf16")
    v = synth.normal_array((n, H * 128), seed=614 + causal, dtype="bf16")
    _run(jav, q, k, v, cu, H, causal, label=f"ragged c={causal}")


def test_fp8_attention_several_tiles_and_peaky_scores(jav):
    """700 tokens (three query blocks, eleven key tiles, a ragged tail) with
    scores of spread 4 (q and k of std 2, per-head scales far from 1) and a
    shifted v, causal and not."""
    n, H = 700, 2
    q = synth.normal_array((n, H * 128), seed=620, std=2.0, dtype="bf16")
    k = synth.normal_array((n, H * 128), seed=621, std=2.0, dtype="bf16")
    v = synth.round_to_bf16(synth.normal_array((n, H * 128), seed=622) * 0.05 + 0.3)
    _run(jav, q, k, v, [0, n], H, False, label="peaky")
    _run(jav, q, k, v, [0, 333, n], H, True, label="peaky causal")


def test_fp8_attention_workspace_reuse_rescales(jav):
    """A second prepare into the same workspace with 1000x smaller k and v
    recomputes the per-(segment, head) scales from zero (no stale maximum)."""
    import torch
    n, H = 200, 2
    cu = [0, 77, 200]
    q = synth.normal_array((n, H * 128), seed=630, dtype="bf16")
    big = synth.normal_array((n, H * 128), seed=631, dtype="bf16")
    small = synth.round_to_bf16(big * 1e-3)
    cu_d = dev_int(np.array(cu, np.int32), torch.int32)
    ws = jav.attn_fp8_prepare(dev(q, "bf16"), dev(big, "bf16"), dev(big, "bf16"), cu_d, 123, H)
    jav.attn_fp8_prepare(dev(q, "bf16"), dev(small, "bf16"), dev(small, "bf16"), cu_d, 123, H,
                         workspace=ws)
    o = jav.attn_packed_fp8(ws, cu_d, 123, n, H)
    _sync()
    r = oracle.attention_fp8(q, small, small, cu, H, 128)
    views = _views(jav, ws, n, len(cu) - 1, H)
    np.testing.assert_array_equal(views["sv"].cpu().numpy(), r["v_scales"])
    _, _, vd = oracle.dequantize_attention_operands(r, H, 128)
    _check_o(host(o), r, float(np.max(np.abs(vd))), 123, "fp8 attn[reuse]")


@pytest.mark.parametrize("variant", ["full", "varlen", "varlen_causal"])
def test_fp8_attention_full_shape(jav, variant):
    """58,758 tokens, 40 heads: the operands and o of heads 0, 17 and 39 on
    sampled rows (heads are independent: q's scales are per row and head, k's
    and v's per segment and head)."""
    wl = synth.WORKLOADS["varlen" if variant.startswith("varlen") else "full"]
    n, H = wl.n_tokens, wl.n_heads
    cu = list(wl.expected_cu_seqlens) if variant.startswith("varlen") else [0, n]
    q = synth.normal_array((n, H * 128), seed=640, dtype="bf16")
    k = synth.normal_array((n, H * 128), seed=641, dtype="bf16")
    v = synth.normal_array((n, H * 128), seed=642, dtype="bf16")
    rows = sample_rows(cu, n, extra_every=1499, edge=3, limit=96)
    _run(jav, q, k, v, cu, H, variant == "varlen_causal", rows=rows, heads=(0, 17, 39),
         label=variant)


def test_fp8_attention_poisoned_workspace_and_tail(jav):
    """Operands prepared into a workspace filled with 0xFF bytes (NaN codes,
    NaN floats) give bit for bit the output of a zero-filled workspace: no
    byte the preparation does not write (gaps between segments' v columns,
    padding) is read.  Output rows at and past n_tokens keep their NaN, rows
    before them are finite."""
    import torch
    cu = _cu([5, 70, 1, 130])
    n, H = cu[-1], 2
    q = synth.normal_array((n, H * 128), seed=650, dtype="bf16")
    k = synth.normal_array((n, H * 128), seed=651, dtype="bf16")
    v = synth.normal_array((n, H * 128), seed=652, dtype="bf16")
    cu_d = dev_int(np.array(cu, np.int32), torch.int32)
    need = jav.attn_fp8_workspace_bytes(n, len(cu) - 1, H)
    outs = []
    for fill in (0x00, 0xFF):
        print(f"fp8 attn poison fill=0x{fill:02X} N={n}", flush=True)
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        jav.attn_fp8_prepare(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), cu_d, 130, H,
                             workspace=ws)
        o = torch.full((n + 40, H * 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        jav.attn_packed_fp8(ws, cu_d, 130, n, H, out=o)
        _sync()
        outs.append(o)
    assert torch.isfinite(outs[1][:n].float()).all()
    assert torch.isnan(outs[1][n:].float()).all()
    assert torch.equal(outs[0][:n].view(torch.int16), outs[1][:n].view(torch.int16))


def test_fp8_attention_validate_env_rejects_broken_cu_seqlens(jav):
    """DIT_VALIDATE=1: attn_fp8_prepare and attn_packed_fp8 return DIT_EINVAL for
    a broken cu_seqlens before any launch; a valid one passes.  (Memory-safe
    even unchecked: 512-row inputs and output, a workspace sized for 400
    tokens, every segment inside it.)"""
    import os
    import torch
    n, H = 512, 2
    q = torch.zeros((n, H * 128), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    cases = [([0, 300, 200, 400], 300, "decreases"), ([0, 200, 480], 280, "ends at"),
             ([0, 100, 400], 200, "max_seqlen"), ([5, 400], 395, "not 0")]
    old = os.environ.get("DIT_VALIDATE")
    os.environ["DIT_VALIDATE"] = "1"
    try:
        for cu, ms, msg in cases:
            cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
            ws = torch.zeros(jav.attn_fp8_workspace_bytes(400, len(cu) - 1, H),
                             dtype=torch.uint8, device="cuda")
            with pytest.raises(jav.DitError) as ei:
                jav.attn_fp8_prepare(q, q, q, cu_d, ms, H, workspace=ws, n_tokens=400)
            assert ei.value.status == jav.DIT_EINVAL and msg in str(ei.value), (cu, str(ei.value))
            with pytest.raises(jav.DitError) as ei:
                jav.attn_packed_fp8(ws, cu_d, ms, 400, H, out=o)
            assert ei.value.status == jav.DIT_EINVAL and msg in str(ei.value), (cu, str(ei.value))
        cu_d = torch.tensor([0, 150, 400], dtype=torch.int32, device="cuda")
        ws = jav.attn_fp8_prepare(q, q, q, cu_d, 250, H, n_tokens=400)
        jav.attn_packed_fp8(ws, cu_d, 250, 400, H, out=o)
        torch.cuda.synchronize()
        assert torch.isfinite(o[:400].float()).all()
    finally:
        if old is None:
            os.environ.pop("DIT_VALIDATE", None)
        else:
            os.environ["DIT_VALIDATE"] = old


def test_fp8_attention_segment_longer_than_max_seqlen_becomes_nan(jav):
    """cu_seqlens breaking its contract (a 400-row segment against max_seqlen 300,
    inside the buffers): the operand preparation and the attention do not cover that
    segment, and its output rows come out NaN; the other segment is bit-identical to
    a call with the right max_seqlen."""
    import torch
    n, H = 700, 2
    q, k, v = (dev(synth.normal_array((n, H * 128), seed=270 + i, dtype="bf16"), "bf16")
               for i in range(3))
    cu_d = dev_int(np.array([0, 300, 700], np.int32), torch.int32)
    ws = jav.attn_fp8_prepare(q, k, v, cu_d, 400, H)
    good = jav.attn_packed_fp8(ws, cu_d, 400, n, H)
    ws_bad = jav.attn_fp8_prepare(q, k, v, cu_d, 300, H)
    bad = jav.attn_packed_fp8(ws_bad, cu_d, 300, n, H)
    _sync()
    assert torch.equal(bad[:300].view(torch.int16), good[:300].view(torch.int16))
    assert torch.isnan(bad[300:].float()).all()
