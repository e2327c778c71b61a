"""Parity of the feed-forward half's entry points against the float64 oracle (MI355X only).

ffn_up_gelu, ffn_down_gated and dit_ffn_forward on the workloads' shapes
(d_ff = 4 d_model), with an odd k-step count and ragged tiles, and at the
full 58,758-token shape on sampled rows (first and last rows of every
segment, the ragged tail, every 97th row).  The down projection is checked on
its own up to the medium shape; at the full shape it runs inside
dit_ffn_forward, whose oracle rebuilds h itself from x.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import check, dev, dev_f32, dev_int, host, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jav():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import joint_audio_video_amd as m
    return m


@functools.lru_cache(maxsize=2)
def _ffn(name, bias):
    return synth.ffn_inputs(synth.WORKLOADS[name], with_bias=bias)


@functools.lru_cache(maxsize=4)
def _layout(name):
    wl = synth.WORKLOADS[name]
    return oracle.pack_layout([r.grid for r in wl.requests])


def _x(name):
    wl = synth.WORKLOADS[name]
    return synth.normal_array((wl.n_tokens, wl.d_model), seed=500 + wl.seed, dtype=wl.dtype)


def _rows(name):
    wl = synth.WORKLOADS[name]
    if wl.n_tokens <= 4096:
        return None
    return sample_rows(_layout(name)["cu_seqlens"], wl.n_tokens, limit=600)


def _sync():
    import torch
    torch.cuda.synchronize()


def _take(t, rows):
    import torch
    return host(t) if rows is None else host(t[torch.from_numpy(rows).cuda()])


@pytest.mark.parametrize("name,bias", [("tiny", True), ("small", False), ("small", True),
                                       ("full", False)])
def test_ffn_up_gelu_parity(jav, name, bias):
    wl = synth.WORKLOADS[name]
    f = _ffn(name, bias)
    print(f"ffn_up {name} bias={bias} d_ff={wl.d_ff}", flush=True)
    y_h = synth.normal_array((wl.n_tokens, wl.d_model), seed=510 + wl.seed, dtype=wl.dtype)
    h = jav.ffn_up_gelu(dev(y_h, wl.dtype), dev(f.w1, wl.dtype),
                        dev(f.b1, wl.dtype) if bias else None)
    _sync()
    rows = _rows(name)
    ref = oracle.ffn_up(y_h if rows is None else y_h[rows], f.w1, f.b1 if bias else None)
    check(_take(h, rows), ref, wl.dtype, f"ffn_up[{name}]")


@pytest.mark.parametrize("name,bias,inplace", [("tiny", True, False), ("small", False, True),
                                               ("medium", True, True)])
def test_ffn_down_gated_parity(jav, name, bias, inplace):
    import torch
    wl = synth.WORKLOADS[name]
    f = _ffn(name, bias)
    lay = _layout(name)
    print(f"ffn_down {name} bias={bias} inplace={inplace}", flush=True)
    # h values in GELU's output range (mostly >= -0.17), as the up projection leaves them
    h_h = synth.normal_array((wl.n_tokens, wl.d_ff), seed=520 + wl.seed, dtype=wl.dtype)
    h_h = np.asarray(oracle.gelu_tanh(h_h), np.float32)
    h_h = synth.round_to_bf16(h_h) if wl.dtype == "bf16" else h_h
    x_h = _x(name)
    x = dev(x_h, wl.dtype)
    mod = dev_int(lay["modality"], torch.uint8)
    out = jav.ffn_down_gated(dev(h_h, wl.dtype), dev(f.w2, wl.dtype), x, mod, dev_f32(f.table),
                             dev(f.b2, wl.dtype) if bias else None, out=x if inplace else None)
    _sync()
    rows = _rows(name)
    ref = oracle.out_proj_gated(h_h if rows is None else h_h[rows], f.w2, x_h, lay["modality"],
                                f.table, f.b2 if bias else None, rows=rows)
    check(_take(out, rows), ref, wl.dtype, f"ffn_down[{name}]")


@pytest.mark.parametrize("name", ["tiny", "small", "full"])
def test_ffn_forward_parity(jav, name):
    import torch
    wl = synth.WORKLOADS[name]
    f = _ffn(name, False)
    lay = _layout(name)
    print(f"ffn_forward {name}", flush=True)
    x_h = _x(name)
    desc = jav.ffn_desc(jav.DIT_BF16 if wl.dtype == "bf16" else jav.DIT_F32, wl.d_model, wl.d_ff,
                        wl.eps)
    out = jav.ffn_forward(desc, dev(x_h, wl.dtype), dev_int(lay["modality"], torch.uint8),
                          dev_f32(f.table), dev(f.w1, wl.dtype), dev(f.w2, wl.dtype))
    _sync()
    rows = _rows(name)
    ref = oracle.ffn_forward(x_h, lay["modality"], f.table, f.w1, f.w2, eps=wl.eps, rows=rows)
    got = _take(out, rows)
    check(got, ref, wl.dtype, f"ffn[{name}]")
    # the branch alone (out - x), where the residual does not hide errors
    xr = np.asarray(x_h if rows is None else x_h[rows], np.float64)
    branch_ref = ref - xr
    scale = max(float(np.abs(branch_ref).max()), 1e-30)
    assert float(np.abs((got - xr) - branch_ref).max()) <= (1e-5 if wl.dtype == "f32" else 0.1) * scale


def test_ffn_forward_odd_shapes_bias_and_trim(jav):
    """d_model 1600 (25 k-steps up), d_ff 6400 (100 down), 777 tokens inside a
    larger buffer: rows past n_tokens stay untouched; biases on; modalities per row."""
    import torch
    d, f_, n, alloc = 1600, 6400, 777, 800
    x_h = synth.normal_array((alloc, d), seed=530, dtype="bf16")
    table = synth.normal_array((3, 3, d), seed=531, std=0.1)
    w1 = synth.normal_array((f_, d), seed=532, std=0.02, dtype="bf16")
    w2 = synth.normal_array((d, f_), seed=533, std=0.02, dtype="bf16")
    b1 = synth.normal_array((f_,), seed=534, std=0.02, dtype="bf16")
    b2 = synth.normal_array((d,), seed=535, std=0.02, dtype="bf16")
    mod = synth.uniform_ints((alloc,), 0, 3, seed=536).astype(np.uint8)
    x = dev(x_h, "bf16")
    out = torch.full_like(x, float("nan"))
    desc = jav.ffn_desc(jav.DIT_BF16, d, f_)
    jav.ffn_forward(desc, x, dev_int(mod, torch.uint8), dev_f32(table), dev(w1, "bf16"),
                    dev(w2, "bf16"), dev(b1, "bf16"), dev(b2, "bf16"), out=out, n_tokens=n)
    _sync()
    ref = oracle.ffn_forward(x_h[:n], mod[:n], table, w1, w2, b1, b2)
    check(host(out[:n]), ref, "bf16", "ffn odd shapes")
    assert torch.isnan(out[n:]).all()
