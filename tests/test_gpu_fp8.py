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
from gpu_util import check, dev, dev_f32, dev_int, host, sample_rows

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
