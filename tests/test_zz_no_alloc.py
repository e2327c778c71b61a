"""attn_packed_backward_noalloc (MI355X only): the attention backward with its
scratch in the library's fixed device array gives bit for bit the gradients of
attn_packed_backward with a caller workspace (the same kernels, deterministic),
on two calls in a row, the second smaller than the first, so the second reuses
the array the first left behind; and sizes past the array's capacity are
rejected before anything is enqueued."""
import numpy as np
import pytest

import synth
from gpu_util import dev, dev_int

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jav():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import joint_audio_video_amd as m
    return m


def _case(jav, n, H, cu, causal, seed):
    import torch
    print(f"noalloc backward n={n} H={H} segments={len(cu) - 1} causal={causal}", flush=True)
    arrs = [dev(synth.normal_array((n, H * 128), seed + i, dtype="bf16"), "bf16") for i in range(4)]
    q, k, v, dout = arrs
    cu_d = dev_int(np.array(cu, np.int32), torch.int32)
    ms = max(b - a for a, b in zip(cu, cu[1:]))
    o, lse = jav.attn_packed_lse(q, k, v, cu_d, ms, H, 128, causal=causal)
    ref = jav.attn_packed_backward(q, k, v, o, dout, lse, cu_d, ms, H, 128, causal=causal)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    jav.attn_packed_backward_noalloc(q, k, v, o, dout, lse, cu_d, ms, H, 128, causal=causal,
                                     dq=got[0], dk=got[1], dv=got[2])
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(a.float()).all(), name
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


def test_noalloc_backward_matches_workspace_entry_point(jav):
    wl = synth.WORKLOADS["full"]
    assert wl.n_heads * wl.n_tokens <= jav.attn_backward_noalloc_max_elements()
    # the full pack, then a smaller ragged causal one reusing the same array
    _case(jav, wl.n_tokens, wl.n_heads, [0, wl.n_tokens], False, 700)
    _case(jav, 1000, 4, [0, 1, 64, 128, 129, 259, 559, 560, 1000], True, 710)


def test_noalloc_backward_rejects_past_capacity(jav):
    import torch
    cap = jav.attn_backward_noalloc_max_elements()
    H = 64
    n = cap // H + 1
    q = torch.zeros((1, H * 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((H, 1), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    with pytest.raises(jav.DitError) as e:
        jav.attn_packed_backward_noalloc(q, q, q, q, q, lse, cu, n, H, 128, dq=q, dk=q, dv=q,
                                         n_tokens=n)
    assert e.value.status == jav.DIT_EWORKSPACE and "fixed scratch" in str(e.value)
