"""Helpers for the GPU parity tests: device copies of seeded inputs and the
tolerance checks (bf16: max-abs <= 3e-2 and rel-L2 <= 1e-2; f32: rel-L2 <= 1e-5)."""
import numpy as np

BF16_MAX_ABS = 3e-2
BF16_REL_L2 = 1e-2
F32_REL_L2 = 1e-5


def torch_mod():
    import torch
    return torch


def dev(a, dtype: str):
    """float32 host array (bf16-exact for bf16) -> device tensor of the workload dtype."""
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def dev_f32(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_int(a, dtype):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def check(got, ref, dtype: str, what: str = ""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref))) if got.size else 0.0
    print(f"  {what}: rel_l2={r:.3e} max_abs={m:.3e}", flush=True)
    if dtype == "bf16":
        assert m <= BF16_MAX_ABS and r <= BF16_REL_L2, (what, r, m)
    else:
        assert r <= F32_REL_L2, (what, r, m)
    return r, m


def sample_rows(cu, n, extra_every=97, edge=8, seed=0, limit=None):
    """First/last `edge` rows of every segment, every extra_every-th row, the last row."""
    rows = set()
    for a, b in zip(cu, cu[1:]):
        rows.update(range(a, min(b, a + edge)))
        rows.update(range(max(a, b - edge), b))
    rows.update(range(0, n, extra_every))
    rows.add(n - 1)
    rows = sorted(r for r in rows if 0 <= r < n)
    if limit is not None and len(rows) > limit:
        rng = np.random.Generator(np.random.PCG64(seed))
        keep = set(rows[:edge]) | set(rows[-edge:])
        rest = [r for r in rows if r not in keep]
        keep |= set(rng.choice(rest, size=limit - len(keep), replace=False).tolist())
        rows = sorted(keep)
    return np.array(rows, dtype=np.int64)


def ci_sample_rows(layout, every=97, edge=64):
    """The CI row sample of a packed layout: the first and last `edge` rows of
    every segment, every text row, the first and last audio frame of both
    channels of every request (k = 0 and k = n_a - 1), every `every`-th row,
    and two rows on each side of every change of modality.  About 800 rows of
    the full 58,758-token pack."""
    mod = np.asarray(layout["modality"])
    pos = np.asarray(layout["pos"])
    cu = [int(c) for c in layout["cu_seqlens"]]
    n = int(mod.size)
    rows = set(range(0, n, every))
    for a, b in zip(cu, cu[1:]):
        if b <= a:
            continue
        rows.update(range(a, min(b, a + edge)))
        rows.update(range(max(a, b - edge), b))
        seg_mod = mod[a:b]
        rows.update((a + np.nonzero(seg_mod == 2)[0]).tolist())
        aud = a + np.nonzero(seg_mod == 1)[0]
        if aud.size:
            t = pos[aud, 0]
            last = int(t.max())
            rows.update(aud[(t == 0) | (t == last)].tolist())
    # two rows on each side of every change of modality (video/audio, audio/text)
    for i in (np.nonzero(mod[1:] != mod[:-1])[0] + 1).tolist():
        rows.update(r for r in range(i - 2, i + 2) if 0 <= r < n)
    return np.array(sorted(rows), dtype=np.int64)
