"""Writes block_backward_medium.npz: the float64 oracle's gradients of the
attention half at the medium workload (16,384 tokens, d_model 3072, 24 heads x
128, bidirectional, no biases), for the GPU test of dit_block_backward at that
shape.  Calls only oracle/ and synth/ (the oracle takes about ten minutes here,
too long to run inside the GPU suite).

The inputs are synth.block_inputs(medium) and dout = synth.normal_array((N, D),
seed=1500 + N, dtype="bf16"), the recipe of the GPU test.  Stored per gradient:
  * db_qkv, db_o, dtable: the whole gradient (float32);
  * dx, dw_qkv, dw_o: the values at 16,384 sampled element positions (seeded),
    every row's L2 norm, the Frobenius norm, and a two-sided Gaussian sketch
    A G B (A [32][rows], B [cols][32], standard normal, seeded), whose relative
    L2 distance to the GPU gradient's sketch estimates the whole tensor's.

Run from the repository root: python tests/golden/make_block_backward_medium.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_backward_medium.npz")
SAMPLES = 16384
SKETCH = 32


def sketch_mats(rows, cols, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((SKETCH, rows)), rng.standard_normal((cols, SKETCH))


def sample_positions(size, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(size, size=SAMPLES, replace=False)).astype(np.int64)


BIG = {"dx": 11, "dw_qkv": 12, "dw_o": 13}   # gradient -> seed of its sample and sketch


def main():
    wl = synth.WORKLOADS["medium"]
    inp = synth.block_inputs(wl)
    lay = oracle.pack_layout([r.grid for r in wl.requests])
    n, d = wl.n_tokens, wl.d_model
    dout = synth.normal_array((n, d), seed=1500 + n, dtype="bf16")
    ref = oracle.block_backward(inp.x, lay["modality"], lay["pos"], lay["cu_seqlens"], inp.table,
                                inp.w_qkv, inp.w_o, dout, n_heads=wl.n_heads,
                                head_dim=wl.head_dim, sections=wl.sections, theta=wl.theta,
                                eps=wl.eps)
    out = {}
    for key in ("db_qkv", "db_o", "dtable"):
        out[key] = ref[key].astype(np.float32)
    for key, seed in BIG.items():
        g = np.asarray(ref[key], np.float64)
        pos = sample_positions(g.size, seed)
        a, b = sketch_mats(g.shape[0], g.shape[1], seed)
        out[f"{key}_pos"] = pos
        out[f"{key}_val"] = g.reshape(-1)[pos].astype(np.float32)
        out[f"{key}_rownorm"] = np.linalg.norm(g, axis=1)
        out[f"{key}_norm"] = np.array(np.linalg.norm(g))
        out[f"{key}_maxabs"] = np.array(np.abs(g).max())
        out[f"{key}_sketch"] = a @ g @ b
    np.savez_compressed(OUT, **out)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
