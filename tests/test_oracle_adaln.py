"""Pins of the oracle's per-modality AdaLN (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import brute
import synth


def _case(n=37, d=48, seed=11):
    x = synth.normal_array((n, d), seed, 1.0).astype(np.float64) * 3.0 + 0.7
    table = synth.normal_array((3, 3, d), seed + 1, 0.3).astype(np.float64)
    mod = synth.uniform_ints((n,), 0, 3, seed + 2)
    return x, table, mod


def test_matches_torch_layer_norm_with_affine():
    """Each row equals torch layer_norm with weight 1 + scale[m] and bias shift[m]."""
    x, table, mod = _case()
    y = oracle.adaln_modulate(x, mod, table, eps=1e-6)
    xt = torch.from_numpy(x)
    for i in range(x.shape[0]):
        m = int(mod[i])
        ref = F.layer_norm(xt[i:i + 1], (x.shape[1],),
                           weight=torch.from_numpy(1.0 + table[m, 1]),
                           bias=torch.from_numpy(table[m, 0]), eps=1e-6)
        np.testing.assert_allclose(y[i], ref.numpy()[0], rtol=0, atol=1e-12)


def test_zero_table_is_plain_layer_norm():
    x, table, mod = _case(seed=3)
    y = oracle.adaln_modulate(x, mod, np.zeros_like(table), eps=1e-6)
    ref = F.layer_norm(torch.from_numpy(x), (x.shape[1],), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


def test_token_permutation_equivariance():
    x, table, mod = _case(seed=5)
    perm = np.random.Generator(np.random.PCG64(9)).permutation(x.shape[0])
    y = oracle.adaln_modulate(x, mod, table)
    yp = oracle.adaln_modulate(x[perm], mod[perm], table)
    np.testing.assert_array_equal(yp, y[perm])


def test_modality_relabel_equals_table_row_swap():
    x, table, mod = _case(seed=6)
    y = oracle.adaln_modulate(x, mod, table)
    swap = np.array([2, 1, 0])
    y2 = oracle.adaln_modulate(x, swap[mod], table[swap])
    np.testing.assert_array_equal(y, y2)


def test_rows_subset_matches_full():
    x, table, mod = _case(seed=8)
    rows = [0, 5, 36, 17]
    np.testing.assert_allclose(oracle.adaln_modulate(x, mod, table, rows=rows),
                                  oracle.adaln_modulate(x, mod, table)[rows])


def test_brute_force_agreement():
    x, table, mod = _case(n=9, d=16, seed=12)
    y = oracle.adaln_modulate(x, mod, table)
    yb = brute.adaln(x.tolist(), mod.tolist(), table.tolist())
    np.testing.assert_allclose(y, np.array(yb), rtol=0, atol=1e-12)
