"""The C ABI on the CPU: symbols, host layout bit-exact against the oracle, and
argument validation that returns before anything is enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest

import joint_audio_video_amd as jav
import oracle
import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dit.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_exported_set():
    assert _declared_functions() == sorted(jav.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(jav.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert jav.abi_version() == 1


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_grid_from_media_matches_oracle(name):
    for r in synth.WORKLOADS[name].requests:
        assert jav.grid_from_media(*r.media) == oracle.grid_from_media(*r.media)


@pytest.mark.parametrize("media", [
    (121, 288, 448, 32000, 7), (1, 32, 32, 0, 0), (0, 0, 0, 1600, 3), (5, 0, 64, 0, 1),
    (0, 256, 256, 800, 0)])
def test_grid_from_media_edge_cases(media):
    assert jav.grid_from_media(*media) == oracle.grid_from_media(*media)


@pytest.mark.parametrize("bad", [(120, 256, 256, 0, 0), (5, 400, 640, 0, 0), (5, 256, 256, 801, 0),
                                 (-1, 256, 256, 0, 0), (5, 256, 256, 0, -1)])
def test_grid_from_media_rejects(bad):
    with pytest.raises(ValueError):
        oracle.grid_from_media(*bad)
    with pytest.raises(jav.DitError) as e:
        jav.grid_from_media(*bad)
    assert e.value.status == jav.DIT_EINVAL


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_pack_layout_bit_exact(name):
    grids = [r.grid for r in synth.WORKLOADS[name].requests]
    ref = oracle.pack_layout(grids)
    got = jav.pack_layout(grids)
    assert got["n_tokens"] == ref["n_tokens"]
    assert got["max_seqlen"] == ref["max_seqlen"]
    np.testing.assert_array_equal(got["cu_seqlens"], np.array(ref["cu_seqlens"], np.int32))
    np.testing.assert_array_equal(got["modality"], np.array(ref["modality"], np.uint8))
    np.testing.assert_array_equal(got["pos"], np.array(ref["pos"], np.int32).reshape(-1, 3))


def test_pack_layout_golden_and_page_example():
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pack_tiny.json")))
    got = jav.pack_layout(g["grids"])
    assert got["modality"].tolist() == g["modality"]
    assert got["pos"].tolist() == g["pos"]
    assert got["cu_seqlens"].tolist() == g["cu_seqlens"]
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cu_seqlens_example.json")))
    got = jav.pack_layout([(0, 0, 0, 0, n) for n in ex["lengths_three"]])
    assert got["cu_seqlens"].tolist() == ex["cu_three"]


def test_pack_layout_errors():
    with pytest.raises(jav.DitError) as e:
        jav.pack_layout([(2, 2, 2, 1, 1)], capacity=5)
    assert e.value.status == jav.DIT_EINVAL
    with pytest.raises(jav.DitError):
        jav.pack_layout([(1, 1, -1, 0, 0)])
    with pytest.raises(jav.DitError):
        jav.pack_layout([])


def _call(fn, *args):
    return getattr(jav._lib, fn)(*args)


def test_device_entry_points_validate_before_enqueue():
    """Bad host scalars are rejected with exact codes; nothing touches a device."""
    fake = 1 << 20            # never dereferenced: validation fails first
    sec = (ctypes.c_int32 * 3)(32, 48, 48)
    bad_sec = (ctypes.c_int32 * 3)(31, 49, 48)
    # adaln
    assert _call("adaln_modulate", 7, fake, 64, fake, fake, fake, 64, 10, 64, 1e-6, None) == jav.DIT_EINVAL
    assert _call("adaln_modulate", jav.DIT_BF16, None, 64, fake, fake, fake, 64, 10, 64, 1e-6, None) == jav.DIT_EINVAL
    assert _call("adaln_modulate", jav.DIT_BF16, fake, 32, fake, fake, fake, 64, 10, 64, 1e-6, None) == jav.DIT_EINVAL
    assert _call("adaln_modulate", jav.DIT_BF16, fake, 64, fake, fake, fake, 64, 10, 64, 0.0, None) == jav.DIT_EINVAL
    assert _call("adaln_modulate", jav.DIT_BF16, fake + 2, 64, fake, fake, fake, 64, 10, 64, 1e-6, None) == jav.DIT_EUNSUPPORTED
    assert _call("adaln_modulate", jav.DIT_BF16, fake, 68, fake, fake, fake, 68, 10, 68, 1e-6, None) == jav.DIT_EUNSUPPORTED
    assert "adaln_modulate" in jav.last_error()
    # rope
    assert _call("rope3d_apply", jav.DIT_BF16, fake, 384, fake, 384, fake, 10, 3, 128, bad_sec, 1e4, None) == jav.DIT_EINVAL
    assert _call("rope3d_apply", jav.DIT_BF16, fake, 100, fake, 384, fake, 10, 3, 128, sec, 1e4, None) == jav.DIT_EINVAL
    assert _call("rope3d_apply", jav.DIT_BF16, fake, 384, fake, 384, fake, 10, 3, 128, sec, 0.0, None) == jav.DIT_EINVAL
    sec96 = (ctypes.c_int32 * 3)(32, 32, 32)
    assert _call("rope3d_apply", jav.DIT_BF16, fake, 384, fake, 384, fake, 10, 4, 96, sec96, 1e4, None) == jav.DIT_EUNSUPPORTED
    # attention
    A = [jav.DIT_BF16, fake, 5120, fake, 5120, fake, 5120, fake, 5120]
    assert _call("attn_packed", *A, fake, 0, 10, 10, 40, 128, 0.0, 0, None) == jav.DIT_EINVAL     # n_seqs
    assert _call("attn_packed", *A, fake, 1, 0, 10, 40, 128, 0.0, 0, None) == jav.DIT_EINVAL      # max_seqlen
    assert _call("attn_packed", *A, fake, 1, 10, 10, 40, 128, -1.0, 0, None) == jav.DIT_EINVAL    # scale
    assert _call("attn_packed", *A, fake, 1, 10, 10, 80, 64, 0.0, 0, None) == jav.DIT_EUNSUPPORTED  # bf16 dh 64
    assert _call("attn_packed", *A, None, 1, 10, 10, 40, 128, 0.0, 0, None) == jav.DIT_EINVAL
    # n_tokens == 0 is a no-op even with a null stream
    assert _call("attn_packed", *A, fake, 1, 0, 0, 40, 128, 0.0, 0, None) == jav.DIT_OK
    # projections
    assert _call("qkv_project", jav.DIT_BF16, fake, 4096, fake, None, fake, 15360, 10, 5120, None) == jav.DIT_EINVAL
    assert _call("qkv_project", jav.DIT_BF16, fake, 5120, fake, None, fake, 15360, 10, 5064, None) == jav.DIT_EUNSUPPORTED
    assert _call("out_proj_gated", jav.DIT_BF16, fake, 5120, fake, None, None, 5120, fake, fake, fake, 5120, 10, 5120, None) == jav.DIT_EINVAL


def test_block_workspace_and_descriptor_checks():
    desc = jav.block_desc(jav.DIT_BF16, 5120, 40, 128, (32, 48, 48))
    n = 58758
    planes = 5 * (((n * 5120 * 2 + 255) // 256) * 256)    # y, q', k', v, o planes
    assert jav.block_workspace_bytes(desc, n) == planes
    fake = 1 << 20
    args = [fake, fake, fake, fake, fake, 1, 100, 100, fake, fake, None, fake, None]
    # workspace too small
    st = jav._lib.dit_block_forward(ctypes.byref(desc), *args, fake, 10, None)
    assert st == jav.DIT_EWORKSPACE
    bad = jav.block_desc(jav.DIT_BF16, 5120, 40, 64, (16, 24, 24))   # D != H * Dh
    st = jav._lib.dit_block_forward(ctypes.byref(bad), *args, fake, 1 << 40, None)
    assert st == jav.DIT_EINVAL
    assert jav.block_workspace_bytes(jav.block_desc(9, 64, 1, 64, (16, 24, 24)), 10) == 0


def test_ffn_entry_points_validate_before_enqueue():
    fake = 1 << 20            # never dereferenced: validation fails first
    B = jav.DIT_BF16
    # ffn_up_gelu(dt, y, ld_y, w1, b1, h, ld_h, n, d_model, d_ff, stream)
    assert _call("ffn_up_gelu", B, None, 5120, fake, None, fake, 20480, 10, 5120, 20480, None) == jav.DIT_EINVAL
    assert _call("ffn_up_gelu", B, fake, 5120, fake, None, fake, 20000, 10, 5120, 20480, None) == jav.DIT_EINVAL   # ld_h
    assert _call("ffn_up_gelu", B, fake, 5120, fake, None, fake, 20480, 10, 5120, 0, None) == jav.DIT_EINVAL       # d_ff
    assert _call("ffn_up_gelu", B, fake, 5120, fake, None, fake, 20480, 10, 5120, 20420, None) == jav.DIT_EUNSUPPORTED  # d_ff % 64
    assert _call("ffn_up_gelu", B, fake, 5120, fake, fake + 8, fake, 20480, 10, 5120, 20480, None) == jav.DIT_EUNSUPPORTED  # b1 align
    assert _call("ffn_up_gelu", B, fake, 5120, fake, None, fake, 20480, 0, 5120, 20480, None) == jav.DIT_OK      # no rows
    # ffn_down_gated(dt, h, ld_h, w2, b2, x, ld_x, mod, table, out, ld_out, n, d_model, d_ff, stream)
    D = [B, fake, 20480, fake, None]
    assert _call("ffn_down_gated", *D, None, 5120, fake, fake, fake, 5120, 10, 5120, 20480, None) == jav.DIT_EINVAL   # x
    assert _call("ffn_down_gated", *D, fake, 5120, fake, fake, fake, 5120, 10, 5064, 20480, None) == jav.DIT_EUNSUPPORTED  # d_model % 64
    assert _call("ffn_down_gated", *D, fake, 5120, fake, fake, fake, 5184, 10, 5120, 20480, None) == jav.DIT_EINVAL   # in place, ld differs
    assert _call("ffn_down_gated", *D, fake, 5120, fake, fake, fake + 16, 5120, 0, 5120, 20480, None) == jav.DIT_OK


def test_ffn_workspace_and_descriptor_checks():
    desc = jav.ffn_desc(jav.DIT_BF16, 5120, 20480)
    n = 58758
    want = sum(((n * w * 2 + 255) // 256) * 256 for w in (5120, 20480))
    assert jav.ffn_workspace_bytes(desc, n) == want
    fake = 1 << 20
    # (desc, x, out, mod, n, table, w1, b1, w2, b2, ws, ws_bytes, stream)
    st = jav._lib.dit_ffn_forward(ctypes.byref(desc), fake, fake, fake, 100, fake, fake, None,
                                  fake, None, fake, 10, None)
    assert st == jav.DIT_EWORKSPACE
    st = jav._lib.dit_ffn_forward(ctypes.byref(desc), fake, fake, fake, 100, fake, fake, None,
                                  fake, None, fake + 128, 1 << 40, None)
    assert st == jav.DIT_EUNSUPPORTED           # workspace not 256-byte aligned
    bad = jav.ffn_desc(jav.DIT_BF16, 5120, 20420)
    st = jav._lib.dit_ffn_forward(ctypes.byref(bad), fake, fake, fake, 100, fake, fake, None,
                                  fake, None, fake, 1 << 40, None)
    assert st == jav.DIT_EUNSUPPORTED           # d_ff not a multiple of 64
    assert jav.ffn_workspace_bytes(jav.ffn_desc(9, 64, 256), 10) == 0


def test_denoise_step_validates_before_enqueue():
    fake = 1 << 20            # never dereferenced: validation fails first
    B, F = jav.DIT_BF16, jav.DIT_F32
    sig = (ctypes.c_float * 4)(0.8, 0.6, 0.7, 0.5)

    def call(dt=B, z=fake, ldz=96, v=fake, ldv=96, x0=fake, ldx=96, mod=fake, anchor=None,
             av=None, lda=0, n=10, c=96, sigmas=sig, sign=1):
        return _call("denoise_step", dt, z, ldz, v, ldv, x0, ldx, mod, anchor, av, lda, n, c,
                     sigmas, sign, None)

    assert call(dt=5) == jav.DIT_EINVAL
    assert call(z=None) == jav.DIT_EINVAL
    assert call(mod=None) == jav.DIT_EINVAL
    assert call(sigmas=None) == jav.DIT_EINVAL
    assert call(anchor=fake) == jav.DIT_EINVAL              # flags without values
    assert call(ldv=64) == jav.DIT_EINVAL
    assert call(anchor=fake, av=fake, lda=32) == jav.DIT_EINVAL
    assert call(n=-1) == jav.DIT_EINVAL
    assert call(c=0) == jav.DIT_EINVAL
    assert call(sign=0) == jav.DIT_EINVAL
    for bad in ((1.5, 0.6, 0.7, 0.5), (0.8, -0.1, 0.7, 0.5), (0.8, 0.6, float("nan"), 0.5)):
        assert call(sigmas=(ctypes.c_float * 4)(*bad)) == jav.DIT_EINVAL
    assert "sigma" in jav.last_error()
    assert call(c=94, ldz=96, ldv=96, ldx=96) == jav.DIT_EUNSUPPORTED     # channels % 4
    assert call(z=fake + 8) == jav.DIT_EUNSUPPORTED
    assert call(dt=F, ldv=98) == jav.DIT_EUNSUPPORTED                     # f32 rows of 392 B
    assert call(n=(1 << 31) // 24 + 1) == jav.DIT_EUNSUPPORTED
    assert call(n=0) == jav.DIT_OK                                        # no rows: no-op
    assert call(x0=None, ldx=0, n=0) == jav.DIT_OK
    assert jav.timestep_from_sigma(1.0) == 0.0 and jav.timestep_from_sigma(0.0) == 1.0


def test_nft_loss_validates_before_enqueue():
    fake = 1 << 20            # never dereferenced: validation fails first
    B = jav.DIT_BF16
    # 4 int32 row counts (16 -> 256 B) + 460 chunks of 32 rows x 4 samples x 2 floats
    # (14,720 -> 14,848 B)
    assert jav.nft_workspace_bytes(4, 14690) == 256 + 14848
    assert jav.nft_workspace_bytes(0, 10) == 0 and jav.nft_workspace_bytes(2, 0) == 0

    def call(dt=B, vt=fake, ldvt=96, vo=fake, ldvo=96, tg=fake, ldt=96, mask=None, cu=fake,
             ns=4, mr=14690, n=58758, c=96, rew=fake, beta=0.5, sign=1, scale=0.25, g=fake,
             ldg=96, out=fake, ws=fake, wsb=1 << 30):
        return _call("nft_loss", dt, vt, ldvt, vo, ldvo, tg, ldt, mask, cu, ns, mr, n, c, rew,
                     beta, sign, scale, g, ldg, out, ws, wsb, None)

    assert call(dt=3) == jav.DIT_EINVAL
    assert call(vt=None) == jav.DIT_EINVAL
    assert call(out=None) == jav.DIT_EINVAL
    assert call(rew=None) == jav.DIT_EINVAL
    assert call(ns=0) == jav.DIT_EINVAL
    assert call(mr=0) == jav.DIT_EINVAL
    assert call(c=0) == jav.DIT_EINVAL
    assert call(ldt=64) == jav.DIT_EINVAL
    assert call(beta=float("inf")) == jav.DIT_EINVAL
    assert call(scale=float("nan")) == jav.DIT_EINVAL
    assert call(sign=2) == jav.DIT_EINVAL
    assert call(c=94, ldvt=96, ldvo=96, ldt=96, ldg=96) == jav.DIT_EUNSUPPORTED
    assert call(ns=70000) == jav.DIT_EUNSUPPORTED
    assert call(vo=fake + 4) == jav.DIT_EUNSUPPORTED
    assert call(ldvt=100) == jav.DIT_EUNSUPPORTED        # bf16 rows of 200 B
    assert call(wsb=16) == jav.DIT_EWORKSPACE
    assert call(ws=None) == jav.DIT_EWORKSPACE
    assert call(ws=fake + 64) == jav.DIT_EUNSUPPORTED
    assert "nft_loss" in jav.last_error()


def test_rope3d_apply_to_overlap_rules():
    fake = 1 << 24            # never dereferenced: validation fails first
    sec = (ctypes.c_int32 * 3)(32, 48, 48)
    B, n, w = jav.DIT_BF16, 10, 5120
    row = w * 2

    def call(q, k, qo, ko, ldq=w, ldk=w, ldqo=w, ldko=w, n=n):
        return _call("rope3d_apply_to", B, q, ldq, k, ldk, qo, ldqo, ko, ldko, fake, n, 40, 128,
                     sec, 1e4, None)

    q, k = fake, fake + 64 * row
    assert call(q, k, None, fake + 128 * row) == jav.DIT_EINVAL          # missing output
    assert call(q, None, fake + 128 * row, fake + 160 * row) == jav.DIT_EINVAL   # k_out without k
    assert call(q, k, fake + 128 * row, fake + 160 * row, ldko=4000) == jav.DIT_EINVAL
    assert call(q, k, q + 4 * row, fake + 160 * row) == jav.DIT_EINVAL   # output shifted into q
    assert call(q, k, fake + 128 * row, fake + 133 * row) == jav.DIT_EINVAL   # outputs overlap
    assert call(q, k, fake + 128 * row, fake + 160 * row + 8) == jav.DIT_EUNSUPPORTED
    # allowed: separate outputs, in place, and k_out = q (the block's arrangement)
    assert call(q, k, fake + 128 * row, fake + 160 * row, n=0) == jav.DIT_OK
    assert call(q, k, q, k, n=0) == jav.DIT_OK
    assert call(q, k, fake + 128 * row, q, n=0) == jav.DIT_OK


def test_fp8_block_halves_validate_before_enqueue():
    fake = 1 << 24            # never dereferenced: validation fails first
    B, F32 = jav.DIT_BF16, jav.DIT_F32
    # adaln_modulate_fp8(dt, x, ld_x, mod, table, q, ld_q, scales, n, d, eps, stream)
    assert _call("adaln_modulate_fp8", B, fake, 5120, fake, fake, None, 5120, fake, 10, 5120, 1e-6, None) == jav.DIT_EINVAL
    assert _call("adaln_modulate_fp8", B, fake, 5120, fake, fake, fake, 5000, fake, 10, 5120, 1e-6, None) == jav.DIT_EINVAL
    assert _call("adaln_modulate_fp8", B, fake, 5120, fake, fake, fake, 5128, fake, 10, 5120, 1e-6, None) == jav.DIT_EUNSUPPORTED
    assert _call("adaln_modulate_fp8", B, fake, 5120, fake, fake, fake, 5120, fake + 4, 10, 5120, 1e-6, None) == jav.DIT_EUNSUPPORTED
    assert "adaln_modulate_fp8" in jav.last_error()
    assert _call("adaln_modulate_fp8", F32, fake, 256, fake, fake, fake, 256, fake, 0, 256, 1e-6, None) == jav.DIT_OK

    desc = jav.block_desc(B, 5120, 40, 128, (32, 48, 48))
    n = 58758
    plane = ((n * 5120 * 2 + 255) // 256) * 256
    assert jav.block_fp8_workspace_bytes(desc, n) == 5 * plane + ((n * 4 + 255) // 256) * 256
    assert jav.block_fp8_workspace_bytes(jav.block_desc(F32, 256, 4, 64, (16, 24, 24)), 10) == 0
    # (desc, x, out, mod, pos, cu, n_seqs, max_seqlen, n, table, wq, wqs, bq, wo, wos, bo, ws, bytes, s)
    args = [fake, fake, fake, fake, fake, 1, 100, 100, fake, fake, fake, None, fake, fake, None]
    st = jav._lib.dit_block_forward_fp8(ctypes.byref(desc), *args, fake, 10, None)
    assert st == jav.DIT_EWORKSPACE
    f32 = jav.block_desc(F32, 256, 4, 64, (16, 24, 24))
    st = jav._lib.dit_block_forward_fp8(ctypes.byref(f32), *args, fake, 1 << 40, None)
    assert st == jav.DIT_EUNSUPPORTED            # bf16 activations only
    a2 = list(args)
    a2[10] = fake + 8                            # w_qkv scales misaligned
    st = jav._lib.dit_block_forward_fp8(ctypes.byref(desc), *a2, fake, 1 << 40, None)
    assert st == jav.DIT_EUNSUPPORTED
    a2 = list(args)
    a2[9] = None                                 # no w_qkv
    st = jav._lib.dit_block_forward_fp8(ctypes.byref(desc), *a2, fake, 1 << 40, None)
    assert st == jav.DIT_EINVAL
    odd = jav.block_desc(B, 192, 3, 64, (16, 24, 24))   # d_model not a multiple of 128
    st = jav._lib.dit_block_forward_fp8(ctypes.byref(odd), *args, fake, 1 << 40, None)
    assert st == jav.DIT_EUNSUPPORTED
    st = jav._lib.dit_block_forward_fp8(ctypes.byref(desc), *args[:7], 0, *args[8:], fake,
                                        1 << 40, None)
    assert st == jav.DIT_OK                      # no rows: nothing enqueued

    fdesc = jav.ffn_desc(B, 5120, 20480)
    want = (((n * 20480 + 255) // 256) * 256 + ((n * 20480 * 2 + 255) // 256) * 256
            + ((n * 4 + 255) // 256) * 256)
    assert jav.ffn_fp8_workspace_bytes(fdesc, n) == want
    # (desc, x, out, mod, n, table, w1, w1s, b1, w2, w2s, b2, ws, bytes, s)
    fargs = [fake, fake, fake, 100, fake, fake, fake, None, fake, fake, None]
    assert jav._lib.dit_ffn_forward_fp8(ctypes.byref(fdesc), *fargs, fake, 10, None) == jav.DIT_EWORKSPACE
    wide = jav.ffn_desc(B, 5120, 20480 + 128)
    assert jav._lib.dit_ffn_forward_fp8(ctypes.byref(wide), *fargs, fake, 1 << 40, None) == jav.DIT_EUNSUPPORTED
    narrow = jav.ffn_desc(B, 5120, 20480 - 64)
    assert jav._lib.dit_ffn_forward_fp8(ctypes.byref(narrow), *fargs, fake, 1 << 40, None) == jav.DIT_EUNSUPPORTED
    assert jav.ffn_fp8_workspace_bytes(jav.ffn_desc(F32, 256, 1024), 10) == 0


def test_fp8_attention_layout_and_validation():
    """Workspace layout arithmetic of the FP8 attention operands and the
    argument checks of attn_fp8_prepare / attn_packed_fp8 (nothing enqueued)."""
    n, s, h = 58758, 1, 40
    lay = jav.attn_fp8_layout(n, s, h)
    r = lambda b: (b + 255) // 256 * 256
    ld_vt = (n + 63) // 64 * 64 + 128 * s
    assert lay["ld8"] == h * 128 and lay["ld_vt"] == ld_vt
    sizes = [n * h * 128, n * h * 128, h * 128 * ld_vt, h * n * 4, h * 4, h * 4, 2 * h * 4]
    offs = [0]
    for b in sizes:
        offs.append(offs[-1] + r(b))
    assert [lay[k] for k in ("q8", "k8", "vt", "sq", "sk", "sv", "amax")] == offs[:-1]
    assert jav.attn_fp8_workspace_bytes(n, s, h) == offs[-1]
    assert jav.attn_fp8_workspace_bytes(n, s, h, 64) == 0
    assert jav.attn_fp8_workspace_bytes(n, 0, h) == 0
    with pytest.raises(jav.DitError):
        jav.attn_fp8_layout(n, s, h, 64)
    fake = 1 << 20
    need = jav.attn_fp8_workspace_bytes(100, 1, 40)
    # attn_fp8_prepare(q, ld_q, k, ld_k, v, ld_v, cu, n_seqs, max_seqlen, n, H, dh, ws, bytes, stream)
    Q = [fake, 5120, fake, 5120, fake, 5120]
    assert _call("attn_fp8_prepare", None, 5120, fake, 5120, fake, 5120, fake, 1, 100, 100, 40, 128, fake, need, None) == jav.DIT_EINVAL
    assert _call("attn_fp8_prepare", *Q, fake, 1, 100, 100, 40, 64, fake, need, None) == jav.DIT_EUNSUPPORTED
    assert _call("attn_fp8_prepare", *Q, fake, 1, 100, 100, 40, 128, fake, need - 1, None) == jav.DIT_EWORKSPACE
    assert _call("attn_fp8_prepare", fake, 5000, fake, 5120, fake, 5120, fake, 1, 100, 100, 40, 128, fake, need, None) == jav.DIT_EINVAL
    assert _call("attn_fp8_prepare", fake + 8, 5120, fake, 5120, fake, 5120, fake, 1, 100, 100, 40, 128, fake, need, None) == jav.DIT_EUNSUPPORTED
    assert _call("attn_fp8_prepare", *Q, fake, 1, 101, 100, 40, 128, fake, need, None) == jav.DIT_EINVAL   # max_seqlen > n
    assert _call("attn_fp8_prepare", *Q, fake, 0, 100, 100, 40, 128, fake, need, None) == jav.DIT_EINVAL   # n_seqs
    assert "attn_fp8_prepare" in jav.last_error()
    # attn_packed_fp8(ws, bytes, o, ld_o, cu, n_seqs, max_seqlen, n, H, dh, scale, causal, stream)
    assert _call("attn_packed_fp8", fake, need, None, 5120, fake, 1, 100, 100, 40, 128, 0.0, 0, None) == jav.DIT_EINVAL
    assert _call("attn_packed_fp8", fake, need, fake, 5120, fake, 1, 100, 100, 40, 128, -1.0, 0, None) == jav.DIT_EINVAL
    assert _call("attn_packed_fp8", fake, need, fake, 4096, fake, 1, 100, 100, 40, 128, 0.0, 0, None) == jav.DIT_EINVAL
    assert _call("attn_packed_fp8", fake, 10, fake, 5120, fake, 1, 100, 100, 40, 128, 0.0, 0, None) == jav.DIT_EWORKSPACE
    assert _call("attn_packed_fp8", fake, need, fake + 2, 5120, fake, 1, 100, 100, 40, 128, 0.0, 0, None) == jav.DIT_EUNSUPPORTED
    assert _call("attn_packed_fp8", fake, need, fake, 5120, fake, 1, 0, 0, 40, 128, 0.0, 0, None) == jav.DIT_OK


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_pack_count_matches_layout(name):
    grids = [r.grid for r in synth.WORKLOADS[name].requests]
    lay = oracle.pack_layout(grids)
    assert jav.pack_count(grids) == (lay["n_tokens"], max(
        b - a for a, b in zip(lay["cu_seqlens"], lay["cu_seqlens"][1:])))


def test_pack_count_rejects_and_edge_cases():
    assert jav.pack_count([(0, 0, 0, 0, 0)]) == (0, 0)
    assert jav.pack_count([(1, 2, 3, 4, 5), (0, 0, 0, 0, 7)]) == (6 + 8 + 5 + 7, 19)
    for bad in ([], [(1, 1, -1, 0, 0)], [(1, 1, 1, 0, -2)], [(2000, 2000, 1000, 0, 0)]):
        with pytest.raises(jav.DitError) as e:
            jav.pack_count(bad)
        assert e.value.status == jav.DIT_EINVAL


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_block_intermediates_fit_the_workspace(name):
    """y, q', k', v and o: five distinct [N][D] planes, 256-byte aligned, inside
    dit_block_workspace_bytes."""
    wl = synth.WORKLOADS[name]
    code = jav.DIT_BF16 if wl.dtype == "bf16" else jav.DIT_F32
    desc = jav.block_desc(code, wl.d_model, wl.n_heads, wl.head_dim, wl.sections)
    n, es = wl.n_tokens, 2 if wl.dtype == "bf16" else 4
    offs = jav.block_intermediates(desc, n)
    total = jav.block_workspace_bytes(desc, n)
    assert list(offs) == ["y", "q_rot", "k_rot", "v", "o"]
    spans = sorted((o, o + n * wl.d_model * es) for o in offs.values())
    assert all(o % 256 == 0 for o, _ in spans)
    assert all(b <= c for (_, b), (c, _) in zip(spans, spans[1:]))
    assert spans[-1][1] <= total
    with pytest.raises(jav.DitError):
        jav.block_intermediates(desc, -1)
