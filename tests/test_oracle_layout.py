"""Pins of the oracle's token arithmetic and packing (CPU only)."""
import json
import os

import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_page_values_token_arithmetic():
    g = _golden("token_arithmetic.json")
    assert oracle.SPATIAL_DOWNSAMPLE == g["spatial_downsample"]
    assert oracle.SAMPLES_PER_AUDIO_TOKEN == g["samples_per_audio_token"]
    t, h, w, a, L = oracle.grid_from_media(g["clip_frames"], 32, 32, 0, 0)
    assert t == g["clip_latent_frames"]
    t, h, w, a, L = oracle.grid_from_media(1, *g["train_resolution"], 0, 0)
    assert (h, w) == tuple(g["train_grid"])
    _, _, _, a, _ = oracle.grid_from_media(0, 0, 0, g["one_second_stereo_samples_per_ch"], 0)
    assert a == g["one_second_tokens_per_ch"]
    with pytest.raises(ValueError):
        oracle.grid_from_media(1, *g["reference_image"], 0, 0)
    assert g["full_pack_aligned"] - g["full_pack_tokens"] == g["full_pack_padding"]


@pytest.mark.parametrize("bad", [
    (120, 256, 256, 0, 0),      # (F-1) % 4 != 0
    (5, 250, 256, 0, 0),        # height not a multiple of 32
    (5, 256, 100, 0, 0),
    (5, 256, 256, 801, 0),      # not a whole number of audio tokens
    (-1, 256, 256, 0, 0),
    (5, 256, 256, 0, -3),
])
def test_rejects_non_divisible_media(bad):
    with pytest.raises(ValueError):
        oracle.grid_from_media(*bad)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_media_round_trip(name):
    wl = synth.WORKLOADS[name]
    total = 0
    for r in wl.requests:
        assert oracle.grid_from_media(*r.media) == r.grid
        total += oracle.request_length(r.grid)
    assert total == wl.expected_tokens
    lay = oracle.pack_layout([r.grid for r in wl.requests])
    assert lay["cu_seqlens"] == list(wl.expected_cu_seqlens)
    assert lay["n_tokens"] == wl.expected_tokens


def test_full_pack_matches_page_token_count():
    g = _golden("token_arithmetic.json")
    wl = synth.WORKLOADS["full"]
    assert wl.expected_tokens == g["full_pack_tokens"]
    # The last 64-key tile of the full pack is ragged: 58,758 = 918 * 64 + 6.
    assert g["full_pack_tokens"] % 64 == 6


def test_cu_seqlens_page_example():
    g = _golden("cu_seqlens_example.json")
    two = oracle.pack_layout([(0, 0, 0, 0, n) for n in g["lengths_two"]])
    assert two["cu_seqlens"] == g["cu_two"]
    three = oracle.pack_layout([(0, 0, 0, 0, n) for n in g["lengths_three"]])
    assert three["cu_seqlens"] == g["cu_three"]
    assert three["max_seqlen"] == 20


def test_pack_tiny_golden():
    g = _golden("pack_tiny.json")
    lay = oracle.pack_layout(g["grids"])
    assert lay["modality"] == g["modality"]
    assert [list(p) for p in lay["pos"]] == g["pos"]
    assert lay["cu_seqlens"] == g["cu_seqlens"]
    assert lay["max_seqlen"] == g["max_seqlen"]


@pytest.mark.parametrize("name", ["tiny", "small", "varlen"])
def test_pack_invariants(name):
    wl = synth.WORKLOADS[name]
    lay = oracle.pack_layout([r.grid for r in wl.requests])
    mod, pos, cu = lay["modality"], lay["pos"], lay["cu_seqlens"]
    for r, (a, b) in zip(wl.requests, zip(cu, cu[1:])):
        m = mod[a:b]
        p = pos[a:b]
        nv = r.t * r.h * r.w
        assert m.count(0) == nv and m.count(1) == 2 * r.audio_per_ch and m.count(2) == r.text_len
        # modality blocks are contiguous: video, then audio, then text
        assert m == sorted(m)
        vid = p[:nv]
        assert len(set(vid)) == nv
        assert all(0 <= t < r.t and 0 <= h < r.h and 0 <= w < r.w for t, h, w in vid)
        aud = p[nv:nv + 2 * r.audio_per_ch]
        for k in range(r.audio_per_ch):
            assert aud.count((k, 0, 0)) == 2
        txt = p[nv + 2 * r.audio_per_ch:]
        assert txt == [(j, 0, 0) for j in range(r.text_len)]
        # positions restart in every request
        assert p[0] == (0, 0, 0)
