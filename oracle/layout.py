"""Token arithmetic and packing of one request (pure Python ints).

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

MOD_VIDEO, MOD_AUDIO, MOD_TEXT = 0, 1, 2

# [H3-NFT], section "MiniMax H3 and Why Joint Audio-Video Generation
# Complicates RL Training": the visual VAE compresses 16x in space and 4x in
# time (temporally causal), and a 1x2x2 patchify follows, so a latent token
# covers 32x32 pixels of one latent frame.
VAE_SPATIAL = 16
PATCH_SPATIAL = 2
SPATIAL_DOWNSAMPLE = VAE_SPATIAL * PATCH_SPATIAL       # 32
TEMPORAL_DOWNSAMPLE = 4
# Same section: the audio VAE maps 32 kHz stereo audio to 40 latent tokens per
# second per channel, each channel on its own, so one token covers 800 samples.
AUDIO_SAMPLE_RATE = 32000
AUDIO_TOKEN_RATE = 40
SAMPLES_PER_AUDIO_TOKEN = AUDIO_SAMPLE_RATE // AUDIO_TOKEN_RATE   # 800
AUDIO_CHANNELS = 2


def grid_from_media(frames: int, height_px: int, width_px: int,
                    audio_samples_per_ch: int, text_len: int) -> Tuple[int, int, int, int, int]:
    """Latent token grid of one request from its media dimensions.

    Reading of [H3-NFT] (section on H3's architecture): a temporally causal
    4x VAE keeps the first frame on its own and folds each later group of 4
    frames into one latent frame, so F pixel frames give 1 + (F - 1) / 4 latent
    frames; the 121-frame clip the page mentions (section "Limitations of the
    Current Pipeline") gives 31.  Height and width must be multiples of the
    32x spatial factor, the audio sample count a multiple of 800; nothing is
    cropped or padded.  Raises ValueError otherwise.

    Returns (t, h, w, audio_tokens_per_channel, text_len).
    """
    for name, v in (("frames", frames), ("height_px", height_px),
                    ("width_px", width_px),
                    ("audio_samples_per_ch", audio_samples_per_ch),
                    ("text_len", text_len)):
        if not isinstance(v, int) or v < 0:
            raise ValueError(f"{name} must be a non-negative int, got {v!r}")
    if frames == 0:
        t = 0
    elif (frames - 1) % TEMPORAL_DOWNSAMPLE != 0:
        raise ValueError(f"frames - 1 = {frames - 1} is not a multiple of {TEMPORAL_DOWNSAMPLE}")
    else:
        t = 1 + (frames - 1) // TEMPORAL_DOWNSAMPLE
    if height_px % SPATIAL_DOWNSAMPLE or width_px % SPATIAL_DOWNSAMPLE:
        raise ValueError(f"{height_px}x{width_px} px is not a multiple of {SPATIAL_DOWNSAMPLE}")
    if audio_samples_per_ch % SAMPLES_PER_AUDIO_TOKEN:
        raise ValueError(f"{audio_samples_per_ch} samples is not a multiple of "
                         f"{SAMPLES_PER_AUDIO_TOKEN}")
    h = height_px // SPATIAL_DOWNSAMPLE
    w = width_px // SPATIAL_DOWNSAMPLE
    if t == 0 or h == 0 or w == 0:
        t = h = w = 0
    return (t, h, w, audio_samples_per_ch // SAMPLES_PER_AUDIO_TOKEN, text_len)


def request_length(grid: Sequence[int]) -> int:
    t, h, w, a, L = grid
    return t * h * w + AUDIO_CHANNELS * a + L


def pack_layout(grids: Sequence[Sequence[int]]) -> Dict[str, object]:
    """Packed modality ids, (t, h, w) positions and cu_seqlens of several requests.

    [vLLM-Omni] section "3. Packed Sequences and Modality Identity
    Preservation": rows of each modality carry a modality tag and their
    temporal/spatial position, the rows are concatenated into one 1-D
    sequence, and cu_seqlens holds the cumulative offsets of the
    sub-sequences.  Section 1's pipeline table orders a request as video
    latents, then audio latents, then text.  Readings (the pages do not fix
    them): video rows in row-major (t, h, w) order, w fastest; audio channel 0
    for all its frames, then channel 1, both with position (k, 0, 0); text
    token j at (j, 0, 0); every request and every modality starts at
    position 0; one cu_seqlens segment per request.

    Returns dict(modality=[int], pos=[(t, h, w)], cu_seqlens=[int],
    max_seqlen=int, n_tokens=int).
    """
    modality: List[int] = []
    pos: List[Tuple[int, int, int]] = []
    cu = [0]
    max_len = 0
    for g in grids:
        t_n, h_n, w_n, a_n, L = (int(v) for v in g)
        if min(t_n, h_n, w_n, a_n, L) < 0:
            raise ValueError("negative grid entry")
        for t in range(t_n):
            for h in range(h_n):
                for w in range(w_n):
                    modality.append(MOD_VIDEO)
                    pos.append((t, h, w))
        for _channel in range(AUDIO_CHANNELS):
            for k in range(a_n):
                modality.append(MOD_AUDIO)
                pos.append((k, 0, 0))
        for j in range(L):
            modality.append(MOD_TEXT)
            pos.append((j, 0, 0))
        n = len(modality) - cu[-1]
        if n != request_length((t_n, h_n, w_n, a_n, L)):
            raise AssertionError("request length mismatch")
        cu.append(len(modality))
        max_len = max(max_len, n)
    return dict(modality=modality, pos=pos, cu_seqlens=cu, max_seqlen=max_len,
                n_tokens=len(modality))
