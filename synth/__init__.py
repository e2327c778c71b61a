"""Seeded synthetic inputs for the joint audio-video DiT block.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It holds workload descriptions (sizes, grids, seeds and value
distributions) and random-number generation only: no step of the block's
arithmetic lives here.  Token layouts (modality ids, positions, cu_seqlens)
are derived separately by the oracle and by the library from the per-request
grids listed below.

Workloads follow the one pack the vLLM-Omni deep-dive page describes
(video latents, then audio latents, then text tokens; 58,758 effective tokens
per request, section "1. Unified Architecture and the 118 GB VRAM Wall"),
scaled to five sizes.  Media dimensions are listed beside each grid so that
the token arithmetic can be checked against them.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Request:
    """One request of a pack.

    Grid: video latent grid (t, h, w), audio latent tokens per stereo channel,
    text tokens.  Media: the pixel/sample dimensions that produce that grid.
    """
    t: int
    h: int
    w: int
    audio_per_ch: int
    text_len: int
    frames: int
    height_px: int
    width_px: int
    audio_samples_per_ch: int

    @property
    def grid(self) -> Tuple[int, int, int, int, int]:
        return (self.t, self.h, self.w, self.audio_per_ch, self.text_len)

    @property
    def media(self) -> Tuple[int, int, int, int, int]:
        return (self.frames, self.height_px, self.width_px,
                self.audio_samples_per_ch, self.text_len)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    d_model: int
    n_heads: int
    head_dim: int
    sections: Tuple[int, int, int]
    requests: Tuple[Request, ...]
    seed: int
    theta: float = 10000.0
    eps: float = 1e-6
    expected_tokens: int = 0
    expected_cu_seqlens: Tuple[int, ...] = ()

    @property
    def n_tokens(self) -> int:
        return self.expected_tokens

    @property
    def d_ff(self) -> int:
        """Feed-forward width: 4 x d_model (a reading; the pages give none)."""
        return 4 * self.d_model


def _req(grid, media) -> Request:
    return Request(*grid, *media[:4])


# Five workloads: tiny fp32, small / medium / full-shape bf16, and the 4-request
# varlen pack (run both bidirectional and causal).
WORKLOADS = {
    "tiny": Workload(
        "tiny", F32, 256, 4, 64, (16, 24, 24),
        (_req((4, 8, 8, 20, 32), (13, 256, 256, 16000, 32)),),
        seed=1, expected_tokens=328, expected_cu_seqlens=(0, 328)),
    "small": Workload(
        "small", BF16, 1536, 12, 128, (32, 48, 48),
        (_req((8, 16, 30, 100, 56), (29, 512, 960, 80000, 56)),),
        seed=2, expected_tokens=4096, expected_cu_seqlens=(0, 4096)),
    "medium": Workload(
        "medium", BF16, 3072, 24, 128, (32, 48, 48),
        (_req((12, 30, 44, 260, 24), (45, 960, 1408, 208000, 24)),),
        seed=3, expected_tokens=16384, expected_cu_seqlens=(0, 16384)),
    "full": Workload(
        "full", BF16, 5120, 40, 128, (32, 48, 48),
        (_req((20, 46, 62, 800, 118), (77, 1472, 1984, 640000, 118)),),
        seed=4, expected_tokens=58758, expected_cu_seqlens=(0, 58758)),
    "varlen": Workload(
        "varlen", BF16, 5120, 40, 128, (32, 48, 48),
        tuple(_req((11, 30, 43, 240, L), (41, 960, 1376, 192000, L))
              for L in (20, 20, 19, 19)),
        seed=5, expected_tokens=58758,
        expected_cu_seqlens=(0, 14690, 29380, 44069, 58758)),
}

# Aligned length of the full-shape pack and its padding (vLLM-Omni deep dive,
# section "6. Boundary Trimming for Packed Attention", table): buffers of this
# many rows whose tail rows hold garbage must give the same result as the
# trimmed run.
FULL_ALIGNED_TOKENS = 58816


# ---------------------------------------------------------------------------
# bf16 storage helpers (input formatting: round-to-nearest-even, done once)
# ---------------------------------------------------------------------------

def _bf16_rounded_words(a: np.ndarray) -> np.ndarray:
    """float32 bit patterns rounded to bfloat16 (nearest, ties to even) in the high
    half.  In uint32 the sum wraps only for NaN inputs, which callers replace."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    return r


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = (_bf16_rounded_words(a) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array whose values are exactly representable in bfloat16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    r = _bf16_rounded_words(a)
    r &= np.uint32(0xFFFF0000)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint32(0x7FC00000)
    return r.view(np.float32)


# ---------------------------------------------------------------------------
# Seeded draws
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class BlockInputs:
    """Float32 host arrays; for bf16 workloads every value is bf16-exact."""
    x: np.ndarray          # [N][D], N(0, 1)
    table: np.ndarray      # [3][3][D], N(0, 0.1): per modality rows shift, scale, gate
    w_qkv: np.ndarray      # [3D][D], N(0, 0.02)
    w_o: np.ndarray        # [D][D], N(0, 0.02)
    b_qkv: Optional[np.ndarray] = None   # [3D], N(0, 0.02) when drawn
    b_o: Optional[np.ndarray] = None     # [D]


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def block_inputs(wl: Workload, n_tokens: Optional[int] = None,
                 with_bias: bool = False, seed: Optional[int] = None) -> BlockInputs:
    """Draw x, table, W_qkv, W_o (then biases) in that fixed order from PCG64(seed)."""
    n = wl.n_tokens if n_tokens is None else n_tokens
    d = wl.d_model
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    x = _normal(rng, (n, d), 1.0)
    table = _normal(rng, (3, 3, d), 0.1)
    w_qkv = _normal(rng, (3 * d, d), 0.02)
    w_o = _normal(rng, (d, d), 0.02)
    b_qkv = b_o = None
    if with_bias:
        b_qkv = _normal(rng, (3 * d,), 0.02)
        b_o = _normal(rng, (d,), 0.02)
    if wl.dtype == BF16:
        x, w_qkv, w_o = round_to_bf16(x), round_to_bf16(w_qkv), round_to_bf16(w_o)
        if with_bias:
            b_qkv, b_o = round_to_bf16(b_qkv), round_to_bf16(b_o)
    return BlockInputs(x, table, w_qkv, w_o, b_qkv, b_o)


@dataclasses.dataclass
class FfnInputs:
    """Float32 host arrays for the feed-forward half; bf16-exact for bf16 workloads."""
    table: np.ndarray      # [3][3][D], N(0, 0.1): MLP rows shift, scale, gate per modality
    w1: np.ndarray         # [F][D], N(0, 0.02)   (ff.net.0.proj)
    w2: np.ndarray         # [D][F], N(0, 0.02)   (ff.net.2)
    b1: Optional[np.ndarray] = None   # [F], N(0, 0.02) when drawn
    b2: Optional[np.ndarray] = None   # [D]


def ffn_inputs(wl: Workload, with_bias: bool = False, seed: Optional[int] = None) -> FfnInputs:
    """Draw the MLP table, W1, W2 (then biases) in that order from PCG64(seed), a stream of
    its own (default wl.seed + 1000) so the attention-half draws are unchanged; the
    half's input x is the block's x."""
    d, f = wl.d_model, wl.d_ff
    rng = np.random.Generator(np.random.PCG64(wl.seed + 1000 if seed is None else seed))
    table = _normal(rng, (3, 3, d), 0.1)
    w1 = _normal(rng, (f, d), 0.02)
    w2 = _normal(rng, (d, f), 0.02)
    b1 = b2 = None
    if with_bias:
        b1 = _normal(rng, (f,), 0.02)
        b2 = _normal(rng, (d,), 0.02)
    if wl.dtype == BF16:
        w1, w2 = round_to_bf16(w1), round_to_bf16(w2)
        if with_bias:
            b1, b2 = round_to_bf16(b1), round_to_bf16(b2)
    return FfnInputs(table, w1, w2, b1, b2)


def normal_array(shape, seed: int, std: float = 1.0, dtype: str = F32) -> np.ndarray:
    """Seeded N(0, std^2) float32 array, bf16-exact when dtype is bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = _normal(rng, shape, std)
    return round_to_bf16(a) if dtype == BF16 else a


def uniform_ints(shape, low: int, high: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(low, high, size=shape, dtype=np.int64)


def random_segments(n_tokens: int, n_segs: int, seed: int, min_len: int = 1) -> List[int]:
    """Seeded cumulative offsets [0, ..., n_tokens] splitting n_tokens into n_segs parts."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cuts = set()
    while len(cuts) < n_segs - 1:
        c = int(rng.integers(min_len, n_tokens - min_len + 1))
        cuts.add(c)
    offs = [0] + sorted(cuts) + [n_tokens]
    return offs


@dataclasses.dataclass
class DenoiseInputs:
    """Float32 host arrays for one denoising step over a packed latent state."""
    z: np.ndarray            # [N][C] state, N(0, 1)
    v: np.ndarray            # [N][C] predicted velocity, N(0, 1); bf16-exact for bf16 workloads
    anchor_vals: np.ndarray  # [N][C] original values of anchor rows, N(0, 1)


def denoise_inputs(wl: Workload, channels: int = 96, n_rows: Optional[int] = None,
                   seed: Optional[int] = None) -> DenoiseInputs:
    """Draw z, v, anchor values in that order from PCG64(seed) (default wl.seed + 2000).

    The state stays float32 (it carries 50 steps of updates); the velocity has
    the workload's dtype, as the DiT's output head would produce it."""
    n = wl.n_tokens if n_rows is None else n_rows
    rng = np.random.Generator(np.random.PCG64(wl.seed + 2000 if seed is None else seed))
    z = _normal(rng, (n, channels), 1.0)
    v = _normal(rng, (n, channels), 1.0)
    a = _normal(rng, (n, channels), 1.0)
    if wl.dtype == BF16:
        v = round_to_bf16(v)
    return DenoiseInputs(z, v, a)


def sigma_schedule(n_steps: int, power: float = 1.0) -> np.ndarray:
    """A synthetic decreasing schedule sigma_i = (1 - i / n_steps) ** power, i = 0..n_steps,
    in float32 (the pages give no sigma values)."""
    i = np.arange(n_steps + 1, dtype=np.float64)
    return ((1.0 - i / n_steps) ** power).astype(np.float32)


@dataclasses.dataclass
class NftInputs:
    """Float32 host arrays for the DiffusionNFT loss over a packed batch."""
    v_theta: np.ndarray     # [N][C] current policy's velocity: v_old + N(0, 0.05^2)
    v_old: np.ndarray       # [N][C] frozen adapter's velocity, N(0, 1)
    v_target: np.ndarray    # [N][C] eps - x0 with eps, x0 ~ N(0, 1)
    reward: np.ndarray      # [S] uniform in [0, 1)


def nft_inputs(wl: Workload, n_samples: int, channels: int = 96, n_rows: Optional[int] = None,
               seed: Optional[int] = None) -> NftInputs:
    """Draw v_old, the policy's drift, eps, x0 and the rewards in that order from
    PCG64(seed) (default wl.seed + 3000).  Velocities are bf16-exact for bf16 workloads
    (network outputs); the target stays float32."""
    n = wl.n_tokens if n_rows is None else n_rows
    rng = np.random.Generator(np.random.PCG64(wl.seed + 3000 if seed is None else seed))
    v_old = _normal(rng, (n, channels), 1.0)
    drift = _normal(rng, (n, channels), 0.05)
    eps = _normal(rng, (n, channels), 1.0)
    x0 = _normal(rng, (n, channels), 1.0)
    reward = rng.random(n_samples, dtype=np.float32)
    v_theta = v_old + drift
    if wl.dtype == BF16:
        v_old, v_theta = round_to_bf16(v_old), round_to_bf16(v_theta)
    return NftInputs(v_theta, v_old, (eps - x0).astype(np.float32), reward)
