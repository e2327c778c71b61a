"""Reference oracle for one block of the joint audio-video DiT.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only the test suite, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` use it.  It shares no code with the HIP
library and reads no value the library produced.

The oracle is plain and slow on purpose: integer layout work in pure Python
ints, floating-point stages in NumPy float64 with no intermediate rounding,
each stage written as its textbook definition.  ``oracle.brute`` repeats every
floating-point stage with explicit Python loops for tiny inputs.

Sources (cited by title and section throughout):

* [H3-NFT]     "DiffusionNFT on MiniMax H3: Open-Source RL Training for Joint
               Audio-Video Generation" (gpts24.com news page).
* [VeRL-Omni]  "多模态强化学习工程解析：VeRL-Omni 架构与 MiniMax-H3 训练实录"
               (princepride.github.io, VeRL-Omni RL blog).
* [vLLM-Omni]  "Joint Audio-Video Generation in Production: Architecture Deep
               Dive into MiniMax-H3 and vLLM-Omni" (princepride.github.io,
               vLLM-Omni blog, English).

Readings where those pages leave a step open are listed in each function's
docstring.  Pins for every function live in ``tests/test_oracle_*.py``.
Parity of the pack order and of the RoPE pair convention is pinned by the
stated readings only (the pages fix neither), see ``oracle.layout`` and
``oracle.block.rope3d``; so are the feed-forward half's activation (tanh
GELU) and width (4 x d_model), see ``oracle.block.gelu_tanh`` and
``oracle.block.ffn_forward``.  ``oracle.denoise`` holds the denoising step
around the block (Rectified Flow X0, Euler with eta = 0, dual schedules,
anchor re-pinning, H3's timestep and velocity conventions); ``oracle.nft`` the
DiffusionNFT loss and its gradient; ``oracle.fp8`` the e4m3 quantization and the
FP8 projections and the FP8 block halves; ``oracle.backward`` the gradients
of the attention half (the chain rule through the forward definitions).
"""
from .layout import (MOD_AUDIO, MOD_TEXT, MOD_VIDEO, SAMPLES_PER_AUDIO_TOKEN,
                     SPATIAL_DOWNSAMPLE, TEMPORAL_DOWNSAMPLE, grid_from_media,
                     pack_layout, request_length)
from .block import (adaln_modulate, attention, attention_probs, block_forward,
                    ffn_forward, ffn_up, gelu_tanh, out_proj_gated, qkv_project, rope3d,
                    rope_frequencies)
from .denoise import (VIDEO_LATENT_CHANNELS, clean_estimate, denoise_loop, denoise_step,
                      euler_step, standard_velocity, timestep_from_sigma)
from .nft import implicit_policies, nft_loss
from .backward import (adaln_backward, attention_backward, attention_backward_rows,
                       attention_lse, block_backward, ffn_backward, gelu_tanh_grad,
                       rope3d_backward)
from .fp8 import (E4M3_MAX, adaln_modulate_fp8, attention_fp8, attention_fp8_operands,
                  dequantize_attention_operands, quantize_tensor, block_forward_fp8, dequantize_rows, e4m3_decode,
                  e4m3_encode, e4m3_encode_bruteforce, e4m3_table, ffn_forward_fp8, linear_fp8,
                  quantize_rows, row_scales)

__all__ = [
    "MOD_VIDEO", "MOD_AUDIO", "MOD_TEXT", "SAMPLES_PER_AUDIO_TOKEN",
    "SPATIAL_DOWNSAMPLE", "TEMPORAL_DOWNSAMPLE", "grid_from_media",
    "pack_layout", "request_length", "adaln_modulate", "qkv_project",
    "rope3d", "rope_frequencies", "attention", "attention_probs",
    "out_proj_gated", "block_forward", "gelu_tanh", "ffn_up", "ffn_forward",
    "VIDEO_LATENT_CHANNELS", "timestep_from_sigma", "standard_velocity", "clean_estimate",
    "euler_step", "denoise_step", "denoise_loop", "implicit_policies", "nft_loss",
    "E4M3_MAX", "e4m3_decode", "e4m3_table", "e4m3_encode", "e4m3_encode_bruteforce",
    "row_scales", "quantize_rows", "quantize_tensor", "attention_fp8_operands",
    "dequantize_attention_operands", "attention_fp8", "dequantize_rows", "linear_fp8", "adaln_modulate_fp8",
    "block_forward_fp8", "ffn_forward_fp8", "attention_backward", "rope3d_backward",
    "adaln_backward", "block_backward", "attention_lse", "attention_backward_rows",
    "ffn_backward", "gelu_tanh_grad",
]
