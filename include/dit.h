/*
 * dit.h -- C ABI of libdit: one block of the joint audio-video DiT (MiniMax-H3)
 * on one AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by title and section:
 *   [H3-NFT]    "DiffusionNFT on MiniMax H3: Open-Source RL Training for Joint
 *               Audio-Video Generation" (gpts24.com news page).
 *   [VeRL-Omni] "多模态强化学习工程解析：VeRL-Omni 架构与 MiniMax-H3 训练实录"
 *               (princepride.github.io VeRL-Omni RL blog).
 *   [vLLM-Omni] "Joint Audio-Video Generation in Production: Architecture Deep
 *               Dive into MiniMax-H3 and vLLM-Omni" (princepride.github.io
 *               vLLM-Omni blog, English).
 *
 * The block: per-modality AdaLN -> fused QKV projection -> 3D (t, h, w) RoPE on
 * q and k -> softmax attention inside cu_seqlens segments -> output projection
 * -> gated residual; then the feed-forward half (AdaLN -> ff.net.0.proj ->
 * GELU -> ff.net.2 -> gated residual).  Around the block: the denoising step
 * that advances the packed audio-video latent state after each DiT forward.
 *
 * Conventions shared by every device entry point
 * ----------------------------------------------
 * Ownership.  The caller owns every buffer.  The library allocates no device
 *   memory and keeps no per-call state (apart from the optional profiling
 *   events, which the caller creates and frees through dit_profile_*).
 * Execution.  Device entry points only enqueue work on `stream` (a
 *   hipStream_t; NULL means the null stream) and never synchronise.  DIT_OK
 *   means "validated and enqueued"; a fault inside a kernel surfaces at the
 *   caller's next synchronisation.
 * Layout.  Row-major, one token per row.  `ld_*` is the distance in elements
 *   between consecutive rows.  In a q/k/v/o row, head h occupies columns
 *   [h*head_dim, (h+1)*head_dim).  Weights are [out][in] (torch Linear): a
 *   projection computes x W^T.
 * Element types.  DIT_BF16: activations and weights are bfloat16 bit patterns
 *   (uint16); arithmetic is float32; every bf16 store rounds to nearest even.
 *   DIT_F32: everything float32.  The AdaLN table is float32 for both.
 * Effective length.  `n_tokens` is the effective token count.  Rows at or past
 *   n_tokens are never read or written, whatever the buffers' padded size, so
 *   a caller trims alignment padding by passing the effective length and a
 *   pointer offset, with no copy ([vLLM-Omni] section 6, "Boundary Trimming
 *   for Packed Attention").  n_tokens == 0 is a no-op returning DIT_OK.
 * Alignment.  Device pointers must be 16-byte aligned and every ld a multiple
 *   of 16 bytes (8 bf16 or 4 f32 elements); otherwise DIT_EUNSUPPORTED.
 * Errors.  Host-side argument checks return DIT_EINVAL / DIT_EUNSUPPORTED /
 *   DIT_EWORKSPACE before anything is enqueued; a failed launch returns
 *   DIT_EHIP.  dit_last_error() gives the calling thread's message for its
 *   last non-OK status.  There is never a silent fallback to another path: a
 *   combination a kernel does not implement is DIT_EUNSUPPORTED ([H3-NFT]
 *   section "The Six Silent Failures" and [VeRL-Omni] section 5.2 ask for an
 *   explicit error instead of a silent mis-registration).
 * Device-array contents are a contract and are not checked on the hot path:
 *   cu_seqlens[0] == 0, non-decreasing, cu_seqlens[n_seqs] == n_tokens, every
 *   segment no longer than max_seqlen, every modality id < 3, positions >= 0.
 *   dit_pack_layout() produces such arrays.  With DIT_VALIDATE=1 in the
 *   environment, the entry points that take cu_seqlens or modality ids
 *   (attention, AdaLN, the block and feed-forward halves, their FP8 and
 *   backward forms) first copy those arrays to the host on the call's stream,
 *   synchronously, and return DIT_EINVAL if they break the contract.  Without
 *   it, the attention kernels (bf16, FP8, backward) still guard one breach
 *   on the device: a segment longer than max_seqlen (which their grids and
 *   32-bit buffer ranges are sized from) gets NaN in its output rows (and its
 *   log-sum-exps) inside [0, n_tokens) instead of partly unwritten ones.
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIT_ABI_VERSION 1

typedef enum {
  DIT_OK = 0,
  DIT_EINVAL = 1,        /* bad argument (null pointer, inconsistent sizes, ...) */
  DIT_EUNSUPPORTED = 2,  /* valid but not implemented (head_dim, alignment, ...) */
  DIT_EWORKSPACE = 3,    /* workspace missing or too small */
  DIT_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} dit_status;

typedef enum { DIT_F32 = 0, DIT_BF16 = 1 } dit_dtype;

/* Modality ids of the packed sequence ([vLLM-Omni] section 3: each token
 * carries a text / video / audio tag). */
enum { DIT_MOD_VIDEO = 0, DIT_MOD_AUDIO = 1, DIT_MOD_TEXT = 2, DIT_NUM_MOD = 3 };

/* Rows of the per-modality AdaLN table, float32 [DIT_NUM_MOD][3][d_model]. */
enum { DIT_ADA_SHIFT = 0, DIT_ADA_SCALE = 1, DIT_ADA_GATE = 2 };

int dit_abi_version(void);

/* Message of the calling thread's last non-OK status ("" if none).  The
 * string stays valid until the thread's next library call. */
const char* dit_last_error(void);

/* ------------------------------------------------------------------------ */
/* Host-only integer layout (bit-exact)                                       */
/* ------------------------------------------------------------------------ */

/* Media of one request: pixel frames and size, audio samples per stereo
 * channel at 32 kHz, and text tokens. */
typedef struct {
  int32_t frames, height_px, width_px;
  int64_t audio_samples_per_ch;
  int32_t text_len;
} dit_media;

/* Token grid of one request: video latent grid t x h x w, audio latent tokens
 * per channel, text tokens. */
typedef struct {
  int32_t t, h, w, audio_per_ch, text_len;
} dit_grid;

/* [H3-NFT] section "MiniMax H3 and Why Joint Audio-Video Generation
 * Complicates RL Training": the video VAE compresses 16x in space and 4x in
 * time (temporally causal) and a 1x2x2 patchify follows (32x in space); the
 * audio VAE gives 40 latent tokens per second per channel of 32 kHz stereo
 * audio (800 samples per token).  t = 1 + (frames - 1) / 4, h = height_px / 32,
 * w = width_px / 32, audio_per_ch = audio_samples_per_ch / 800.  frames == 0,
 * or a zero height or width, gives a request without video (t = h = w = 0).
 * DIT_EINVAL for a null pointer, a negative count, (frames - 1) % 4 != 0,
 * a size not a multiple of 32, or samples not a multiple of 800 (nothing is
 * cropped or padded). */
dit_status dit_grid_from_media(const dit_media* m, dit_grid* g);

/* Pack n_reqs requests into one sequence ([vLLM-Omni] section 3, "Packed
 * Sequences and Modality Identity Preservation"; order video, audio, text as
 * in its section 1 pipeline table).  Per request: video rows in row-major
 * (t, h, w) order (w fastest) with id DIT_MOD_VIDEO and position (t, h, w);
 * then audio channel 0 frames k = 0..n-1, then channel 1 frames k = 0..n-1,
 * id DIT_MOD_AUDIO, position (k, 0, 0); then text token j, id DIT_MOD_TEXT,
 * position (j, 0, 0).  Positions restart at 0 in every request and modality.
 * Outputs (host buffers, caller-owned): modality[capacity_tokens] (uint8),
 * pos_thw[capacity_tokens][3] (int32), cu_seqlens[n_reqs + 1] (int32),
 * *n_tokens, *max_seqlen.  DIT_EINVAL for null pointers, n_reqs < 1, a
 * negative grid entry, or a total above capacity_tokens or INT32_MAX. */
dit_status dit_pack_layout(const dit_grid* reqs, int32_t n_reqs,
                           uint8_t* modality, int32_t* pos_thw, int32_t* cu_seqlens,
                           int64_t capacity_tokens, int64_t* n_tokens,
                           int32_t* max_seqlen);

/* Size of the pack dit_pack_layout would build, without building it: the
 * total token count (the capacity its host buffers need) and the longest
 * request.  One request holds t*h*w video + 2*audio_per_ch audio + text_len
 * text tokens ([H3-NFT] section "MiniMax H3 and Why Joint Audio-Video
 * Generation Complicates RL Training": stereo audio, one token stream per
 * channel; [vLLM-Omni] section 1 table: the three modalities of a request).
 * Host-only.  DIT_EINVAL for null pointers, n_reqs < 1, a negative grid entry
 * or a total above INT32_MAX; nothing is written on failure. */
dit_status dit_pack_count(const dit_grid* reqs, int32_t n_reqs, int64_t* n_tokens,
                          int32_t* max_seqlen);

/* ------------------------------------------------------------------------ */
/* Device stages (asynchronous on `stream`; all pointers device memory)      */
/* ------------------------------------------------------------------------ */

/* Per-modality adaptive LayerNorm ([H3-NFT] section on H3's architecture:
 * AdaLN branches per modality whose outputs can be precomputed and cached;
 * [VeRL-Omni] section 3: all modalities share AdaLN modulation).  For token i
 * with m = modality[i]: LayerNorm over d_model (biased variance, no affine of
 * its own), then y = xhat * (1 + table[m][SCALE]) + table[m][SHIFT].
 * x: [n_tokens][ld_x]; modality: uint8 [n_tokens]; table: f32 [3][3][d_model];
 * y: [n_tokens][ld_y], must not overlap x.  eps > 0 (1e-6 in the block).
 * DIT_EINVAL: null pointer, d_model < 1, ld < d_model, eps <= 0, bad dtype.
 * DIT_EUNSUPPORTED: d_model above 16384 or not a multiple of 8 (bf16) / 4 (f32). */
dit_status adaln_modulate(dit_dtype dt, const void* x, int64_t ld_x,
                          const uint8_t* modality, const float* table,
                          void* y, int64_t ld_y, int64_t n_tokens, int32_t d_model,
                          float eps, void* stream);

/* 3D rotary position embedding of q and k, in place ([H3-NFT] section on
 * H3's architecture: RoPE over time, height and width; [vLLM-Omni] section 3:
 * positions per row, modality-independent position spaces).  head_dim splits
 * into sections[0..2] (t, h, w) at offsets 0, s_t, s_t + s_h; inside section a
 * the adjacent pair (x[o+2j], x[o+2j+1]) is rotated by phi = pos[a] *
 * theta^(-2j / s_a): (u, w) -> (u cos phi - w sin phi, u sin phi + w cos phi).
 * Every head is rotated alike; a pair with phi == 0 is left bit-identical.
 * q: [n_tokens][ld_q], k: [n_tokens][ld_k] (may be strided views into one
 * fused qkv buffer); pos_thw: int32 [n_tokens][3].  k may be NULL (q only).
 * DIT_EINVAL: null q/pos, n_heads < 1, sections odd or not summing to
 * head_dim, theta <= 0, ld < n_heads * head_dim.
 * DIT_EUNSUPPORTED: head_dim not 64 or 128. */
dit_status rope3d_apply(dit_dtype dt, void* q, int64_t ld_q, void* k, int64_t ld_k,
                        const int32_t* pos_thw, int64_t n_tokens, int32_t n_heads,
                        int32_t head_dim, const int32_t sections[3], float theta,
                        void* stream);

/* rope3d_apply_to: the same rotation written to separate outputs: q_out gets
 * the rotated q and k_out the rotated k (k and k_out both NULL: q only).
 * Out of place, each line is read once and written once elsewhere, with no
 * read-modify-write of the same lines.  An output may be its own input (in
 * place) or the other input with the same pointer and ld (k_out = q: each
 * vector is read before it is overwritten); any other overlap between an
 * output and an input, or between the outputs, is DIT_EINVAL.  Errors as
 * rope3d_apply, plus DIT_EINVAL for a missing output or an output ld below
 * n_heads * head_dim. */
dit_status rope3d_apply_to(dit_dtype dt, const void* q, int64_t ld_q, const void* k,
                           int64_t ld_k, void* q_out, int64_t ld_qo, void* k_out, int64_t ld_ko,
                           const int32_t* pos_thw, int64_t n_tokens, int32_t n_heads,
                           int32_t head_dim, const int32_t sections[3], float theta, void* stream);

/* Softmax attention over a packed sequence ([vLLM-Omni] section 3: the
 * kernel derives its mask from cu_seqlens, so a token attends only to keys of
 * its own segment; section 1: audio and video share one attention context;
 * [H3-NFT] "Limitations": the released weights use full attention).  Per
 * segment [cu[s], cu[s+1]) and head h: o_i = sum_j softmax_j(scale q_i . k_j)
 * v_j over keys j of the segment (j <= i too when causal != 0).
 * q, k, v, o: [n_tokens][ld] with n_heads * head_dim columns used; o must not
 * overlap q, k or v.  cu_seqlens: device int32 [n_seqs + 1].  softmax_scale
 * 0 means 1/sqrt(head_dim).  Zero-length segments are allowed.
 * DIT_EINVAL: null pointer, n_seqs < 1, max_seqlen < 1 with n_tokens > 0,
 * n_heads < 1, ld too small, softmax_scale < 0.
 * DIT_EUNSUPPORTED: head_dim not 64 or 128 (bf16 needs 128). */
dit_status attn_packed(dit_dtype dt, const void* q, int64_t ld_q, const void* k,
                       int64_t ld_k, const void* v, int64_t ld_v, void* o, int64_t ld_o,
                       const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                       int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                       float softmax_scale, int32_t causal, void* stream);

/* Fused QKV projection ([VeRL-Omni] section 5.2: the rollout side packs the Q,
 * K and V projections into one matrix; [H3-NFT] names them to_q, to_k, to_v):
 * qkv = y W_qkv^T (+ b_qkv).  w_qkv rows are to_q, then to_k, then to_v:
 * [3 d_model][d_model]; b_qkv [3 d_model] or NULL; qkv: [n_tokens][ld_qkv]
 * with columns [0, D) q, [D, 2D) k, [2D, 3D) v; must not overlap y.
 * DIT_EINVAL: null pointer, ld too small.  DIT_EUNSUPPORTED: d_model not a
 * multiple of 64. */
dit_status qkv_project(dit_dtype dt, const void* y, int64_t ld_y, const void* w_qkv,
                       const void* b_qkv, void* qkv, int64_t ld_qkv, int64_t n_tokens,
                       int32_t d_model, void* stream);

/* Output projection to_out.0 ([H3-NFT]) and gated residual with the gate row of
 * the per-modality AdaLN table: out = x + table[m][GATE] * (o W_o^T + b_o).
 * o: [n_tokens][ld_o] (heads side by side); w_o [d_model][d_model]; b_o
 * [d_model] or NULL; x, out: [n_tokens][ld]; out may be x itself (in place),
 * but must not otherwise overlap x or o.  Errors as qkv_project. */
dit_status out_proj_gated(dit_dtype dt, const void* o, int64_t ld_o, const void* w_o,
                          const void* b_o, const void* x, int64_t ld_x,
                          const uint8_t* modality, const float* table, void* out,
                          int64_t ld_out, int64_t n_tokens, int32_t d_model, void* stream);

/* ------------------------------------------------------------------------ */
/* Feed-forward half: ff.net.0.proj -> GELU -> ff.net.2                       */
/* ------------------------------------------------------------------------ */

/* [H3-NFT] section "How VeRL-Omni's Adapter Architecture Keeps H3-Specific
 * Logic Contained" names the feed-forward weights ff.net.0.proj and ff.net.2;
 * [vLLM-Omni] section 3 (DiT stage of the packed data flow) runs attention and
 * an MLP in every block.  The activation is tanh-form GELU and the half is
 * modulated by its own per-modality AdaLN rows (readings; the pages give
 * neither).
 *
 * ffn_up_gelu: h = gelu_tanh(y W1^T + b1), gelu_tanh(z) =
 * 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).  y: [n_tokens][ld_y] (first
 * d_model columns used); w1: [d_ff][d_model] contiguous ([out][in]); b1:
 * [d_ff] or NULL; h: [n_tokens][ld_h], must not overlap y.  Computed in float32,
 * h rounded once (bf16: RNE).
 * Errors: DIT_EINVAL for a null pointer, d_model or d_ff < 1, ld too small;
 * DIT_EUNSUPPORTED when d_model or d_ff is not a multiple of 64 or a pointer,
 * bias or ld is not 16-byte aligned; DIT_EHIP on a launch failure. */
dit_status ffn_up_gelu(dit_dtype dt, const void* y, int64_t ld_y, const void* w1,
                       const void* b1, void* h, int64_t ld_h, int64_t n_tokens,
                       int32_t d_model, int32_t d_ff, void* stream);

/* ffn_down_gated: out = x + table[m][GATE] * (h W2^T + b2), with the gate row of
 * the feed-forward half's own AdaLN table.  h: [n_tokens][ld_h] (first d_ff
 * columns); w2: [d_model][d_ff] contiguous; b2: [d_model] or NULL; x, out:
 * [n_tokens][ld]; out may be x itself (in place) but must not otherwise overlap
 * x or h; modality: device uint8 [n_tokens]; table: device f32 [3][3][d_model].
 * Errors as ffn_up_gelu. */
dit_status ffn_down_gated(dit_dtype dt, const void* h, int64_t ld_h, const void* w2,
                          const void* b2, const void* x, int64_t ld_x,
                          const uint8_t* modality, const float* table, void* out,
                          int64_t ld_out, int64_t n_tokens, int32_t d_model, int32_t d_ff,
                          void* stream);

typedef struct {
  dit_dtype dtype;
  int32_t d_model, d_ff;   /* d_ff: 4 * d_model in the workloads here */
  float ln_eps;            /* 1e-6 */
} dit_ffn_desc;

/* Bytes of scratch dit_ffn_forward needs: y [N][D] + h [N][d_ff] elements, each
 * region rounded up to 256 bytes.  0 for a bad descriptor. */
size_t dit_ffn_workspace_bytes(const dit_ffn_desc* d, int64_t n_tokens);

/* The whole feed-forward half: y = AdaLN(x) with the half's table (shift,
 * scale rows), h = ffn_up_gelu(y), out = ffn_down_gated(h, x) (gate row).
 * x, out: [n_tokens][d_model] contiguous (out may equal x); modality: device
 * uint8 [n_tokens]; ada_table: device f32 [3][3][d_model] (the MLP rows);
 * w1 [d_ff][d_model]; w2 [d_model][d_ff]; biases nullable; workspace: device, at
 * least dit_ffn_workspace_bytes() bytes, 256-byte aligned.  Enqueues
 * adaln_modulate -> ffn_up_gelu -> ffn_down_gated on stream, after validating
 * all three.  Errors: those of the stages, plus DIT_EWORKSPACE. */
dit_status dit_ffn_forward(const dit_ffn_desc* d, const void* x, void* out,
                           const uint8_t* modality, int64_t n_tokens, const float* ada_table,
                           const void* w1, const void* b1, const void* w2, const void* b2,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Attention backward                                                         */
/* ------------------------------------------------------------------------ */

/* The gradient of attn_packed: the chain rule through softmax(q k^T scale) v
 * per segment and head (the pages print no backward pass; the DiffusionNFT
 * objective of [H3-NFT] section "DiffusionNFT: Skipping the Reverse Chain
 * Entirely" trains the DiT through it).  bf16, head_dim 128 only. */

/* attn_packed_lse: attn_packed that also writes lse float32
 * [n_heads][n_tokens] (device), lse[h][i] = log sum_j exp(q_i k_j^T scale)
 * over row i's keys.  Arguments and errors as attn_packed, plus DIT_EINVAL for
 * a null lse and DIT_EUNSUPPORTED for a dtype other than DIT_BF16. */
dit_status attn_packed_lse(dit_dtype dt, const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                           const void* v, int64_t ld_v, void* o, int64_t ld_o, float* lse,
                           const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                           int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                           float softmax_scale, int32_t causal, void* stream);

/* Bytes of scratch attn_packed_backward needs: n_heads * n_tokens floats
 * (delta = rowsum(dout * o) per head), rounded up to 256.  0 for bad sizes. */
size_t dit_attn_backward_workspace_bytes(int64_t n_tokens, int32_t n_heads);

/* attn_packed_backward: given q, k, v, the forward's o and lse and
 * dout = dL/do (all [n_tokens][ld] bf16 rows, lse as above), writes
 * dq = dL/dq, dk, dv ([n_tokens][ld] bf16, device; they must not overlap the
 * inputs).  P = exp(q k^T scale - lse) is recomputed; dv = P^T dout,
 * dS = P * (dout v^T - rowsum(dout * o)), dq = scale dS k, dk = scale dS^T q,
 * float32 accumulation.  Deterministic (no atomics).  Rows past a segment's
 * end are never read; rows outside every segment are not written.  Errors:
 * those of attn_packed (prefix attn_packed or attn_packed_backward), DIT_EINVAL
 * for a null dout / lse / dq / dk / dv or an ld below n_heads * head_dim,
 * DIT_EUNSUPPORTED for a dtype other than DIT_BF16, DIT_EWORKSPACE. */
dit_status attn_packed_backward(dit_dtype dt, const void* q, int64_t ld_q, const void* k,
                                int64_t ld_k, const void* v, int64_t ld_v, const void* o,
                                int64_t ld_o, const void* dout, int64_t ld_do, const float* lse,
                                void* dq, int64_t ld_dq, void* dk, int64_t ld_dk, void* dv,
                                int64_t ld_dv, const int32_t* cu_seqlens, int32_t n_seqs,
                                int32_t max_seqlen, int64_t n_tokens, int32_t n_heads,
                                int32_t head_dim, float softmax_scale, int32_t causal,
                                void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * attn_packed_backward with the same arguments, results and errors, minus
 * the workspace.  Its scratch (delta, n_heads * n_tokens floats) is a fixed
 * array in the library's device memory, one per GPU, kept until the process
 * ends; its address is looked up on the first call with a device current, so
 * the stream must belong to the current device.  Limit: n_heads * n_tokens <=
 * dit_attn_backward_noalloc_max_elements() (4,194,304: 40 heads x 58,758
 * tokens fit), otherwise DIT_EWORKSPACE.  Every call on one GPU uses that
 * GPU's array: calls that overlap on one GPU (other streams or threads) race
 * and must be serialised by the caller.  Allocates nothing. */
size_t dit_attn_backward_noalloc_max_elements(void);
dit_status attn_packed_backward_noalloc(dit_dtype dt, const void* q, int64_t ld_q, const void* k,
                                        int64_t ld_k, const void* v, int64_t ld_v, const void* o,
                                        int64_t ld_o, const void* dout, int64_t ld_do,
                                        const float* lse, void* dq, int64_t ld_dq, void* dk,
                                        int64_t ld_dk, void* dv, int64_t ld_dv,
                                        const int32_t* cu_seqlens, int32_t n_seqs,
                                        int32_t max_seqlen, int64_t n_tokens, int32_t n_heads,
                                        int32_t head_dim, float softmax_scale, int32_t causal,
                                        void* stream);

/* ------------------------------------------------------------------------ */
/* FP8 projections                                                            */
/* ------------------------------------------------------------------------ */

/* [vLLM-Omni] section 5 ("Distributed Layerwise Offload") runs the active DiT
 * layers in FP8; the pages give no scaling recipe.  Here: OCP e4m3 ("fn")
 * codes, one float32 scale per row (per token for activations, per output
 * channel for weights), scale = amax(|row|) / 448 (1 for an all-zero row),
 * code = e4m3(x * (1 / scale)) rounded to nearest with ties to the even code
 * and saturated at +-448; the two divisions are IEEE float32, once per row,
 * and the product one float32 rounding.  On gfx950 the e4m3 MFMA
 * runs at twice the bf16 rate. */

/* quantize_rows_fp8: x [n_rows][ld_x] of dt (bf16 or f32), first d columns ->
 * q uint8 [n_rows][ld_q] e4m3 codes and scales float32 [n_rows] (device).
 * Errors: DIT_EINVAL for a null pointer, d < 1, ld_x < d, ld_q < d, n_rows <
 * 0, an unknown dtype; DIT_EUNSUPPORTED for d not a multiple of 8 or above
 * 20480 (bf16; 10240 f32), or pointers / ld off the 16-byte rule (ld_q in
 * bytes); DIT_EHIP on a launch failure. */
dit_status quantize_rows_fp8(dit_dtype dt, const void* x, int64_t ld_x, uint8_t* q, int64_t ld_q,
                             float* scales, int64_t n_rows, int32_t d, void* stream);

/* adaln_modulate_fp8: adaln_modulate whose output y (float32, never rounded
 * to dt) leaves as per-row e4m3 codes q uint8 [n_tokens][ld_q] and scales
 * float32 [n_tokens], quantized by the rule above from y's float32 values.
 * Arguments and errors as adaln_modulate (prefix adaln_modulate_fp8), with
 * ld_q in bytes, a multiple of 16. */
dit_status adaln_modulate_fp8(dit_dtype dt, const void* x, int64_t ld_x,
                              const uint8_t* modality, const float* table, uint8_t* q,
                              int64_t ld_q, float* scales, int64_t n_tokens, int32_t d_model,
                              float eps, void* stream);

typedef enum { DIT_EPI_PLAIN = 0, DIT_EPI_GATED = 1, DIT_EPI_GELU = 2 } dit_epilogue;

/* linear_fp8: out = epi((decode(a) * a_scales[row]) (decode(w) * w_scales[col])^T
 * + bias), float32 accumulation, bf16 output (RNE).  a: e4m3 codes
 * [n_tokens][ld_a] (first k_in used); w: codes [n_out][k_in] contiguous
 * ([out][in]); a_scales [n_tokens], w_scales [n_out] float32; bias bf16
 * [n_out] or NULL.  epi PLAIN stores the product; GELU stores its tanh-form
 * GELU; GATED stores x + table[modality[row]][GATE] * product with x bf16
 * [n_tokens][ld_x], modality uint8 [n_tokens] and table float32 [3][3][n_out]
 * (out may be x, in place).  All pointers device.  Errors: DIT_EINVAL for a
 * null required pointer, an unknown epilogue, k_in or n_out < 1, an ld too
 * small, n_tokens < 0; DIT_EUNSUPPORTED when k_in is not a multiple of 128,
 * n_out not a multiple of 4, or a pointer / ld breaks the 16-byte rule;
 * DIT_EHIP on a launch failure. */
dit_status linear_fp8(const uint8_t* a, int64_t ld_a, const float* a_scales, const uint8_t* w,
                      const float* w_scales, const void* bias, dit_epilogue epi, const void* x,
                      int64_t ld_x, const uint8_t* modality, const float* table, void* out,
                      int64_t ld_out, int64_t n_tokens, int32_t k_in, int32_t n_out,
                      void* stream);

/* ------------------------------------------------------------------------ */
/* FP8 attention                                                              */
/* ------------------------------------------------------------------------ */

/* The attention of attn_packed ([vLLM-Omni] section 3: softmax inside each
 * cu_seqlens segment, full or causal) with both products in FP8 (section 5:
 * the active layers in FP8; no recipe on the pages).  Here: q is quantized
 * per (token, head) row, k and v with one scale per (segment, head) (amax /
 * 448 over the segment's rows of that head, 1 for an empty segment: a
 * request's codes do not depend on the other requests of its pack), codes and
 * scales as quantize_rows_fp8.  Scores
 * and the softmax are float32; the probabilities enter the second product as
 * e4m3 codes of 2^8 times their value relative to the row's running maximum
 * (at most 2^8.75), o is float32 until its bf16 store.  Against attention of
 * the dequantized operands with exact probabilities, an o element moves by at
 * most 2^-4 sum_k P_k |v_k| / sum_k P_k (plus 2^-18 max_k |v_k| per key for
 * probabilities below 2^-14 and the bf16 rounding of o).  bf16 inputs and
 * output, head_dim 128 only.  NaN inputs give unspecified results. */

/* Bytes of the operand workspace for n_tokens, n_seqs segments and n_heads:
 * q and k codes (n_tokens x n_heads x 128 bytes each), v codes transposed
 * (n_heads x 128 rows of ld_vt = roundup64(n_tokens) + 128 n_seqs bytes),
 * n_heads x n_tokens q scales, n_seqs x n_heads k and v scales and 2 x n_seqs
 * x n_heads words of scratch, each part rounded up to 256.  0 for bad sizes or a head_dim
 * other than 128. */
size_t dit_attn_fp8_workspace_bytes(int64_t n_tokens, int32_t n_seqs, int32_t n_heads,
                                    int32_t head_dim);

/* Byte offsets in that workspace, out[9] = {q8, k8, vt, sq, sk, sv, amax, ld8,
 * ld_vt}: q8 / k8 e4m3 codes [n_tokens][ld8 = n_heads * 128] ([token][head][d]),
 * vt e4m3 codes [n_heads * 128][ld_vt] (row h * 128 + d; segment s's key r at
 * column roundup64(cu_seqlens[s]) + 128 s + r, zero codes up to the segment's
 * next multiple of 64), sq float32 [n_heads][n_tokens], sk and sv float32
 * [n_seqs][n_heads].  Errors: DIT_EINVAL for a null out or bad sizes,
 * DIT_EUNSUPPORTED for head_dim != 128. */
dit_status dit_attn_fp8_layout(int64_t n_tokens, int32_t n_seqs, int32_t n_heads,
                               int32_t head_dim, int64_t* out);

/* attn_fp8_prepare: q, k, v bf16 [n_tokens][ld] (device; the first
 * n_heads * head_dim columns, [head][d]) -> the operands in workspace (device,
 * caller-owned, dit_attn_fp8_workspace_bytes), enqueued on stream.
 * cu_seqlens int32 [n_seqs + 1] (device), as attn_packed.  Errors: DIT_EINVAL
 * for a null pointer, n_seqs / n_heads < 1, an ld below n_heads * head_dim,
 * max_seqlen < 1 or above n_tokens; DIT_EUNSUPPORTED for head_dim != 128,
 * more than 65535 segments or 32767 heads, n_tokens * n_heads above 2^27, a
 * segment's k codes spanning 2 GiB, or a pointer / ld off the 16-byte rule;
 * DIT_EWORKSPACE for a missing or short workspace; DIT_EHIP on a launch
 * failure. */
dit_status attn_fp8_prepare(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                            const void* v, int64_t ld_v, const int32_t* cu_seqlens,
                            int32_t n_seqs, int32_t max_seqlen, int64_t n_tokens,
                            int32_t n_heads, int32_t head_dim, void* workspace,
                            size_t workspace_bytes, void* stream);

/* attn_packed_fp8: o bf16 [n_tokens][ld_o] (device) from the operands that
 * attn_fp8_prepare wrote for the same cu_seqlens, sizes and n_heads.
 * softmax_scale 0 means 1/sqrt(head_dim); causal as attn_packed.  Rows outside
 * every segment are not written.  Errors: those of attn_fp8_prepare (prefix
 * attn_packed_fp8), plus DIT_EINVAL for a null o, ld_o below
 * n_heads * head_dim or softmax_scale < 0. */
dit_status attn_packed_fp8(const void* workspace, size_t workspace_bytes, void* o, int64_t ld_o,
                           const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                           int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                           float softmax_scale, int32_t causal, void* stream);

/* ------------------------------------------------------------------------ */
/* The denoising step around the block                                        */
/* ------------------------------------------------------------------------ */

/* [vLLM-Omni] section 4, "Joint Audio-Video Denoising Execution Flow" (runtime
 * loop, stages 4-7): the DiT's packed output is split by modality into a video
 * and an audio velocity; the Rectified Flow parameterisation turns it into a
 * clean estimate X0; a deterministic Euler step (eta = 0) advances each
 * modality with its own schedule (sigma_video, sigma_audio), written back
 * together; anchor rows are then re-pinned to their original values.
 * [VeRL-Omni] section 5.1: H3's DiT takes data-progress time t = 1 - sigma
 * (sigma = 1 pure noise, 0 clean) and emits the negated velocity.
 *
 * denoise_step: for each row r of the packed latent state, with modality
 * m = modality[r]:
 *   m == VIDEO or AUDIO, anchor absent or anchor[r] == 0:
 *     v_std = velocity_sign * v[r];   (s, s') = the sigmas of modality m
 *     x0[r] = z[r] - s * v_std        (Rectified Flow: z = (1-s) x0 + s eps,
 *     z[r]  = z[r] + (s' - s) * v_std  v_std = eps - x0; Euler in sigma)
 *   m == VIDEO or AUDIO, anchor[r] != 0:  z[r] = x0[r] = anchor_vals[r]
 *   m == TEXT: nothing is read or written (text rows condition the DiT but
 *   are not latent state).
 * z: device float32 [n_rows][ld_z], updated in place; v: [n_rows][ld_v] of
 * v_dtype (bf16 or f32, the DiT's output head); x0: float32 [n_rows][ld_x0]
 * or NULL (not written); modality: device uint8 [n_rows] (the block's ids);
 * anchor: device uint8 [n_rows] or NULL (no anchors); anchor_vals: float32
 * [n_rows][ld_a], read on anchor rows only (required when anchor is given).
 * The first `channels` columns of each row are the state (96 = 24 latent
 * channels x the 1x2x2 patch of a video token, [H3-NFT]).  sigmas: host
 * float[4] = {sigma_video, sigma_video_next, sigma_audio, sigma_audio_next},
 * each in [0, 1]; the step is sigma_next - sigma in float32, exactly -sigma
 * when sigma_next is 0, so the last step leaves z == x0.  velocity_sign: +1
 * when v is eps - x0 (generic schedulers), -1 for H3's own output.
 * x0 must not overlap z, v or anchor_vals; z must not overlap v.
 * Errors: DIT_EINVAL for a null z / v / modality / sigmas, anchor without
 * anchor_vals, channels < 1, an ld below channels, n_rows < 0, a sigma that
 * is not finite or outside [0, 1], velocity_sign not +-1, an unknown dtype;
 * DIT_EUNSUPPORTED when channels is not a multiple of 4, n_rows * channels / 4
 * exceeds 2^31 - 1, or a pointer or ld breaks the 16-byte rule; DIT_EHIP on
 * a launch failure. */
dit_status denoise_step(dit_dtype v_dtype, float* z, int64_t ld_z, const void* v, int64_t ld_v,
                        float* x0, int64_t ld_x0, const uint8_t* modality,
                        const uint8_t* anchor, const float* anchor_vals, int64_t ld_a,
                        int64_t n_rows, int32_t channels, const float sigmas[4],
                        int32_t velocity_sign, void* stream);

/* ------------------------------------------------------------------------ */
/* The DiffusionNFT loss on the block's velocity output                       */
/* ------------------------------------------------------------------------ */

/* [VeRL-Omni] section 4 (DiffusionNFT with a scalar optimality reward): the
 * current policy's velocity v_theta and the frozen old adapter's v_old define
 * v_pos = beta v_theta + (1 - beta) v_old and v_neg = (1 + beta) v_old -
 * beta v_theta; a sample with reward r in [0, 1] has the loss
 * L = r MSE(v_pos, v_target) + (1 - r) MSE(v_neg, v_target).  [H3-NFT]
 * section "FL2VA: First-Frame Conditioning With Shared Infrastructure":
 * condition-frame latents are masked out of the loss.  [VeRL-Omni] section
 * 5.1: H3's velocity is sign-reversed (velocity_sign = -1 converts it).
 *
 * nft_loss: samples are row ranges [cu_samples[s], cu_samples[s+1]) of a
 * packed batch (device int32 [n_samples + 1], the cu_seqlens contract, every
 * range at most max_rows long).  For each sample, MSE is the mean over the
 * rows whose loss_mask flag is non-zero (all rows when loss_mask is NULL),
 * every one of their `channels` columns.  loss_out (device float32
 * [n_samples][3]) receives (L_s, MSE(v_pos), MSE(v_neg)); a sample with no
 * loss-bearing row gets zeros.  grad (device float32 [n_rows][ld_g], or NULL
 * for the loss alone) receives d(grad_scale * sum_s L_s)/d v_theta for every
 * row of every sample (zero on masked rows), with respect to the raw output
 * (so it carries velocity_sign); grad_scale = 1/n_samples is the mean over
 * samples.  v_theta, v_old: [n_rows][ld] of v_dtype (bf16 or f32); v_target:
 * float32 [n_rows][ld_t] in the standard convention (eps - x0); reward:
 * device float32 [n_samples]; beta, grad_scale: host.  grad must not overlap
 * the inputs.  Accumulation: per 32-row chunk in float32, across chunks in
 * float64, in a fixed order (deterministic, no atomics).
 * workspace: device, at least dit_nft_workspace_bytes(n_samples, max_rows)
 * bytes, 256-byte aligned.  Three launches on stream; with n_rows == 0 they
 * still write zero losses (the outputs are per sample).
 * Errors: DIT_EINVAL for a null required pointer, n_samples < 1, max_rows < 1
 * with n_rows > 0, channels < 1, an ld below channels, non-finite beta or
 * grad_scale, velocity_sign not +-1, an unknown dtype; DIT_EUNSUPPORTED when
 * channels is not a multiple of 4, n_samples > 65535, or a pointer or ld
 * breaks the 16-byte rule; DIT_EWORKSPACE; DIT_EHIP on a launch failure. */
size_t dit_nft_workspace_bytes(int32_t n_samples, int32_t max_rows);
dit_status nft_loss(dit_dtype v_dtype, const void* v_theta, int64_t ld_vt, const void* v_old,
                    int64_t ld_vo, const float* v_target, int64_t ld_t, const uint8_t* loss_mask,
                    const int32_t* cu_samples, int32_t n_samples, int32_t max_rows,
                    int64_t n_rows, int32_t channels, const float* reward, float beta,
                    int32_t velocity_sign, float grad_scale, float* grad, int64_t ld_g,
                    float* loss_out, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* The whole attention half of the block                                      */
/* ------------------------------------------------------------------------ */

typedef struct {
  dit_dtype dtype;
  int32_t d_model, n_heads, head_dim;
  int32_t rope_sections[3];   /* t, h, w; even, summing to head_dim */
  float rope_theta;           /* 10000 */
  float ln_eps;               /* 1e-6 */
  float softmax_scale;        /* 0 => 1/sqrt(head_dim) */
  int32_t causal;             /* 0: bidirectional inside each segment */
} dit_block_desc;

/* Bytes of scratch dit_block_forward needs: five [N][D] planes y, q', k', v,
 * o (q', k', v are the fused projection's output split by column, q and k
 * rotated), each rounded up to 256 bytes.  0 for a bad descriptor. */
size_t dit_block_workspace_bytes(const dit_block_desc* d, int64_t n_tokens);

/* x, out: [n_tokens][d_model] contiguous (out may equal x); modality, pos_thw,
 * cu_seqlens as above (device); ada_table f32 [3][3][d_model]; w_qkv
 * [3D][D]; w_o [D][D]; biases nullable; workspace: device, at least
 * dit_block_workspace_bytes() bytes, 256-byte aligned.  Enqueues the stages
 * of adaln_modulate -> qkv_project -> rope3d_apply -> attn_packed ->
 * out_proj_gated on stream; in bf16 the rotation of q and k is applied by the
 * QKV projection as it stores them (the same rotation with float32 angles
 * and sines, one bf16 rounding of q' and k' instead of two).  On completion the workspace holds the block's
 * intermediates (dit_block_intermediates).  Errors: those of the stages, plus
 * DIT_EWORKSPACE. */
dit_status dit_block_forward(const dit_block_desc* d, const void* x, void* out,
                             const uint8_t* modality, const int32_t* pos_thw,
                             const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                             int64_t n_tokens, const float* ada_table,
                             const void* w_qkv, const void* b_qkv,
                             const void* w_o, const void* b_o,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Where dit_block_forward leaves its intermediates in the workspace: byte
 * offsets[0..4] of y (the AdaLN output), q' (the rotated queries), k' (the
 * rotated keys), v and o (the attention output before to_out.0), each
 * [n_tokens][d_model] of the block's dtype with leading dimension d_model,
 * valid once the call has completed on its stream and until the workspace is
 * reused.  Host-only.  DIT_EINVAL for a null pointer, a bad descriptor or
 * n_tokens < 0. */
dit_status dit_block_intermediates(const dit_block_desc* d, int64_t n_tokens,
                                   int64_t offsets[5]);

/* ------------------------------------------------------------------------ */
/* Backward pass of the attention half                                        */
/* ------------------------------------------------------------------------ */

/* The gradients of sum(dout * out) for out = dit_block_forward(x): the chain
 * rule through the gated residual, the output projection, attention, the 3D
 * rotation (its transpose is the rotation by the negated angle), the fused
 * QKV projection and the per-modality AdaLN (the pages print no backward
 * pass; the DiffusionNFT objective of [H3-NFT] section "DiffusionNFT:
 * Skipping the Reverse Chain Entirely" trains the DiT through it).  The
 * forward stages are recomputed inside the call (nothing is saved between
 * calls).  bf16, head_dim 128, d_model a multiple of 64. */

/* Bytes of scratch dit_block_backward needs: about 12 bf16 planes of
 * [n_tokens rounded up to 64][d_model], plus 2 * n_heads * n_tokens floats,
 * 3 * d_model^2 bf16 and small reduction buffers.  0 for a bad descriptor
 * (also for a dtype other than DIT_BF16). */
size_t dit_block_backward_workspace_bytes(const dit_block_desc* d, int64_t n_tokens);

/* Inputs as dit_block_forward, plus dout = dL/d(out) [n_tokens][d_model] bf16.
 * Outputs (device): dx [n_tokens][d_model] bf16 (may be dout, must not
 * overlap x); dtable float32 [3][3][d_model] (the shift, scale and gate rows
 * of every modality; modalities absent from the pack get zero rows);
 * dw_qkv [3D][D] and dw_o [D][D] bf16 ([out][in], as the weights); db_qkv
 * [3D] and db_o [D] float32, or NULL to skip them.  Sums over tokens are
 * deterministic (fixed chunks, fixed order), accumulation float32.  Errors:
 * those of the forward's stages, DIT_EINVAL for a null required pointer or
 * dx overlapping x, DIT_EUNSUPPORTED for a dtype other than DIT_BF16,
 * d_model not a multiple of 64 or a misaligned pointer, DIT_EWORKSPACE. */
dit_status dit_block_backward(const dit_block_desc* d, const void* x, const void* dout,
                              const uint8_t* modality, const int32_t* pos_thw,
                              const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                              int64_t n_tokens, const float* ada_table, const void* w_qkv,
                              const void* b_qkv, const void* w_o, const void* b_o, void* dx,
                              float* dtable, void* dw_qkv, float* db_qkv, void* dw_o,
                              float* db_o, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Backward pass of the feed-forward half (dit_ffn_forward): the gradients of
 * sum(dout * out) through the gated residual, ff.net.2, the tanh-form GELU,
 * ff.net.0.proj and the AdaLN with the MLP table rows; the forward is
 * recomputed inside the call.  bf16; d_model and d_ff multiples of 64. */

/* Bytes of scratch dit_ffn_backward needs: about 5 bf16 [N][d_model] and 5
 * [N][d_ff] planes (N rounded up to 64), d_ff * d_model bf16 and small
 * buffers.  0 for a bad descriptor (also a dtype other than DIT_BF16). */
size_t dit_ffn_backward_workspace_bytes(const dit_ffn_desc* d, int64_t n_tokens);

/* Inputs as dit_ffn_forward plus dout [n_tokens][d_model] bf16.  Outputs
 * (device): dx bf16 (may be dout, must not overlap x); dtable float32
 * [3][3][d_model] (the MLP shift, scale and gate rows); dw1 [d_ff][d_model]
 * and dw2 [d_model][d_ff] bf16; db1 [d_ff], db2 [d_model] float32 or NULL.
 * Deterministic.  Errors as dit_block_backward. */
dit_status dit_ffn_backward(const dit_ffn_desc* d, const void* x, const void* dout,
                            const uint8_t* modality, int64_t n_tokens, const float* ada_table,
                            const void* w1, const void* b1, const void* w2, const void* b2,
                            void* dx, float* dtable, void* dw1, float* db1, void* dw2,
                            float* db2, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* FP8 block halves                                                           */
/* ------------------------------------------------------------------------ */

/* The attention and feed-forward halves with their projections in FP8
 * ([vLLM-Omni] section 5: the active layers run in FP8), with the
 * quantization rule of the FP8 projections: each projection's operand (the
 * AdaLN output, the attention output, the activated hidden state) is
 * quantized per row, weights come as e4m3 codes [out][in] contiguous with
 * float32 scales [out] (device, 16-byte aligned).  Activations, q, k, v,
 * attention and the output stay bf16 (d->dtype must be DIT_BF16, else
 * DIT_EUNSUPPORTED); widths must be multiples of 128. */

/* Bytes of scratch dit_block_forward_fp8 needs: five bf16 [N][D] planes and
 * N float32 row scales, each region rounded up to 256 bytes.  0 for a bad
 * descriptor (also for a dtype other than DIT_BF16). */
size_t dit_block_fp8_workspace_bytes(const dit_block_desc* d, int64_t n_tokens);

/* As dit_block_forward, with w_qkv codes [3D][D] and w_qkv_scales [3D],
 * w_o codes [D][D] and w_o_scales [D].  Enqueues adaln_modulate_fp8 ->
 * linear_fp8 (QKV, split into planes) -> rope3d_apply_to -> attn_packed ->
 * quantize_rows_fp8 -> linear_fp8 (gated) on stream, after validating all.
 * Errors: those of the stages, plus DIT_EWORKSPACE. */
dit_status dit_block_forward_fp8(const dit_block_desc* d, const void* x, void* out,
                                 const uint8_t* modality, const int32_t* pos_thw,
                                 const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                                 int64_t n_tokens, const float* ada_table, const uint8_t* w_qkv,
                                 const float* w_qkv_scales, const void* b_qkv,
                                 const uint8_t* w_o, const float* w_o_scales, const void* b_o,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of scratch dit_block_forward_fp8_attn needs: that of
 * dit_block_forward_fp8, then the FP8 attention operands
 * (dit_attn_fp8_workspace_bytes for n_tokens, n_seqs and the descriptor's
 * heads).  0 for a bad descriptor, n_seqs < 1 or head_dim != 128. */
size_t dit_block_fp8_attn_workspace_bytes(const dit_block_desc* d, int64_t n_tokens,
                                          int32_t n_seqs);

/* dit_block_forward_fp8 with the attention in FP8 as well: its attention
 * stage is attn_fp8_prepare + attn_packed_fp8 (operands in the workspace past
 * the block's own planes) instead of attn_packed.  Arguments as
 * dit_block_forward_fp8; errors those of its stages, plus DIT_EWORKSPACE. */
dit_status dit_block_forward_fp8_attn(const dit_block_desc* d, const void* x, void* out,
                                      const uint8_t* modality, const int32_t* pos_thw,
                                      const int32_t* cu_seqlens, int32_t n_seqs,
                                      int32_t max_seqlen, int64_t n_tokens,
                                      const float* ada_table, const uint8_t* w_qkv,
                                      const float* w_qkv_scales, const void* b_qkv,
                                      const uint8_t* w_o, const float* w_o_scales,
                                      const void* b_o, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* Bytes of scratch dit_ffn_forward_fp8 needs: codes [N][max(d_ff, d_model)]
 * bytes, h bf16 [N][d_ff] and N float32 row scales, each region rounded up to
 * 256 bytes.  0 for a bad descriptor (also for a dtype other than DIT_BF16). */
size_t dit_ffn_fp8_workspace_bytes(const dit_ffn_desc* d, int64_t n_tokens);

/* As dit_ffn_forward, with w1 codes [d_ff][d_model] and w1_scales [d_ff], w2
 * codes [d_model][d_ff] and w2_scales [d_model]; d_ff at most 20480.
 * Enqueues adaln_modulate_fp8 -> linear_fp8 (GELU) -> quantize_rows_fp8 ->
 * linear_fp8 (gated) on stream.  Errors: those of the stages, plus
 * DIT_EWORKSPACE. */
dit_status dit_ffn_forward_fp8(const dit_ffn_desc* d, const void* x, void* out,
                               const uint8_t* modality, int64_t n_tokens, const float* ada_table,
                               const uint8_t* w1, const float* w1_scales, const void* b1,
                               const uint8_t* w2, const float* w2_scales, const void* b2,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Optional stage timing of dit_block_forward (measurement plumbing)         */
/* ------------------------------------------------------------------------ */

enum { DIT_STAGE_ADALN = 0, DIT_STAGE_QKV = 1, DIT_STAGE_ROPE = 2,
       DIT_STAGE_ATTN = 3, DIT_STAGE_OUT = 4, DIT_NUM_STAGES = 5 };

/* max_calls > 0: create HIP events for that many subsequent dit_block_forward
 * calls (process-wide; each call records DIT_NUM_STAGES + 1 events on its
 * stream).  max_calls == 0: stop recording and destroy the events. */
dit_status dit_profile_enable(int32_t max_calls);

/* Wait for the recorded events and write, per stage, the summed milliseconds
 * over the *n_calls recorded calls into stage_ms[DIT_NUM_STAGES]; then reset
 * the record (events are kept for reuse). */
dit_status dit_profile_read(float* stage_ms, int32_t* n_calls);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H */
