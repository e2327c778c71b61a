// Host-side token arithmetic and packing (integer, bit-exact).
//
// [H3-NFT] section "MiniMax H3 and Why Joint Audio-Video Generation Complicates
// RL Training" fixes the factors: 16x spatial and 4x (causal) temporal video
// VAE, a 1x2x2 patchify (32x spatial in total), and 40 audio latent tokens per
// second per channel of 32 kHz stereo (800 samples per token).
// [vLLM-Omni] section 3 "Packed Sequences and Modality Identity Preservation":
// per-row modality tag and (t, h, w) position, one packed 1-D sequence, and
// cu_seqlens holding cumulative segment offsets; its section 1 table orders a
// request as video latents, audio latents, text.
#include <climits>
#include <cstdint>

#include "dit.h"
#include "errors.h"

namespace {
constexpr int kSpatial = 32;        // 16 (VAE) * 2 (patch)
constexpr int kTemporal = 4;
constexpr int kSamplesPerToken = 800;  // 32000 Hz / 40 Hz
constexpr int kChannels = 2;
}  // namespace

extern "C" dit_status dit_grid_from_media(const dit_media* m, dit_grid* g) {
  dit::clear_error();
  if (!m || !g) return dit::fail(DIT_EINVAL, "dit_grid_from_media: null pointer");
  if (m->frames < 0 || m->height_px < 0 || m->width_px < 0 || m->audio_samples_per_ch < 0 ||
      m->text_len < 0)
    return dit::fail(DIT_EINVAL, "dit_grid_from_media: negative count");
  int32_t t = 0;
  if (m->frames > 0) {
    if ((m->frames - 1) % kTemporal != 0)
      return dit::fail(DIT_EINVAL, "dit_grid_from_media: frames - 1 = %d is not a multiple of 4",
                       m->frames - 1);
    t = 1 + (m->frames - 1) / kTemporal;
  }
  if (m->height_px % kSpatial != 0 || m->width_px % kSpatial != 0)
    return dit::fail(DIT_EINVAL, "dit_grid_from_media: %dx%d px is not a multiple of 32",
                     m->height_px, m->width_px);
  if (m->audio_samples_per_ch % kSamplesPerToken != 0)
    return dit::fail(DIT_EINVAL, "dit_grid_from_media: %lld samples is not a multiple of 800",
                     (long long)m->audio_samples_per_ch);
  int64_t a = m->audio_samples_per_ch / kSamplesPerToken;
  if (a > INT32_MAX) return dit::fail(DIT_EINVAL, "dit_grid_from_media: audio too long");
  int32_t h = m->height_px / kSpatial, w = m->width_px / kSpatial;
  if (t == 0 || h == 0 || w == 0) t = h = w = 0;
  g->t = t;
  g->h = h;
  g->w = w;
  g->audio_per_ch = (int32_t)a;
  g->text_len = m->text_len;
  return DIT_OK;
}

namespace {
// Token count of the pack and its longest request; nothing is written on
// failure.  One request holds t*h*w video + 2*audio_per_ch audio + text_len
// text tokens.
dit_status count_pack(const char* who, const dit_grid* reqs, int32_t n_reqs, int64_t* total_out,
                      int32_t* longest_out) {
  if (n_reqs < 1) return dit::fail(DIT_EINVAL, "%s: n_reqs < 1", who);
  int64_t total = 0, longest = 0;
  for (int32_t r = 0; r < n_reqs; ++r) {
    const dit_grid& g = reqs[r];
    if (g.t < 0 || g.h < 0 || g.w < 0 || g.audio_per_ch < 0 || g.text_len < 0)
      return dit::fail(DIT_EINVAL, "%s: negative grid entry in request %d", who, r);
    const int64_t len = (int64_t)g.t * g.h * g.w + (int64_t)kChannels * g.audio_per_ch + g.text_len;
    total += len;
    if (len > longest) longest = len;
    if (total > INT32_MAX) return dit::fail(DIT_EINVAL, "%s: more than 2^31-1 tokens", who);
  }
  *total_out = total;
  *longest_out = (int32_t)longest;
  return DIT_OK;
}
}  // namespace

extern "C" dit_status dit_pack_count(const dit_grid* reqs, int32_t n_reqs, int64_t* n_tokens,
                                     int32_t* max_seqlen) {
  dit::clear_error();
  if (!reqs || !n_tokens || !max_seqlen) return dit::fail(DIT_EINVAL, "dit_pack_count: null pointer");
  return count_pack("dit_pack_count", reqs, n_reqs, n_tokens, max_seqlen);
}

extern "C" dit_status dit_pack_layout(const dit_grid* reqs, int32_t n_reqs, uint8_t* modality,
                                      int32_t* pos_thw, int32_t* cu_seqlens,
                                      int64_t capacity_tokens, int64_t* n_tokens,
                                      int32_t* max_seqlen) {
  dit::clear_error();
  if (!reqs || !modality || !pos_thw || !cu_seqlens || !n_tokens || !max_seqlen)
    return dit::fail(DIT_EINVAL, "dit_pack_layout: null pointer");
  // Size check first, so nothing is written on failure.
  int64_t total = 0;
  int32_t longest_len = 0;
  if (dit_status st = count_pack("dit_pack_layout", reqs, n_reqs, &total, &longest_len)) return st;
  if (total > capacity_tokens)
    return dit::fail(DIT_EINVAL, "dit_pack_layout: %lld tokens exceed capacity %lld",
                     (long long)total, (long long)capacity_tokens);
  int64_t i = 0;
  int32_t longest = 0;
  cu_seqlens[0] = 0;
  auto put = [&](uint8_t m, int32_t t, int32_t h, int32_t w) {
    modality[i] = m;
    pos_thw[3 * i + 0] = t;
    pos_thw[3 * i + 1] = h;
    pos_thw[3 * i + 2] = w;
    ++i;
  };
  for (int32_t r = 0; r < n_reqs; ++r) {
    const dit_grid& g = reqs[r];
    const int64_t start = i;
    for (int32_t t = 0; t < g.t; ++t)
      for (int32_t h = 0; h < g.h; ++h)
        for (int32_t w = 0; w < g.w; ++w) put(DIT_MOD_VIDEO, t, h, w);
    for (int c = 0; c < kChannels; ++c)
      for (int32_t k = 0; k < g.audio_per_ch; ++k) put(DIT_MOD_AUDIO, k, 0, 0);
    for (int32_t j = 0; j < g.text_len; ++j) put(DIT_MOD_TEXT, j, 0, 0);
    cu_seqlens[r + 1] = (int32_t)i;
    const int32_t len = (int32_t)(i - start);
    if (len > longest) longest = len;
  }
  *n_tokens = i;
  *max_seqlen = longest;
  return DIT_OK;
}
