// C ABI shell of libdit: argument validation, error text, workspace carving,
// stage dispatch and optional stage timing.  All compute runs in the HIP
// kernels of this directory; nothing here touches tensor data.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"
#include "dit.h"
#include "errors.h"

namespace dit {

char* error_buffer() {
  static thread_local char buf[512] = {0};
  return buf;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

size_t elt_size(dit_dtype dt) { return dt == DIT_BF16 ? 2 : 4; }

bool dtype_ok(dit_dtype dt) { return dt == DIT_BF16 || dt == DIT_F32; }

// ld counts elements; rows must start on 16-byte boundaries.
bool ld_aligned(dit_dtype dt, int64_t ld) { return (ld * (int64_t)elt_size(dt)) % 16 == 0; }

dit_status hip_fail(hipError_t e, const char* what) {
  return fail(DIT_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- optional stage timing ----
struct Profiler {
  std::mutex mu;
  int max_calls = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;   // max_calls * (DIT_NUM_STAGES + 1)
};
Profiler& prof() {
  static Profiler p;
  return p;
}

// Returns the event array for one call, or nullptr when not recording.
hipEvent_t* prof_slot() {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (p.max_calls == 0 || p.used >= p.max_calls) return nullptr;
  return &p.ev[(size_t)(p.used++) * (DIT_NUM_STAGES + 1)];
}

dit_status check_stream_rows(int64_t n_tokens) {
  if (n_tokens < 0) return fail(DIT_EINVAL, "n_tokens < 0");
  if (n_tokens > INT32_MAX) return fail(DIT_EUNSUPPORTED, "n_tokens above 2^31-1");
  return DIT_OK;
}

// DIT_VALIDATE=1 in the environment: before enqueuing, copy the device arrays
// the kernels take on trust (cu_seqlens, modality ids) to the host on the
// call's stream, synchronously, and check them.  Off by default: the checks
// stall the stream.
bool validate_on() {
  const char* v = std::getenv("DIT_VALIDATE");
  return v != nullptr && v[0] == '1';
}

dit_status validate_segments(const char* who, const int32_t* cu, int32_t n_seqs,
                             int32_t max_seqlen, int64_t n_tokens, void* stream) {
  std::vector<int32_t> h((size_t)n_seqs + 1);
  hipError_t e = hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                                (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, who);
  if (h[0] != 0) return fail(DIT_EINVAL, "%s: cu_seqlens[0] = %d, not 0", who, h[0]);
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (h[i + 1] < h[i])
      return fail(DIT_EINVAL, "%s: cu_seqlens decreases at %d (%d -> %d)", who, i, h[i], h[i + 1]);
    if (h[i + 1] - h[i] > max_seqlen)
      return fail(DIT_EINVAL, "%s: segment %d has %d tokens, max_seqlen is %d", who, i,
                  h[i + 1] - h[i], max_seqlen);
  }
  if (h[n_seqs] != n_tokens)
    return fail(DIT_EINVAL, "%s: cu_seqlens ends at %d, n_tokens is %lld", who, h[n_seqs],
                (long long)n_tokens);
  return DIT_OK;
}

dit_status validate_modality(const char* who, const uint8_t* mod, int64_t n, void* stream) {
  std::vector<uint8_t> h((size_t)n);
  hipError_t e = hipMemcpyAsync(h.data(), mod, h.size(), hipMemcpyDeviceToHost,
                                (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, who);
  for (int64_t i = 0; i < n; ++i)
    if (h[(size_t)i] >= DIT_NUM_MOD)
      return fail(DIT_EINVAL, "%s: modality[%lld] = %d, not below 3", who, (long long)i,
                  (int)h[(size_t)i]);
  return DIT_OK;
}

// Rope frequencies theta^(-2j/s_a) for every pair of a head, in double.
void rope_freqs(const int32_t* sec, double theta, int head_dim, double* out) {
  int p = 0;
  for (int a = 0; a < 3; ++a)
    for (int j = 0; j < sec[a] / 2; ++j) out[p++] = std::pow(theta, -2.0 * j / (double)sec[a]);
  (void)head_dim;
}

}  // namespace
}  // namespace dit

using namespace dit;

extern "C" int dit_abi_version(void) { return DIT_ABI_VERSION; }

extern "C" const char* dit_last_error(void) { return error_buffer(); }

// ---------------------------------------------------------------------------

static dit_status adaln_check(dit_dtype dt, const void* x, int64_t ld_x, const uint8_t* modality,
                              const float* table, void* y, int64_t ld_y, int64_t n_tokens,
                              int32_t d_model, float eps) {
  if (!dtype_ok(dt)) return fail(DIT_EINVAL, "adaln_modulate: unknown dtype %d", (int)dt);
  if (!x || !modality || !table || !y) return fail(DIT_EINVAL, "adaln_modulate: null pointer");
  if (d_model < 1) return fail(DIT_EINVAL, "adaln_modulate: d_model < 1");
  if (ld_x < d_model || ld_y < d_model) return fail(DIT_EINVAL, "adaln_modulate: ld < d_model");
  if (!(eps > 0.0f)) return fail(DIT_EINVAL, "adaln_modulate: eps must be > 0");
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  const int per_vec = dt == DIT_BF16 ? 8 : 4;
  const int max_d = dt == DIT_BF16 ? 16384 : 8192;
  if (d_model % per_vec != 0 || d_model > max_d)
    return fail(DIT_EUNSUPPORTED, "adaln_modulate: d_model %d unsupported", d_model);
  if (!aligned16(x) || !aligned16(y) || !aligned16(table) || !ld_aligned(dt, ld_x) ||
      !ld_aligned(dt, ld_y))
    return fail(DIT_EUNSUPPORTED, "adaln_modulate: pointers/ld must be 16-byte aligned");
  return DIT_OK;
}

extern "C" dit_status adaln_modulate(dit_dtype dt, const void* x, int64_t ld_x,
                                     const uint8_t* modality, const float* table, void* y,
                                     int64_t ld_y, int64_t n_tokens, int32_t d_model, float eps,
                                     void* stream) {
  clear_error();
  if (dit_status st = adaln_check(dt, x, ld_x, modality, table, y, ld_y, n_tokens, d_model, eps))
    return st;
  if (n_tokens == 0) return DIT_OK;
  if (validate_on()) {
    if (dit_status st = validate_modality("adaln_modulate", modality, n_tokens, stream))
      return st;
  }
  hipError_t e = launch_adaln(dt == DIT_BF16, x, ld_x, modality, table, y, ld_y, n_tokens,
                              d_model, eps, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "adaln_modulate launch");
}

static dit_status adaln_fp8_check(dit_dtype dt, const void* x, int64_t ld_x,
                                  const uint8_t* modality, const float* table, const uint8_t* q,
                                  int64_t ld_q, const float* scales, int64_t n_tokens,
                                  int32_t d_model, float eps) {
  if (!dtype_ok(dt)) return fail(DIT_EINVAL, "adaln_modulate_fp8: unknown dtype %d", (int)dt);
  if (!x || !modality || !table || !q || !scales)
    return fail(DIT_EINVAL, "adaln_modulate_fp8: null pointer");
  if (d_model < 1) return fail(DIT_EINVAL, "adaln_modulate_fp8: d_model < 1");
  if (ld_x < d_model || ld_q < d_model)
    return fail(DIT_EINVAL, "adaln_modulate_fp8: ld < d_model");
  if (!(eps > 0.0f)) return fail(DIT_EINVAL, "adaln_modulate_fp8: eps must be > 0");
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  const int per_vec = dt == DIT_BF16 ? 8 : 4;
  const int max_d = dt == DIT_BF16 ? 16384 : 8192;
  if (d_model % per_vec != 0 || d_model > max_d)
    return fail(DIT_EUNSUPPORTED, "adaln_modulate_fp8: d_model %d unsupported", d_model);
  if (!aligned16(x) || !aligned16(table) || !aligned16(q) || !aligned16(scales) ||
      !ld_aligned(dt, ld_x) || ld_q % 16 != 0)
    return fail(DIT_EUNSUPPORTED, "adaln_modulate_fp8: pointers/ld must be 16-byte aligned");
  return DIT_OK;
}

extern "C" dit_status adaln_modulate_fp8(dit_dtype dt, const void* x, int64_t ld_x,
                                         const uint8_t* modality, const float* table, uint8_t* q,
                                         int64_t ld_q, float* scales, int64_t n_tokens,
                                         int32_t d_model, float eps, void* stream) {
  clear_error();
  if (dit_status st = adaln_fp8_check(dt, x, ld_x, modality, table, q, ld_q, scales, n_tokens,
                                      d_model, eps))
    return st;
  if (n_tokens == 0) return DIT_OK;
  if (validate_on()) {
    if (dit_status st = validate_modality("adaln_modulate_fp8", modality, n_tokens, stream))
      return st;
  }
  hipError_t e = launch_adaln_fp8(dt == DIT_BF16, x, ld_x, modality, table, q, ld_q, scales,
                                  n_tokens, d_model, eps, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "adaln_modulate_fp8 launch");
}

// ---------------------------------------------------------------------------

static dit_status rope_check(dit_dtype dt, void* q, int64_t ld_q, void* k, int64_t ld_k,
                             const int32_t* pos, int64_t n_tokens, int32_t n_heads,
                             int32_t head_dim, const int32_t* sec, float theta) {
  if (!dtype_ok(dt)) return fail(DIT_EINVAL, "rope3d_apply: unknown dtype %d", (int)dt);
  if (!q || !pos || !sec) return fail(DIT_EINVAL, "rope3d_apply: null pointer");
  if (n_heads < 1 || head_dim < 1) return fail(DIT_EINVAL, "rope3d_apply: n_heads/head_dim < 1");
  for (int a = 0; a < 3; ++a)
    if (sec[a] < 0 || sec[a] % 2 != 0)
      return fail(DIT_EINVAL, "rope3d_apply: section %d = %d must be even and >= 0", a, sec[a]);
  if (sec[0] + sec[1] + sec[2] != head_dim)
    return fail(DIT_EINVAL, "rope3d_apply: sections sum to %d, head_dim is %d",
                sec[0] + sec[1] + sec[2], head_dim);
  if (!(theta > 0.0f)) return fail(DIT_EINVAL, "rope3d_apply: theta must be > 0");
  const int64_t width = (int64_t)n_heads * head_dim;
  if (ld_q < width || (k && ld_k < width)) return fail(DIT_EINVAL, "rope3d_apply: ld too small");
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  if (head_dim != 64 && head_dim != 128)
    return fail(DIT_EUNSUPPORTED, "rope3d_apply: head_dim %d (64 or 128 only)", head_dim);
  if (!aligned16(q) || !ld_aligned(dt, ld_q) || (k && (!aligned16(k) || !ld_aligned(dt, ld_k))))
    return fail(DIT_EUNSUPPORTED, "rope3d_apply: pointers/ld must be 16-byte aligned");
  return DIT_OK;
}

extern "C" dit_status rope3d_apply(dit_dtype dt, void* q, int64_t ld_q, void* k, int64_t ld_k,
                                   const int32_t* pos_thw, int64_t n_tokens, int32_t n_heads,
                                   int32_t head_dim, const int32_t sections[3], float theta,
                                   void* stream) {
  clear_error();
  if (dit_status st = rope_check(dt, q, ld_q, k, ld_k, pos_thw, n_tokens, n_heads, head_dim,
                                 sections, theta))
    return st;
  if (n_tokens == 0) return DIT_OK;
  double freq[64];
  rope_freqs(sections, (double)theta, head_dim, freq);
  hipError_t e = launch_rope(dt == DIT_BF16, q, ld_q, k, ld_k, q, ld_q, k, ld_k, pos_thw,
                             n_tokens, n_heads, head_dim, sections[0], sections[1], freq,
                             (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "rope3d_apply launch");
}

// Rows [p, p + n*ld) and [o, o + n*ld_o) in bytes overlap only if the spans do.
static bool spans_overlap(const void* a, int64_t lda, const void* b, int64_t ldb, int64_t n,
                          int64_t width, size_t es) {
  if (!a || !b || n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, a1 = a0 + ((n - 1) * lda + width) * es;
  const uintptr_t b0 = (uintptr_t)b, b1 = b0 + ((n - 1) * ldb + width) * es;
  return a0 < b1 && b0 < a1;
}

extern "C" dit_status rope3d_apply_to(dit_dtype dt, const void* q, int64_t ld_q, const void* k,
                                      int64_t ld_k, void* q_out, int64_t ld_qo, void* k_out,
                                      int64_t ld_ko, const int32_t* pos_thw, int64_t n_tokens,
                                      int32_t n_heads, int32_t head_dim,
                                      const int32_t sections[3], float theta, void* stream) {
  clear_error();
  if (dit_status st = rope_check(dt, const_cast<void*>(q), ld_q, const_cast<void*>(k), ld_k,
                                 pos_thw, n_tokens, n_heads, head_dim, sections, theta))
    return st;
  if (!q_out || (k && !k_out) || (!k && k_out))
    return fail(DIT_EINVAL, "rope3d_apply_to: an output is missing (or k_out without k)");
  const int64_t width = (int64_t)n_heads * head_dim;
  if (ld_qo < width || (k_out && ld_ko < width))
    return fail(DIT_EINVAL, "rope3d_apply_to: output ld too small");
  if (!aligned16(q_out) || !ld_aligned(dt, ld_qo) ||
      (k_out && (!aligned16(k_out) || !ld_aligned(dt, ld_ko))))
    return fail(DIT_EUNSUPPORTED, "rope3d_apply_to: pointers/ld must be 16-byte aligned");
  // An output may be its own input or the other input with the same rows and
  // ld; any other overlap is refused.
  const size_t es = elt_size(dt);
  auto same = [](const void* a, int64_t la, const void* b, int64_t lb) {
    return a == b && la == lb;
  };
  const void* ins[2] = {q, k};
  const int64_t ins_ld[2] = {ld_q, ld_k};
  void* outs[2] = {q_out, k_out};
  const int64_t outs_ld[2] = {ld_qo, ld_ko};
  for (int o = 0; o < 2; ++o)
    for (int i = 0; i < 2; ++i)
      if (outs[o] && ins[i] && !same(outs[o], outs_ld[o], ins[i], ins_ld[i]) &&
          spans_overlap(outs[o], outs_ld[o], ins[i], ins_ld[i], n_tokens, width, es))
        return fail(DIT_EINVAL, "rope3d_apply_to: an output partly overlaps an input");
  if (k_out && spans_overlap(q_out, ld_qo, k_out, ld_ko, n_tokens, width, es))
    return fail(DIT_EINVAL, "rope3d_apply_to: the outputs overlap");
  if (n_tokens == 0) return DIT_OK;
  double freq[64];
  rope_freqs(sections, (double)theta, head_dim, freq);
  hipError_t e = launch_rope(dt == DIT_BF16, q, ld_q, k, ld_k, q_out, ld_qo, k_out, ld_ko,
                             pos_thw, n_tokens, n_heads, head_dim, sections[0], sections[1],
                             freq, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "rope3d_apply_to launch");
}

// ---------------------------------------------------------------------------

static dit_status attn_check(dit_dtype dt, const void* q, int64_t ld_q, const void* k,
                             int64_t ld_k, const void* v, int64_t ld_v, void* o, int64_t ld_o,
                             const int32_t* cu, int32_t n_seqs, int32_t max_seqlen,
                             int64_t n_tokens, int32_t n_heads, int32_t head_dim, float scale) {
  if (!dtype_ok(dt)) return fail(DIT_EINVAL, "attn_packed: unknown dtype %d", (int)dt);
  if (!q || !k || !v || !o || !cu) return fail(DIT_EINVAL, "attn_packed: null pointer");
  if (n_seqs < 1) return fail(DIT_EINVAL, "attn_packed: n_seqs < 1");
  if (n_tokens > 0 && max_seqlen < 1) return fail(DIT_EINVAL, "attn_packed: max_seqlen < 1");
  if (n_heads < 1 || head_dim < 1) return fail(DIT_EINVAL, "attn_packed: n_heads/head_dim < 1");
  if (!(scale >= 0.0f)) return fail(DIT_EINVAL, "attn_packed: softmax_scale < 0");
  const int64_t width = (int64_t)n_heads * head_dim;
  if (ld_q < width || ld_k < width || ld_v < width || ld_o < width)
    return fail(DIT_EINVAL, "attn_packed: ld too small");
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  if (max_seqlen > n_tokens && n_tokens > 0)
    return fail(DIT_EINVAL, "attn_packed: max_seqlen %d > n_tokens", max_seqlen);
  if (n_seqs > 65535 || n_heads > 65535)
    return fail(DIT_EUNSUPPORTED, "attn_packed: more than 65535 segments or heads");
  if (dt == DIT_BF16 && (double)max_seqlen * (double)std::max(ld_k, ld_v) * 2.0 >= 4294967296.0)
    return fail(DIT_EUNSUPPORTED, "attn_packed: a segment's K or V rows span 4 GiB or more");
  if (dt == DIT_BF16 ? head_dim != 128 : (head_dim != 64 && head_dim != 128))
    return fail(DIT_EUNSUPPORTED, "attn_packed: head_dim %d unsupported for this dtype", head_dim);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !ld_aligned(dt, ld_q) ||
      !ld_aligned(dt, ld_k) || !ld_aligned(dt, ld_v) || !ld_aligned(dt, ld_o))
    return fail(DIT_EUNSUPPORTED, "attn_packed: pointers/ld must be 16-byte aligned");
  return DIT_OK;
}

extern "C" dit_status attn_packed(dit_dtype dt, const void* q, int64_t ld_q, const void* k,
                                  int64_t ld_k, const void* v, int64_t ld_v, void* o,
                                  int64_t ld_o, const int32_t* cu_seqlens, int32_t n_seqs,
                                  int32_t max_seqlen, int64_t n_tokens, int32_t n_heads,
                                  int32_t head_dim, float softmax_scale, int32_t causal,
                                  void* stream) {
  clear_error();
  if (dit_status st = attn_check(dt, q, ld_q, k, ld_k, v, ld_v, o, ld_o, cu_seqlens, n_seqs,
                                 max_seqlen, n_tokens, n_heads, head_dim, softmax_scale))
    return st;
  if (n_tokens == 0) return DIT_OK;
  if (validate_on()) {
    if (dit_status st = validate_segments("attn_packed", cu_seqlens, n_seqs, max_seqlen,
                                          n_tokens, stream))
      return st;
  }
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  hipError_t e = launch_attn(dt == DIT_BF16, q, ld_q, k, ld_k, v, ld_v, o, ld_o, cu_seqlens,
                             n_seqs, max_seqlen, n_tokens, n_heads, head_dim, scale,
                             causal != 0, nullptr, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "attn_packed launch");
}

extern "C" dit_status attn_packed_lse(dit_dtype dt, const void* q, int64_t ld_q, const void* k,
                                      int64_t ld_k, const void* v, int64_t ld_v, void* o,
                                      int64_t ld_o, float* lse, const int32_t* cu_seqlens,
                                      int32_t n_seqs, int32_t max_seqlen, int64_t n_tokens,
                                      int32_t n_heads, int32_t head_dim, float softmax_scale,
                                      int32_t causal, void* stream) {
  clear_error();
  if (dit_status st = attn_check(dt, q, ld_q, k, ld_k, v, ld_v, o, ld_o, cu_seqlens, n_seqs,
                                 max_seqlen, n_tokens, n_heads, head_dim, softmax_scale))
    return st;
  if (!lse) return fail(DIT_EINVAL, "attn_packed_lse: null lse");
  if (dt != DIT_BF16) return fail(DIT_EUNSUPPORTED, "attn_packed_lse: bf16 only");
  if (n_tokens == 0) return DIT_OK;
  if (validate_on()) {
    if (dit_status st = validate_segments("attn_packed_lse", cu_seqlens, n_seqs, max_seqlen,
                                          n_tokens, stream))
      return st;
  }
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  hipError_t e = launch_attn(1, q, ld_q, k, ld_k, v, ld_v, o, ld_o, cu_seqlens, n_seqs,
                             max_seqlen, n_tokens, n_heads, head_dim, scale, causal != 0, lse,
                             (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "attn_packed_lse launch");
}

extern "C" size_t dit_attn_backward_workspace_bytes(int64_t n_tokens, int32_t n_heads) {
  if (n_tokens < 0 || n_heads < 1) return 0;
  return round256((size_t)n_tokens * (size_t)n_heads * 4);
}

namespace {
// The checks and the launch of attn_packed_backward, with delta (n_heads *
// n_tokens floats) at `delta`, which holds `delta_bytes`.
dit_status attn_backward_impl(
    const char* who, dit_dtype dt, const void* q, int64_t ld_q, const void* k, int64_t ld_k,
    const void* v, int64_t ld_v, const void* o, int64_t ld_o, const void* dout, int64_t ld_do,
    const float* lse, void* dq, int64_t ld_dq, void* dk, int64_t ld_dk, void* dv, int64_t ld_dv,
    const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen, int64_t n_tokens,
    int32_t n_heads, int32_t head_dim, float softmax_scale, int32_t causal, float* delta,
    size_t delta_bytes, void* stream) {
  if (dit_status st = attn_check(dt, q, ld_q, k, ld_k, v, ld_v, const_cast<void*>(o), ld_o,
                                 cu_seqlens, n_seqs, max_seqlen, n_tokens, n_heads, head_dim,
                                 softmax_scale))
    return st;
  if (!dout || !lse || !dq || !dk || !dv) return fail(DIT_EINVAL, "%s: null pointer", who);
  if (dt != DIT_BF16) return fail(DIT_EUNSUPPORTED, "%s: bf16 only", who);
  const int64_t width = (int64_t)n_heads * head_dim;
  if (ld_do < width || ld_dq < width || ld_dk < width || ld_dv < width)
    return fail(DIT_EINVAL, "%s: ld too small", who);
  if ((double)max_seqlen * (double)std::max(ld_q, ld_do) * 2.0 >= 4294967296.0)
    return fail(DIT_EUNSUPPORTED, "%s: a segment's rows span 4 GiB or more", who);
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !ld_aligned(dt, ld_do) || !ld_aligned(dt, ld_dq) || !ld_aligned(dt, ld_dk) ||
      !ld_aligned(dt, ld_dv))
    return fail(DIT_EUNSUPPORTED, "%s: pointers/ld must be 16-byte aligned", who);
  const size_t need = dit_attn_backward_workspace_bytes(n_tokens, n_heads);
  if (!delta || delta_bytes < need)
    return fail(DIT_EWORKSPACE, "%s: workspace %zu bytes, need %zu", who, delta_bytes, need);
  if (n_tokens == 0) return DIT_OK;
  if (validate_on()) {
    if (dit_status st = validate_segments(who, cu_seqlens, n_seqs, max_seqlen, n_tokens, stream))
      return st;
  }
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  hipError_t e = launch_attn_bwd(q, ld_q, k, ld_k, v, ld_v, o, ld_o, dout, ld_do, lse, dq, ld_dq,
                                 dk, ld_dk, dv, ld_dv, cu_seqlens, n_seqs, max_seqlen, n_tokens,
                                 n_heads, scale, causal != 0, delta, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : fail(DIT_EHIP, "%s launch: %s", who, hipGetErrorString(e));
}
}  // namespace

extern "C" dit_status attn_packed_backward(
    dit_dtype dt, const void* q, int64_t ld_q, const void* k, int64_t ld_k, const void* v,
    int64_t ld_v, const void* o, int64_t ld_o, const void* dout, int64_t ld_do, const float* lse,
    void* dq, int64_t ld_dq, void* dk, int64_t ld_dk, void* dv, int64_t ld_dv,
    const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen, int64_t n_tokens,
    int32_t n_heads, int32_t head_dim, float softmax_scale, int32_t causal, void* workspace,
    size_t workspace_bytes, void* stream) {
  clear_error();
  return attn_backward_impl("attn_packed_backward", dt, q, ld_q, k, ld_k, v, ld_v, o, ld_o, dout,
                            ld_do, lse, dq, ld_dq, dk, ld_dk, dv, ld_dv, cu_seqlens, n_seqs,
                            max_seqlen, n_tokens, n_heads, head_dim, softmax_scale, causal,
                            static_cast<float*>(workspace), workspace ? workspace_bytes : 0,
                            stream);
}

// attn_packed_backward without a workspace argument: delta lives in a fixed
// file-scope device array (one copy per GPU, held until the process ends).
// In host code `scratch` names a host-side stand-in, never the device
// memory: its device address is looked up once per device with
// hipGetSymbolAddress (on the first call with that device current) and only
// that address is passed to the kernels.  Every call on a GPU shares that
// GPU's array; calls that overlap on one GPU race.  Every delta value a call
// reads it has first written, so nothing needs clearing between calls.
constexpr size_t kNoAllocScratchFloats = (size_t)4 << 20;   // 16 MiB
static __device__ __align__(256) float scratch[kNoAllocScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};

dit_status scratch_address(const char* who, float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DIT_EHIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DIT_EUNSUPPORTED, "%s: device %d", who, dev);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DIT_EHIP, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return DIT_OK;
}
}  // namespace

extern "C" size_t dit_attn_backward_noalloc_max_elements(void) { return kNoAllocScratchFloats; }

extern "C" dit_status attn_packed_backward_noalloc(
    dit_dtype dt, const void* q, int64_t ld_q, const void* k, int64_t ld_k, const void* v,
    int64_t ld_v, const void* o, int64_t ld_o, const void* dout, int64_t ld_do, const float* lse,
    void* dq, int64_t ld_dq, void* dk, int64_t ld_dk, void* dv, int64_t ld_dv,
    const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen, int64_t n_tokens,
    int32_t n_heads, int32_t head_dim, float softmax_scale, int32_t causal, void* stream) {
  clear_error();
  const char* who = "attn_packed_backward_noalloc";
  if (n_tokens < 0 || n_heads < 1) return fail(DIT_EINVAL, "%s: n_tokens or n_heads", who);
  if ((uint64_t)n_tokens * (uint64_t)n_heads > kNoAllocScratchFloats)
    return fail(DIT_EWORKSPACE,
                "%s: n_heads * n_tokens = %lld exceeds the fixed scratch of %zu values",
                who, (long long)n_tokens * n_heads, kNoAllocScratchFloats);
  float* delta = nullptr;
  if (dit_status st = scratch_address(who, &delta)) return st;
  return attn_backward_impl(who, dt, q, ld_q, k, ld_k, v, ld_v, o, ld_o, dout, ld_do, lse, dq,
                            ld_dq, dk, ld_dk, dv, ld_dv, cu_seqlens, n_seqs, max_seqlen, n_tokens,
                            n_heads, head_dim, softmax_scale, causal, delta,
                            kNoAllocScratchFloats * sizeof(float), stream);
}

// ---------------------------------------------------------------------------
// FP8 attention: operand preparation and the attention itself.

namespace {
struct Fp8AttnLayout {
  size_t q8, k8, vt, sq, sk, sv, amax, total;
  int64_t ld8, ld_vt;
};
Fp8AttnLayout fp8_attn_layout(int64_t n, int32_t n_seqs, int32_t h) {
  Fp8AttnLayout L{};
  L.ld8 = (int64_t)h * 128;
  L.ld_vt = (n + 63) / 64 * 64 + 128 * (int64_t)n_seqs;
  size_t off = 0;
  L.q8 = off;   off += round256((size_t)n * (size_t)L.ld8);
  L.k8 = off;   off += round256((size_t)n * (size_t)L.ld8);
  L.vt = off;   off += round256((size_t)h * 128 * (size_t)L.ld_vt);
  L.sq = off;   off += round256((size_t)h * (size_t)n * 4);
  L.sk = off;   off += round256((size_t)n_seqs * h * 4);     // [segment][head]
  L.sv = off;   off += round256((size_t)n_seqs * h * 4);
  L.amax = off; off += round256((size_t)n_seqs * h * 8);
  L.total = off;
  return L;
}
AttnFp8Ops fp8_attn_ops(void* ws, const Fp8AttnLayout& L) {
  char* b = static_cast<char*>(ws);
  AttnFp8Ops o;
  o.q8 = reinterpret_cast<uint8_t*>(b + L.q8);
  o.k8 = reinterpret_cast<uint8_t*>(b + L.k8);
  o.vt = reinterpret_cast<uint8_t*>(b + L.vt);
  o.sq = reinterpret_cast<float*>(b + L.sq);
  o.sk = reinterpret_cast<float*>(b + L.sk);
  o.sv = reinterpret_cast<float*>(b + L.sv);
  o.amax = reinterpret_cast<uint32_t*>(b + L.amax);
  o.ld8 = L.ld8;
  o.ld_vt = L.ld_vt;
  return o;
}
}  // namespace

extern "C" size_t dit_attn_fp8_workspace_bytes(int64_t n_tokens, int32_t n_seqs, int32_t n_heads,
                                               int32_t head_dim) {
  if (n_tokens < 0 || n_seqs < 1 || n_heads < 1 || head_dim != 128) return 0;
  return fp8_attn_layout(n_tokens, n_seqs, n_heads).total;
}

extern "C" dit_status dit_attn_fp8_layout(int64_t n_tokens, int32_t n_seqs, int32_t n_heads,
                                          int32_t head_dim, int64_t* out) {
  clear_error();
  if (!out) return fail(DIT_EINVAL, "dit_attn_fp8_layout: null out");
  if (n_tokens < 0 || n_seqs < 1 || n_heads < 1)
    return fail(DIT_EINVAL, "dit_attn_fp8_layout: bad sizes");
  if (head_dim != 128) return fail(DIT_EUNSUPPORTED, "dit_attn_fp8_layout: head_dim must be 128");
  const Fp8AttnLayout L = fp8_attn_layout(n_tokens, n_seqs, n_heads);
  const int64_t v[9] = {(int64_t)L.q8, (int64_t)L.k8, (int64_t)L.vt, (int64_t)L.sq, (int64_t)L.sk,
                        (int64_t)L.sv, (int64_t)L.amax, L.ld8, L.ld_vt};
  for (int i = 0; i < 9; ++i) out[i] = v[i];
  return DIT_OK;
}

static dit_status fp8_attn_check(const char* who, const int32_t* cu, int32_t n_seqs,
                                 int32_t max_seqlen, int64_t n_tokens, int32_t n_heads,
                                 int32_t head_dim, const void* workspace,
                                 size_t workspace_bytes) {
  if (!cu) return fail(DIT_EINVAL, "%s: null cu_seqlens", who);
  if (n_seqs < 1) return fail(DIT_EINVAL, "%s: n_seqs < 1", who);
  if (n_heads < 1) return fail(DIT_EINVAL, "%s: n_heads < 1", who);
  if (head_dim != 128) return fail(DIT_EUNSUPPORTED, "%s: head_dim must be 128", who);
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  if (n_tokens > 0 && max_seqlen < 1) return fail(DIT_EINVAL, "%s: max_seqlen < 1", who);
  if (max_seqlen > n_tokens && n_tokens > 0)
    return fail(DIT_EINVAL, "%s: max_seqlen %d > n_tokens", who, max_seqlen);
  if (n_seqs > 65535 || n_heads > 32767)
    return fail(DIT_EUNSUPPORTED, "%s: more than 65535 segments or 32767 heads", who);
  if ((double)n_tokens * (double)n_heads * 16.0 > 2147483647.0)
    return fail(DIT_EUNSUPPORTED, "%s: n_tokens * n_heads too large", who);
  if ((double)max_seqlen * (double)n_heads * 128.0 >= 2147483648.0)
    return fail(DIT_EUNSUPPORTED, "%s: a segment's K codes span 2 GiB or more", who);
  const size_t need = fp8_attn_layout(n_tokens, n_seqs, n_heads).total;
  if (!workspace || workspace_bytes < need)
    return fail(DIT_EWORKSPACE, "%s: workspace %zu bytes, need %zu", who, workspace_bytes, need);
  if (!aligned16(workspace)) return fail(DIT_EUNSUPPORTED, "%s: workspace must be 16-byte aligned", who);
  return DIT_OK;
}

extern "C" dit_status attn_fp8_prepare(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                                       const void* v, int64_t ld_v, const int32_t* cu_seqlens,
                                       int32_t n_seqs, int32_t max_seqlen, int64_t n_tokens,
                                       int32_t n_heads, int32_t head_dim, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  clear_error();
  const char* who = "attn_fp8_prepare";
  if (!q || !k || !v) return fail(DIT_EINVAL, "%s: null pointer", who);
  if (dit_status st = fp8_attn_check(who, cu_seqlens, n_seqs, max_seqlen, n_tokens, n_heads,
                                     head_dim, workspace, workspace_bytes))
    return st;
  const int64_t width = (int64_t)n_heads * head_dim;
  if (ld_q < width || ld_k < width || ld_v < width) return fail(DIT_EINVAL, "%s: ld too small", who);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !ld_aligned(DIT_BF16, ld_q) ||
      !ld_aligned(DIT_BF16, ld_k) || !ld_aligned(DIT_BF16, ld_v))
    return fail(DIT_EUNSUPPORTED, "%s: pointers/ld must be 16-byte aligned", who);
  if (n_tokens == 0) return DIT_OK;
  if (validate_on()) {
    if (dit_status st = validate_segments(who, cu_seqlens, n_seqs, max_seqlen, n_tokens, stream))
      return st;
  }
  const Fp8AttnLayout L = fp8_attn_layout(n_tokens, n_seqs, n_heads);
  hipError_t e = launch_attn_fp8_prepare(
      static_cast<const uint16_t*>(q), ld_q, static_cast<const uint16_t*>(k), ld_k,
      static_cast<const uint16_t*>(v), ld_v, cu_seqlens, n_seqs, max_seqlen, n_tokens, n_heads,
      fp8_attn_ops(workspace, L), (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "attn_fp8_prepare launch");
}

extern "C" dit_status attn_packed_fp8(const void* workspace, size_t workspace_bytes, void* o,
                                      int64_t ld_o, const int32_t* cu_seqlens, int32_t n_seqs,
                                      int32_t max_seqlen, int64_t n_tokens, int32_t n_heads,
                                      int32_t head_dim, float softmax_scale, int32_t causal,
                                      void* stream) {
  clear_error();
  const char* who = "attn_packed_fp8";
  if (!o) return fail(DIT_EINVAL, "%s: null o", who);
  if (dit_status st = fp8_attn_check(who, cu_seqlens, n_seqs, max_seqlen, n_tokens, n_heads,
                                     head_dim, workspace, workspace_bytes))
    return st;
  if (!(softmax_scale >= 0.0f)) return fail(DIT_EINVAL, "%s: softmax_scale < 0", who);
  if (ld_o < (int64_t)n_heads * head_dim) return fail(DIT_EINVAL, "%s: ld_o too small", who);
  if (!aligned16(o) || !ld_aligned(DIT_BF16, ld_o))
    return fail(DIT_EUNSUPPORTED, "%s: o/ld_o must be 16-byte aligned", who);
  if (n_tokens == 0) return DIT_OK;
  if (validate_on()) {
    if (dit_status st = validate_segments(who, cu_seqlens, n_seqs, max_seqlen, n_tokens, stream))
      return st;
  }
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  const Fp8AttnLayout L = fp8_attn_layout(n_tokens, n_seqs, n_heads);
  AttnFp8Ops ops = fp8_attn_ops(const_cast<void*>(workspace), L);
  hipError_t e = launch_attn_fp8(ops, static_cast<uint16_t*>(o), ld_o, cu_seqlens, n_seqs,
                                 max_seqlen, n_tokens, n_heads, scale, causal != 0,
                                 (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "attn_packed_fp8 launch");
}

// ---------------------------------------------------------------------------

// C [n_tokens][width_out] = A [n_tokens][k_in] W^T: inner width k_in (a
// multiple of the 64-deep k-step), output width a multiple of 4 (the
// epilogue stores four features at a time).
static dit_status proj_check(const char* who, dit_dtype dt, const void* a, int64_t lda,
                             const void* w, void* c, int64_t ldc, int64_t n_tokens,
                             int32_t k_in, int64_t width_out) {
  if (!dtype_ok(dt)) return fail(DIT_EINVAL, "%s: unknown dtype %d", who, (int)dt);
  if (!a || !w || !c) return fail(DIT_EINVAL, "%s: null pointer", who);
  if (k_in < 1 || width_out < 1) return fail(DIT_EINVAL, "%s: width < 1", who);
  if (lda < k_in || ldc < width_out) return fail(DIT_EINVAL, "%s: ld too small", who);
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  if (k_in % 64 != 0 || width_out % 4 != 0 || width_out > INT32_MAX)
    return fail(DIT_EUNSUPPORTED, "%s: inner width %d must be a multiple of 64, output width "
                "%lld of 4", who, k_in, (long long)width_out);
  if (!aligned16(a) || !aligned16(w) || !aligned16(c) || !ld_aligned(dt, lda) ||
      !ld_aligned(dt, ldc))
    return fail(DIT_EUNSUPPORTED, "%s: pointers/ld must be 16-byte aligned", who);
  return DIT_OK;
}

extern "C" dit_status qkv_project(dit_dtype dt, const void* y, int64_t ld_y, const void* w_qkv,
                                  const void* b_qkv, void* qkv, int64_t ld_qkv, int64_t n_tokens,
                                  int32_t d_model, void* stream) {
  clear_error();
  if (dit_status st = proj_check("qkv_project", dt, y, ld_y, w_qkv, qkv, ld_qkv, n_tokens,
                                 d_model, 3 * (int64_t)d_model))
    return st;
  if (n_tokens == 0) return DIT_OK;
  GemmEpilogue ep{0, b_qkv, nullptr, 0, nullptr, nullptr};
  hipError_t e = launch_gemm(dt == DIT_BF16, y, ld_y, w_qkv, qkv, ld_qkv, n_tokens, 3 * d_model,
                             d_model, ep, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "qkv_project launch");
}

extern "C" dit_status out_proj_gated(dit_dtype dt, const void* o, int64_t ld_o, const void* w_o,
                                     const void* b_o, const void* x, int64_t ld_x,
                                     const uint8_t* modality, const float* table, void* out,
                                     int64_t ld_out, int64_t n_tokens, int32_t d_model,
                                     void* stream) {
  clear_error();
  if (dit_status st = proj_check("out_proj_gated", dt, o, ld_o, w_o, out, ld_out, n_tokens,
                                 d_model, d_model))
    return st;
  if (!x || !modality || !table) return fail(DIT_EINVAL, "out_proj_gated: null pointer");
  if (ld_x < d_model) return fail(DIT_EINVAL, "out_proj_gated: ld_x too small");
  if (!aligned16(x) || !ld_aligned(dt, ld_x))
    return fail(DIT_EUNSUPPORTED, "out_proj_gated: pointers/ld must be 16-byte aligned");
  if (x == out && ld_x != ld_out)
    return fail(DIT_EINVAL, "out_proj_gated: in-place needs ld_x == ld_out");
  if (n_tokens == 0) return DIT_OK;
  GemmEpilogue ep{1, b_o, x, ld_x, modality, table + 2 * (size_t)d_model};
  hipError_t e = launch_gemm(dt == DIT_BF16, o, ld_o, w_o, out, ld_out, n_tokens, d_model,
                             d_model, ep, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "out_proj_gated launch");
}

// ---------------------------------------------------------------------------
// Feed-forward half

extern "C" dit_status ffn_up_gelu(dit_dtype dt, const void* y, int64_t ld_y, const void* w1,
                                  const void* b1, void* h, int64_t ld_h, int64_t n_tokens,
                                  int32_t d_model, int32_t d_ff, void* stream) {
  clear_error();
  if (d_model < 1 || d_ff < 1) return fail(DIT_EINVAL, "ffn_up_gelu: d_model/d_ff < 1");
  if (dit_status st = proj_check("ffn_up_gelu", dt, y, ld_y, w1, h, ld_h, n_tokens, d_model,
                                 d_ff))
    return st;
  if (d_ff % 64 != 0)
    return fail(DIT_EUNSUPPORTED, "ffn_up_gelu: d_ff %d is not a multiple of 64", d_ff);
  if (b1 && !aligned16(b1)) return fail(DIT_EUNSUPPORTED, "ffn_up_gelu: b1 not 16-byte aligned");
  if (n_tokens == 0) return DIT_OK;
  GemmEpilogue ep{2, b1, nullptr, 0, nullptr, nullptr};
  hipError_t e = launch_gemm(dt == DIT_BF16, y, ld_y, w1, h, ld_h, n_tokens, d_ff, d_model, ep,
                             (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "ffn_up_gelu launch");
}

static dit_status down_check(dit_dtype dt, const void* h, int64_t ld_h, const void* w2,
                             const void* x, int64_t ld_x, const uint8_t* modality,
                             const float* table, void* out, int64_t ld_out, int64_t n_tokens,
                             int32_t d_model, int32_t d_ff) {
  if (d_model < 1 || d_ff < 1) return fail(DIT_EINVAL, "ffn_down_gated: d_model/d_ff < 1");
  if (dit_status st = proj_check("ffn_down_gated", dt, h, ld_h, w2, out, ld_out, n_tokens, d_ff,
                                 d_model))
    return st;
  if (!x || !modality || !table) return fail(DIT_EINVAL, "ffn_down_gated: null pointer");
  if (ld_x < d_model) return fail(DIT_EINVAL, "ffn_down_gated: ld_x too small");
  if (d_model % 64 != 0)
    return fail(DIT_EUNSUPPORTED, "ffn_down_gated: d_model %d is not a multiple of 64", d_model);
  if (!aligned16(x) || !ld_aligned(dt, ld_x))
    return fail(DIT_EUNSUPPORTED, "ffn_down_gated: pointers/ld must be 16-byte aligned");
  if (x == out && ld_x != ld_out)
    return fail(DIT_EINVAL, "ffn_down_gated: in-place needs ld_x == ld_out");
  return DIT_OK;
}

extern "C" dit_status ffn_down_gated(dit_dtype dt, const void* h, int64_t ld_h, const void* w2,
                                     const void* b2, const void* x, int64_t ld_x,
                                     const uint8_t* modality, const float* table, void* out,
                                     int64_t ld_out, int64_t n_tokens, int32_t d_model,
                                     int32_t d_ff, void* stream) {
  clear_error();
  if (dit_status st = down_check(dt, h, ld_h, w2, x, ld_x, modality, table, out, ld_out,
                                 n_tokens, d_model, d_ff))
    return st;
  if (b2 && !aligned16(b2)) return fail(DIT_EUNSUPPORTED, "ffn_down_gated: b2 not 16-byte aligned");
  if (n_tokens == 0) return DIT_OK;
  GemmEpilogue ep{1, b2, x, ld_x, modality, table + 2 * (size_t)d_model};
  hipError_t e = launch_gemm(dt == DIT_BF16, h, ld_h, w2, out, ld_out, n_tokens, d_model, d_ff,
                             ep, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "ffn_down_gated launch");
}

// ---------------------------------------------------------------------------
// FP8 projections

extern "C" dit_status quantize_rows_fp8(dit_dtype dt, const void* x, int64_t ld_x, uint8_t* q,
                                        int64_t ld_q, float* scales, int64_t n_rows, int32_t d,
                                        void* stream) {
  clear_error();
  if (!dtype_ok(dt)) return fail(DIT_EINVAL, "quantize_rows_fp8: unknown dtype %d", (int)dt);
  if (!x || !q || !scales) return fail(DIT_EINVAL, "quantize_rows_fp8: null pointer");
  if (d < 1) return fail(DIT_EINVAL, "quantize_rows_fp8: d < 1");
  if (ld_x < d || ld_q < d) return fail(DIT_EINVAL, "quantize_rows_fp8: ld < d");
  if (dit_status st = check_stream_rows(n_rows)) return st;
  if (d % 8 != 0 || d > (dt == DIT_BF16 ? 20480 : 10240))
    return fail(DIT_EUNSUPPORTED, "quantize_rows_fp8: d %d unsupported", d);
  if (!aligned16(x) || !aligned16(q) || !aligned16(scales) || !ld_aligned(dt, ld_x) ||
      ld_q % 16 != 0)
    return fail(DIT_EUNSUPPORTED, "quantize_rows_fp8: pointers/ld must be 16-byte aligned");
  if (n_rows == 0) return DIT_OK;
  hipError_t e = launch_quant_rows_fp8(dt == DIT_BF16, x, ld_x, q, ld_q, scales, n_rows, d,
                                       (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "quantize_rows_fp8 launch");
}

extern "C" dit_status linear_fp8(const uint8_t* a, int64_t ld_a, const float* a_scales,
                                 const uint8_t* w, const float* w_scales, const void* bias,
                                 dit_epilogue epi, const void* x, int64_t ld_x,
                                 const uint8_t* modality, const float* table, void* out,
                                 int64_t ld_out, int64_t n_tokens, int32_t k_in, int32_t n_out,
                                 void* stream) {
  clear_error();
  if (!a || !a_scales || !w || !w_scales || !out) return fail(DIT_EINVAL, "linear_fp8: null pointer");
  if (epi != DIT_EPI_PLAIN && epi != DIT_EPI_GATED && epi != DIT_EPI_GELU)
    return fail(DIT_EINVAL, "linear_fp8: unknown epilogue %d", (int)epi);
  if (epi == DIT_EPI_GATED && (!x || !modality || !table))
    return fail(DIT_EINVAL, "linear_fp8: the gated epilogue needs x, modality and table");
  if (k_in < 1 || n_out < 1) return fail(DIT_EINVAL, "linear_fp8: width < 1");
  if (ld_a < k_in || ld_out < n_out || (epi == DIT_EPI_GATED && ld_x < n_out))
    return fail(DIT_EINVAL, "linear_fp8: ld too small");
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  if (k_in % 128 != 0 || n_out % 4 != 0)
    return fail(DIT_EUNSUPPORTED, "linear_fp8: k_in %d must be a multiple of 128, n_out %d of 4",
                k_in, n_out);
  if (!aligned16(a) || ld_a % 16 != 0 || !aligned16(w) || !aligned16(w_scales) ||
      !aligned16(out) || !ld_aligned(DIT_BF16, ld_out) || (bias && !aligned16(bias)) ||
      (epi == DIT_EPI_GATED && (!aligned16(x) || !ld_aligned(DIT_BF16, ld_x) || !aligned16(table))))
    return fail(DIT_EUNSUPPORTED, "linear_fp8: pointers/ld must be 16-byte aligned");
  if (epi == DIT_EPI_GATED && x == out && ld_x != ld_out)
    return fail(DIT_EINVAL, "linear_fp8: in-place needs ld_x == ld_out");
  if (n_tokens == 0) return DIT_OK;
  GemmEpilogue ep{(int)epi, bias, epi == DIT_EPI_GATED ? x : nullptr, ld_x,
                  epi == DIT_EPI_GATED ? modality : nullptr,
                  epi == DIT_EPI_GATED ? table + 2 * (size_t)n_out : nullptr};
  hipError_t e = launch_gemm_fp8(a, ld_a, a_scales, w, w_scales, out, ld_out, n_tokens, n_out,
                                 k_in, ep, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "linear_fp8 launch");
}

// ---------------------------------------------------------------------------
// Denoising step

static dit_status denoise_check(dit_dtype dt, const float* z, int64_t ld_z, const void* v,
                                int64_t ld_v, const float* x0, int64_t ld_x0,
                                const uint8_t* modality, const uint8_t* anchor,
                                const float* anchor_vals, int64_t ld_a, int64_t n_rows,
                                int32_t channels, const float* sigmas, int32_t sign) {
  if (!dtype_ok(dt)) return fail(DIT_EINVAL, "denoise_step: unknown dtype %d", (int)dt);
  if (!z || !v || !modality || !sigmas) return fail(DIT_EINVAL, "denoise_step: null pointer");
  if (anchor && !anchor_vals)
    return fail(DIT_EINVAL, "denoise_step: anchor flags given without anchor_vals");
  if (channels < 1) return fail(DIT_EINVAL, "denoise_step: channels < 1");
  if (ld_z < channels || ld_v < channels || (x0 && ld_x0 < channels) ||
      (anchor && ld_a < channels))
    return fail(DIT_EINVAL, "denoise_step: ld < channels");
  if (n_rows < 0) return fail(DIT_EINVAL, "denoise_step: n_rows < 0");
  for (int i = 0; i < 4; ++i)
    if (!(sigmas[i] >= 0.0f && sigmas[i] <= 1.0f))
      return fail(DIT_EINVAL, "denoise_step: sigma[%d] = %g is not in [0, 1]", i,
                  (double)sigmas[i]);
  if (sign != 1 && sign != -1)
    return fail(DIT_EINVAL, "denoise_step: velocity_sign %d is not +1 or -1", sign);
  if (channels % 4 != 0)
    return fail(DIT_EUNSUPPORTED, "denoise_step: channels %d is not a multiple of 4", channels);
  if (n_rows * (int64_t)(channels / 4) > INT32_MAX)
    return fail(DIT_EUNSUPPORTED, "denoise_step: more than 2^31-1 groups of 4 channels");
  if (!aligned16(z) || !aligned16(v) || (x0 && !aligned16(x0)) ||
      (anchor && !aligned16(anchor_vals)) || !ld_aligned(DIT_F32, ld_z) || !ld_aligned(dt, ld_v) ||
      (x0 && !ld_aligned(DIT_F32, ld_x0)) || (anchor && !ld_aligned(DIT_F32, ld_a)))
    return fail(DIT_EUNSUPPORTED, "denoise_step: pointers/ld must be 16-byte aligned");
  return DIT_OK;
}

extern "C" dit_status denoise_step(dit_dtype v_dtype, float* z, int64_t ld_z, const void* v,
                                   int64_t ld_v, float* x0, int64_t ld_x0,
                                   const uint8_t* modality, const uint8_t* anchor,
                                   const float* anchor_vals, int64_t ld_a, int64_t n_rows,
                                   int32_t channels, const float sigmas[4],
                                   int32_t velocity_sign, void* stream) {
  clear_error();
  if (dit_status st = denoise_check(v_dtype, z, ld_z, v, ld_v, x0, ld_x0, modality, anchor,
                                    anchor_vals, ld_a, n_rows, channels, sigmas, velocity_sign))
    return st;
  if (n_rows == 0) return DIT_OK;
  hipError_t e = launch_denoise(v_dtype == DIT_BF16, z, ld_z, v, ld_v, x0, ld_x0, modality,
                                anchor, anchor_vals, ld_a, n_rows, channels, sigmas,
                                (float)velocity_sign, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "denoise_step launch");
}

// ---------------------------------------------------------------------------
// DiffusionNFT loss

extern "C" size_t dit_nft_workspace_bytes(int32_t n_samples, int32_t max_rows) {
  if (n_samples < 1 || max_rows < 1) return 0;
  return nft_workspace_layout(n_samples, max_rows, nullptr);
}

extern "C" dit_status nft_loss(dit_dtype v_dtype, const void* v_theta, int64_t ld_vt,
                               const void* v_old, int64_t ld_vo, const float* v_target,
                               int64_t ld_t, const uint8_t* loss_mask, const int32_t* cu_samples,
                               int32_t n_samples, int32_t max_rows, int64_t n_rows,
                               int32_t channels, const float* reward, float beta,
                               int32_t velocity_sign, float grad_scale, float* grad, int64_t ld_g,
                               float* loss_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  clear_error();
  const dit_dtype dt = v_dtype;
  if (!dtype_ok(dt)) return fail(DIT_EINVAL, "nft_loss: unknown dtype %d", (int)dt);
  if (!v_theta || !v_old || !v_target || !cu_samples || !reward || !loss_out)
    return fail(DIT_EINVAL, "nft_loss: null pointer");
  if (n_samples < 1) return fail(DIT_EINVAL, "nft_loss: n_samples < 1");
  if (dit_status st = check_stream_rows(n_rows)) return st;
  if (n_rows > 0 && max_rows < 1) return fail(DIT_EINVAL, "nft_loss: max_rows < 1");
  if (channels < 1) return fail(DIT_EINVAL, "nft_loss: channels < 1");
  if (ld_vt < channels || ld_vo < channels || ld_t < channels || (grad && ld_g < channels))
    return fail(DIT_EINVAL, "nft_loss: ld < channels");
  if (!std::isfinite(beta) || !std::isfinite(grad_scale))
    return fail(DIT_EINVAL, "nft_loss: beta and grad_scale must be finite");
  if (velocity_sign != 1 && velocity_sign != -1)
    return fail(DIT_EINVAL, "nft_loss: velocity_sign %d is not +1 or -1", velocity_sign);
  if (channels % 4 != 0)
    return fail(DIT_EUNSUPPORTED, "nft_loss: channels %d is not a multiple of 4", channels);
  if (n_samples > 65535) return fail(DIT_EUNSUPPORTED, "nft_loss: more than 65535 samples");
  if (!aligned16(v_theta) || !aligned16(v_old) || !aligned16(v_target) ||
      (grad && !aligned16(grad)) || !ld_aligned(dt, ld_vt) || !ld_aligned(dt, ld_vo) ||
      !ld_aligned(DIT_F32, ld_t) || (grad && !ld_aligned(DIT_F32, ld_g)))
    return fail(DIT_EUNSUPPORTED, "nft_loss: pointers/ld must be 16-byte aligned");
  if (n_rows == 0) max_rows = std::max(max_rows, 1);
  const size_t need = dit_nft_workspace_bytes(n_samples, max_rows);
  if (!workspace || workspace_bytes < need)
    return fail(DIT_EWORKSPACE, "nft_loss: workspace %zu bytes, need %zu", workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(DIT_EUNSUPPORTED, "nft_loss: workspace must be 256-byte aligned");
  hipError_t e = launch_nft_loss(dt == DIT_BF16, v_theta, ld_vt, v_old, ld_vo, v_target, ld_t,
                                 loss_mask, cu_samples, n_samples, max_rows, channels, reward,
                                 beta, (float)velocity_sign, grad_scale, grad, ld_g, loss_out,
                                 workspace, (hipStream_t)stream);
  return e == hipSuccess ? DIT_OK : hip_fail(e, "nft_loss launch");
}

// ---------------------------------------------------------------------------


// An FP8 projection inside a block: W [n_out][k_in] codes with per-row
// scales, optional bf16 bias [n_out].
static dit_status fp8_weight_check(const char* who, const uint8_t* w, const float* w_scales,
                                   const void* bias, int32_t k_in, int32_t n_out) {
  if (!w || !w_scales) return fail(DIT_EINVAL, "%s: null weight pointer", who);
  if (k_in % 128 != 0 || n_out % 32 != 0)
    return fail(DIT_EUNSUPPORTED, "%s: widths %d x %d (multiples of 128 and 32 only)", who,
                n_out, k_in);
  if (!aligned16(w) || !aligned16(w_scales) || (bias && !aligned16(bias)))
    return fail(DIT_EUNSUPPORTED, "%s: weight pointers must be 16-byte aligned", who);
  return DIT_OK;
}

extern "C" size_t dit_ffn_workspace_bytes(const dit_ffn_desc* d, int64_t n_tokens) {
  if (!d || !dtype_ok(d->dtype) || d->d_model < 1 || d->d_ff < 1 || n_tokens < 0) return 0;
  const size_t es = elt_size(d->dtype), n = (size_t)n_tokens;
  return round256(n * (size_t)d->d_model * es) + round256(n * (size_t)d->d_ff * es);
}

extern "C" dit_status dit_ffn_forward(const dit_ffn_desc* d, const void* x, void* out,
                                      const uint8_t* modality, int64_t n_tokens,
                                      const float* ada_table, const void* w1, const void* b1,
                                      const void* w2, const void* b2, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  clear_error();
  if (!d) return fail(DIT_EINVAL, "dit_ffn_forward: null descriptor");
  const dit_dtype dt = d->dtype;
  if (!dtype_ok(dt)) return fail(DIT_EINVAL, "dit_ffn_forward: unknown dtype %d", (int)dt);
  const int32_t D = d->d_model, F = d->d_ff;
  if (D < 1 || F < 1) return fail(DIT_EINVAL, "dit_ffn_forward: d_model/d_ff < 1");
  if (!x || !out || !modality || !ada_table || !w1 || !w2)
    return fail(DIT_EINVAL, "dit_ffn_forward: null pointer");
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  const size_t need = dit_ffn_workspace_bytes(d, n_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(DIT_EWORKSPACE, "dit_ffn_forward: workspace %zu bytes, need %zu",
                workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(DIT_EUNSUPPORTED, "dit_ffn_forward: workspace must be 256-byte aligned");
  const size_t es = elt_size(dt), n = (size_t)n_tokens;
  char* ws = static_cast<char*>(workspace);
  void* y = ws;
  void* h = ws + round256(n * (size_t)D * es);

  // Validate every stage before enqueuing any of them.
  if (dit_status st = adaln_check(dt, x, D, modality, ada_table, y, D, n_tokens, D, d->ln_eps))
    return st;
  if (dit_status st = proj_check("ffn_up_gelu", dt, y, D, w1, h, F, n_tokens, D, F)) return st;
  if (dit_status st = down_check(dt, h, F, w2, x, D, modality, ada_table, out, D, n_tokens, D, F))
    return st;
  if (F % 64 != 0)
    return fail(DIT_EUNSUPPORTED, "dit_ffn_forward: d_ff %d is not a multiple of 64", F);
  if ((b1 && !aligned16(b1)) || (b2 && !aligned16(b2)) || !aligned16(out))
    return fail(DIT_EUNSUPPORTED, "dit_ffn_forward: pointers must be 16-byte aligned");
  if (n_tokens == 0) return DIT_OK;

  if (validate_on()) {
    if (dit_status st = validate_modality("dit_ffn_forward", modality, n_tokens, stream))
      return st;
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_adaln(dt == DIT_BF16, x, D, modality, ada_table, y, D, n_tokens, D,
                              d->ln_eps, s);
  if (e != hipSuccess) return hip_fail(e, "dit_ffn_forward: adaln launch");
  GemmEpilogue ep_up{2, b1, nullptr, 0, nullptr, nullptr};
  e = launch_gemm(dt == DIT_BF16, y, D, w1, h, F, n_tokens, F, D, ep_up, s);
  if (e != hipSuccess) return hip_fail(e, "dit_ffn_forward: up-projection launch");
  GemmEpilogue ep_down{1, b2, x, D, modality, ada_table + 2 * (size_t)D};
  e = launch_gemm(dt == DIT_BF16, h, F, w2, out, D, n_tokens, D, F, ep_down, s);
  if (e != hipSuccess) return hip_fail(e, "dit_ffn_forward: down-projection launch");
  return DIT_OK;
}

// FP8 feed-forward workspace: codes [N][d_ff] (the AdaLN output's codes
// [N][d_model] first, then h's) | h bf16 [N][d_ff] | row scales [N] float32.
extern "C" size_t dit_ffn_fp8_workspace_bytes(const dit_ffn_desc* d, int64_t n_tokens) {
  if (!d || d->dtype != DIT_BF16 || d->d_model < 1 || d->d_ff < 1 || n_tokens < 0) return 0;
  const size_t n = (size_t)n_tokens, F = (size_t)d->d_ff;
  return round256(n * std::max(F, (size_t)d->d_model)) + round256(n * F * 2) + round256(n * 4);
}

extern "C" dit_status dit_ffn_forward_fp8(const dit_ffn_desc* d, const void* x, void* out,
                                          const uint8_t* modality, int64_t n_tokens,
                                          const float* ada_table, const uint8_t* w1,
                                          const float* w1_scales, const void* b1,
                                          const uint8_t* w2, const float* w2_scales,
                                          const void* b2, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  clear_error();
  const char* who = "dit_ffn_forward_fp8";
  if (!d) return fail(DIT_EINVAL, "%s: null descriptor", who);
  if (d->dtype != DIT_BF16)
    return fail(DIT_EUNSUPPORTED, "%s: bf16 activations only (dtype %d)", who, (int)d->dtype);
  const int32_t D = d->d_model, F = d->d_ff;
  if (D < 1 || F < 1) return fail(DIT_EINVAL, "%s: d_model/d_ff < 1", who);
  if (!x || !out || !modality || !ada_table) return fail(DIT_EINVAL, "%s: null pointer", who);
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  const size_t need = dit_ffn_fp8_workspace_bytes(d, n_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(DIT_EWORKSPACE, "%s: workspace %zu bytes, need %zu", who, workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(DIT_EUNSUPPORTED, "%s: workspace must be 256-byte aligned", who);
  const size_t n = (size_t)n_tokens;
  char* ws = static_cast<char*>(workspace);
  uint8_t* codes = reinterpret_cast<uint8_t*>(ws);
  void* h = ws + round256(n * std::max((size_t)F, (size_t)D));
  float* scales = reinterpret_cast<float*>(static_cast<char*>(h) + round256(n * (size_t)F * 2));

  if (dit_status st = adaln_fp8_check(DIT_BF16, x, D, modality, ada_table, codes, D, scales,
                                      n_tokens, D, d->ln_eps))
    return st;
  if (dit_status st = fp8_weight_check(who, w1, w1_scales, b1, D, F)) return st;
  if (dit_status st = fp8_weight_check(who, w2, w2_scales, b2, F, D)) return st;
  if (F > 20480) return fail(DIT_EUNSUPPORTED, "%s: d_ff %d > 20480", who, F);
  if (!aligned16(out)) return fail(DIT_EUNSUPPORTED, "%s: out must be 16-byte aligned", who);
  if (n_tokens == 0) return DIT_OK;

  if (validate_on()) {
    if (dit_status st = validate_modality("dit_ffn_forward_fp8", modality, n_tokens, stream))
      return st;
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_adaln_fp8(1, x, D, modality, ada_table, codes, D, scales, n_tokens, D,
                                  d->ln_eps, s);
  if (e != hipSuccess) return hip_fail(e, "dit_ffn_forward_fp8: adaln launch");
  GemmEpilogue ep_up{2, b1, nullptr, 0, nullptr, nullptr};
  e = launch_gemm_fp8(codes, D, scales, w1, w1_scales, h, F, n_tokens, F, D, ep_up, s);
  if (e != hipSuccess) return hip_fail(e, "dit_ffn_forward_fp8: up-projection launch");
  // h's codes replace the AdaLN codes (consumed by the up-projection).
  e = launch_quant_rows_fp8(1, h, F, codes, F, scales, n_tokens, F, s);
  if (e != hipSuccess) return hip_fail(e, "dit_ffn_forward_fp8: quantization launch");
  GemmEpilogue ep_down{1, b2, x, D, modality, ada_table + 2 * (size_t)D};
  e = launch_gemm_fp8(codes, F, scales, w2, w2_scales, out, D, n_tokens, D, F, ep_down, s);
  if (e != hipSuccess) return hip_fail(e, "dit_ffn_forward_fp8: down-projection launch");
  return DIT_OK;
}

// ---------------------------------------------------------------------------

// Block workspace: five [N][D] planes, y | q' | k' | v | o, each rounded up to
// 256 bytes.  q, k and v are separate planes (not one [N][3D] array), so the
// attention's K/V loads stream contiguous rows.  bf16: the QKV GEMM rotates q
// and k in its epilogue (kind 3, from the positions) and stores q', k', v
// straight into planes 1-3.  float32: the GEMM stores q, k, v and RoPE then
// turns planes 1 and 2 in place.
namespace {
struct BlockLayout {
  size_t plane, total;
};
BlockLayout block_layout(const dit_block_desc* d, int64_t n_tokens) {
  const size_t es = elt_size(d->dtype), n = (size_t)n_tokens, D = (size_t)d->d_model;
  BlockLayout L;
  L.plane = round256(n * D * es);
  L.total = 5 * L.plane;
  return L;
}
}  // namespace

extern "C" size_t dit_block_workspace_bytes(const dit_block_desc* d, int64_t n_tokens) {
  if (!d || !dtype_ok(d->dtype) || d->d_model < 1 || n_tokens < 0) return 0;
  return block_layout(d, n_tokens).total;
}

extern "C" dit_status dit_block_intermediates(const dit_block_desc* d, int64_t n_tokens,
                                              int64_t offsets[5]) {
  clear_error();
  if (!d || !offsets) return fail(DIT_EINVAL, "dit_block_intermediates: null pointer");
  if (!dtype_ok(d->dtype) || d->d_model < 1 || n_tokens < 0)
    return fail(DIT_EINVAL, "dit_block_intermediates: bad descriptor or n_tokens");
  const BlockLayout L = block_layout(d, n_tokens);
  for (int i = 0; i < 5; ++i) offsets[i] = (int64_t)(i * L.plane);
  return DIT_OK;
}

extern "C" dit_status dit_block_forward(const dit_block_desc* d, const void* x, void* out,
                                        const uint8_t* modality, const int32_t* pos_thw,
                                        const int32_t* cu_seqlens, int32_t n_seqs,
                                        int32_t max_seqlen, int64_t n_tokens,
                                        const float* ada_table, const void* w_qkv,
                                        const void* b_qkv, const void* w_o, const void* b_o,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  if (!d) return fail(DIT_EINVAL, "dit_block_forward: null descriptor");
  const dit_dtype dt = d->dtype;
  if (!dtype_ok(dt)) return fail(DIT_EINVAL, "dit_block_forward: unknown dtype %d", (int)dt);
  const int32_t D = d->d_model, H = d->n_heads, Dh = d->head_dim;
  if (D < 1 || H < 1 || Dh < 1 || (int64_t)H * Dh != D)
    return fail(DIT_EINVAL, "dit_block_forward: d_model %d != n_heads %d * head_dim %d", D, H, Dh);
  if (!x || !out || !modality || !pos_thw || !cu_seqlens || !ada_table || !w_qkv || !w_o)
    return fail(DIT_EINVAL, "dit_block_forward: null pointer");
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  const size_t need = dit_block_workspace_bytes(d, n_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(DIT_EWORKSPACE, "dit_block_forward: workspace %zu bytes, need %zu",
                workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(DIT_EUNSUPPORTED, "dit_block_forward: workspace must be 256-byte aligned");

  const size_t es = elt_size(dt);
  const BlockLayout L = block_layout(d, n_tokens);
  char* ws = static_cast<char*>(workspace);
  void* y = ws;
  char* q = ws + L.plane;
  char* k = q + L.plane;
  char* v = k + L.plane;
  void* o = v + L.plane;

  // Validate every stage before enqueuing any of them.
  if (dit_status st = adaln_check(dt, x, D, modality, ada_table, y, D, n_tokens, D, d->ln_eps))
    return st;
  if (dit_status st = proj_check("qkv_project", dt, y, D, w_qkv, q, D, n_tokens, D, D))
    return st;
  if (dit_status st = rope_check(dt, q, D, k, D, pos_thw, n_tokens, H, Dh, d->rope_sections,
                                 d->rope_theta))
    return st;
  if (dit_status st = attn_check(dt, q, D, k, D, v, D, o, D, cu_seqlens, n_seqs, max_seqlen,
                                 n_tokens, H, Dh, d->softmax_scale))
    return st;
  if (dit_status st = proj_check("out_proj_gated", dt, o, D, w_o, out, D, n_tokens, D, D))
    return st;
  if (!aligned16(x) || !aligned16(out))
    return fail(DIT_EUNSUPPORTED, "dit_block_forward: x/out must be 16-byte aligned");
  if (n_tokens == 0) return DIT_OK;

  if (validate_on()) {
    if (dit_status st = validate_segments("dit_block_forward", cu_seqlens, n_seqs, max_seqlen,
                                          n_tokens, stream))
      return st;
    if (dit_status st = validate_modality("dit_block_forward", modality, n_tokens, stream))
      return st;
  }
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t* ev = prof_slot();
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(ev[i], s);
  };
  double freq[64];
  rope_freqs(d->rope_sections, (double)d->rope_theta, Dh, freq);
  const int s_t = d->rope_sections[0], s_h = d->rope_sections[1];
  hipError_t e;
  mark(0);
  e = launch_adaln(dt == DIT_BF16, x, D, modality, ada_table, y, D, n_tokens, D, d->ln_eps, s);
  if (e != hipSuccess) return hip_fail(e, "dit_block_forward: adaln launch");
  mark(1);
  // One GEMM over the fused W_qkv [3D][D], its output split into the q', k', v
  // planes; bf16 rotates q and k in the epilogue.
  if (dt == DIT_BF16) {
    GemmEpilogue ep_qkv{3, b_qkv, nullptr, 0, nullptr, nullptr, D, (int64_t)(L.plane / es),
                        pos_thw, freq, Dh, s_t / 2, (s_t + s_h) / 2};
    e = launch_gemm(1, y, D, w_qkv, q, D, n_tokens, 3 * D, D, ep_qkv, s);
    if (e != hipSuccess) return hip_fail(e, "dit_block_forward: qkv launch");
    mark(2);
  } else {
    GemmEpilogue ep_qkv{0, b_qkv, nullptr, 0, nullptr, nullptr, D, (int64_t)(L.plane / es)};
    e = launch_gemm(0, y, D, w_qkv, q, D, n_tokens, 3 * D, D, ep_qkv, s);
    if (e != hipSuccess) return hip_fail(e, "dit_block_forward: qkv launch");
    mark(2);
    e = launch_rope(0, q, D, k, D, q, D, k, D, pos_thw, n_tokens, H, Dh, s_t, s_h, freq, s);
    if (e != hipSuccess) return hip_fail(e, "dit_block_forward: rope launch");
  }
  mark(3);
  const float scale = d->softmax_scale > 0.0f ? d->softmax_scale : 1.0f / std::sqrt((float)Dh);
  e = launch_attn(dt == DIT_BF16, q, D, k, D, v, D, o, D, cu_seqlens, n_seqs, max_seqlen,
                  n_tokens, H, Dh, scale, d->causal != 0, nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "dit_block_forward: attention launch");
  mark(4);
  GemmEpilogue ep_out{1, b_o, x, D, modality, ada_table + 2 * (size_t)D};
  e = launch_gemm(dt == DIT_BF16, o, D, w_o, out, D, n_tokens, D, D, ep_out, s);
  if (e != hipSuccess) return hip_fail(e, "dit_block_forward: out-proj launch");
  mark(5);
  return DIT_OK;
}

// FP8 block workspace: the five bf16 planes of the bf16 block, then row
// scales [N] float32.  Plane 0 holds the AdaLN codes, then the rotated q,
// then the attention output's codes.
extern "C" size_t dit_block_fp8_workspace_bytes(const dit_block_desc* d, int64_t n_tokens) {
  if (!d || d->dtype != DIT_BF16 || d->d_model < 1 || n_tokens < 0) return 0;
  const size_t n = (size_t)n_tokens, D = (size_t)d->d_model;
  return 5 * round256(n * D * 2) + round256(n * 4);
}

extern "C" size_t dit_block_fp8_attn_workspace_bytes(const dit_block_desc* d, int64_t n_tokens,
                                                     int32_t n_seqs) {
  const size_t base = dit_block_fp8_workspace_bytes(d, n_tokens);
  if (base == 0 || d->n_heads < 1) return 0;
  const size_t att = dit_attn_fp8_workspace_bytes(n_tokens, n_seqs, d->n_heads, d->head_dim);
  return att == 0 ? 0 : base + att;
}

// The FP8 block; with fp8_attn the attention stage is attn_fp8_prepare +
// attn_packed_fp8 on operands in the workspace past the block's own planes.
static dit_status block_forward_fp8_impl(
    const char* who, bool fp8_attn, const dit_block_desc* d, const void* x, void* out,
    const uint8_t* modality, const int32_t* pos_thw, const int32_t* cu_seqlens, int32_t n_seqs,
    int32_t max_seqlen, int64_t n_tokens, const float* ada_table, const uint8_t* w_qkv,
    const float* w_qkv_scales, const void* b_qkv, const uint8_t* w_o, const float* w_o_scales,
    const void* b_o, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  if (!d) return fail(DIT_EINVAL, "%s: null descriptor", who);
  if (d->dtype != DIT_BF16)
    return fail(DIT_EUNSUPPORTED, "%s: bf16 activations only (dtype %d)", who, (int)d->dtype);
  const int32_t D = d->d_model, H = d->n_heads, Dh = d->head_dim;
  if (D < 1 || H < 1 || Dh < 1 || (int64_t)H * Dh != D)
    return fail(DIT_EINVAL, "%s: d_model %d != n_heads %d * head_dim %d", who, D, H, Dh);
  if (!x || !out || !modality || !pos_thw || !cu_seqlens || !ada_table)
    return fail(DIT_EINVAL, "%s: null pointer", who);
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  const size_t base_need = dit_block_fp8_workspace_bytes(d, n_tokens);
  const size_t need = fp8_attn ? dit_block_fp8_attn_workspace_bytes(d, n_tokens, n_seqs) : base_need;
  if (fp8_attn && need == 0)
    return fail(n_seqs < 1 ? DIT_EINVAL : DIT_EUNSUPPORTED, "%s: n_seqs %d / head_dim %d", who,
                n_seqs, Dh);
  if (!workspace || workspace_bytes < need)
    return fail(DIT_EWORKSPACE, "%s: workspace %zu bytes, need %zu", who, workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(DIT_EUNSUPPORTED, "%s: workspace must be 256-byte aligned", who);
  void* attn_ws = static_cast<char*>(workspace) + base_need;
  const size_t attn_ws_bytes = workspace_bytes - base_need;

  const size_t n = (size_t)n_tokens;
  const size_t plane_bytes = round256(n * D * 2);
  char* ws = static_cast<char*>(workspace);
  char* p0 = ws;
  char* q = ws + plane_bytes;
  char* k = q + plane_bytes;
  char* v = k + plane_bytes;
  char* o = v + plane_bytes;
  float* scales = reinterpret_cast<float*>(o + plane_bytes);
  uint8_t* codes = reinterpret_cast<uint8_t*>(p0);
  // Stage by stage: AdaLN codes -> p0; QKV -> q, k, v planes; RoPE: q' -> p0
  // (the codes are consumed), k' -> over q; attention -> o; o's codes -> p0
  // (q' is consumed); output projection -> out.
  void* qr = p0;
  void* kr = q;
  if (dit_status st = adaln_fp8_check(DIT_BF16, x, D, modality, ada_table, codes, D, scales,
                                      n_tokens, D, d->ln_eps))
    return st;
  if (dit_status st = fp8_weight_check(who, w_qkv, w_qkv_scales, b_qkv, D, 3 * D)) return st;
  if (dit_status st = rope_check(DIT_BF16, q, D, k, D, pos_thw, n_tokens, H, Dh,
                                 d->rope_sections, d->rope_theta))
    return st;
  if (dit_status st = attn_check(DIT_BF16, qr, D, kr, D, v, D, o, D, cu_seqlens, n_seqs,
                                 max_seqlen, n_tokens, H, Dh, d->softmax_scale))
    return st;
  if (fp8_attn) {
    if (dit_status st = fp8_attn_check(who, cu_seqlens, n_seqs, max_seqlen, n_tokens, H, Dh,
                                       attn_ws, attn_ws_bytes))
      return st;
  }
  if (dit_status st = fp8_weight_check(who, w_o, w_o_scales, b_o, D, D)) return st;
  if (!aligned16(out)) return fail(DIT_EUNSUPPORTED, "%s: out must be 16-byte aligned", who);
  if (n_tokens == 0) return DIT_OK;

  if (validate_on()) {
    if (dit_status st = validate_segments(who, cu_seqlens, n_seqs, max_seqlen, n_tokens, stream))
      return st;
    if (dit_status st = validate_modality(who, modality, n_tokens, stream)) return st;
  }
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t* ev = prof_slot();
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(ev[i], s);
  };
  hipError_t e;
  mark(0);
  e = launch_adaln_fp8(1, x, D, modality, ada_table, codes, D, scales, n_tokens, D, d->ln_eps, s);
  if (e != hipSuccess) return hip_fail(e, "dit_block_forward_fp8: adaln launch");
  mark(1);
  GemmEpilogue ep_qkv{0, b_qkv, nullptr, 0, nullptr, nullptr, D, (int64_t)(plane_bytes / 2)};
  e = launch_gemm_fp8(codes, D, scales, w_qkv, w_qkv_scales, q, D, n_tokens, 3 * D, D, ep_qkv, s);
  if (e != hipSuccess) return hip_fail(e, "dit_block_forward_fp8: qkv launch");
  mark(2);
  double freq[64];
  rope_freqs(d->rope_sections, (double)d->rope_theta, Dh, freq);
  e = launch_rope(1, q, D, k, D, qr, D, kr, D, pos_thw, n_tokens, H, Dh, d->rope_sections[0],
                  d->rope_sections[1], freq, s);
  if (e != hipSuccess) return hip_fail(e, "dit_block_forward_fp8: rope launch");
  mark(3);
  const float scale = d->softmax_scale > 0.0f ? d->softmax_scale : 1.0f / std::sqrt((float)Dh);
  if (fp8_attn) {
    const AttnFp8Ops ops = fp8_attn_ops(attn_ws, fp8_attn_layout(n_tokens, n_seqs, H));
    e = launch_attn_fp8_prepare(static_cast<const uint16_t*>(qr), D,
                                static_cast<const uint16_t*>(kr), D,
                                static_cast<const uint16_t*>(static_cast<void*>(v)), D,
                                cu_seqlens, n_seqs, max_seqlen, n_tokens, H, ops, s);
    if (e == hipSuccess)
      e = launch_attn_fp8(ops, reinterpret_cast<uint16_t*>(o), D, cu_seqlens, n_seqs, max_seqlen,
                          n_tokens, H, scale, d->causal != 0, s);
  } else {
    e = launch_attn(1, qr, D, kr, D, v, D, o, D, cu_seqlens, n_seqs, max_seqlen, n_tokens, H, Dh,
                    scale, d->causal != 0, nullptr, s);
  }
  if (e != hipSuccess) return hip_fail(e, "dit_block_forward_fp8: attention launch");
  mark(4);
  e = launch_quant_rows_fp8(1, o, D, codes, D, scales, n_tokens, D, s);
  if (e != hipSuccess) return hip_fail(e, "dit_block_forward_fp8: quantization launch");
  GemmEpilogue ep_out{1, b_o, x, D, modality, ada_table + 2 * (size_t)D};
  e = launch_gemm_fp8(codes, D, scales, w_o, w_o_scales, out, D, n_tokens, D, D, ep_out, s);
  if (e != hipSuccess) return hip_fail(e, "dit_block_forward_fp8: out-proj launch");
  mark(5);
  return DIT_OK;
}

extern "C" dit_status dit_block_forward_fp8(
    const dit_block_desc* d, const void* x, void* out, const uint8_t* modality,
    const int32_t* pos_thw, const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
    int64_t n_tokens, const float* ada_table, const uint8_t* w_qkv, const float* w_qkv_scales,
    const void* b_qkv, const uint8_t* w_o, const float* w_o_scales, const void* b_o,
    void* workspace, size_t workspace_bytes, void* stream) {
  return block_forward_fp8_impl("dit_block_forward_fp8", false, d, x, out, modality, pos_thw,
                                cu_seqlens, n_seqs, max_seqlen, n_tokens, ada_table, w_qkv,
                                w_qkv_scales, b_qkv, w_o, w_o_scales, b_o, workspace,
                                workspace_bytes, stream);
}

extern "C" dit_status dit_block_forward_fp8_attn(
    const dit_block_desc* d, const void* x, void* out, const uint8_t* modality,
    const int32_t* pos_thw, const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
    int64_t n_tokens, const float* ada_table, const uint8_t* w_qkv, const float* w_qkv_scales,
    const void* b_qkv, const uint8_t* w_o, const float* w_o_scales, const void* b_o,
    void* workspace, size_t workspace_bytes, void* stream) {
  return block_forward_fp8_impl("dit_block_forward_fp8_attn", true, d, x, out, modality, pos_thw,
                                cu_seqlens, n_seqs, max_seqlen, n_tokens, ada_table, w_qkv,
                                w_qkv_scales, b_qkv, w_o, w_o_scales, b_o, workspace,
                                workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Backward pass of the attention half.
//
// Workspace (each region 256-byte aligned; Np = n_tokens rounded up to 64,
// PT = round256(D * Np * 2) bytes, one bf16 [N][D] or [D][Np] plane):
//   Y | Q K V (3 PT; later dqkv^T [3D][Np]) | O (later dy) | ZD (z, then do) |
//   DZ | T1 (dz^T, then y^T) | T2 (o^T) | DQKV [N][3D] (3 PT) | LSE, DELTA
//   [H][N] float | WT (W_o^T, then W_qkv^T) | STATS [N] float2 | column-sum
//   partials.
namespace {
struct BwdLayout {
  size_t pt, y, qkv, o, zd, dz, t1, t2, dqkv, lse, delta, wt, stats, part, total;
};
BwdLayout bwd_layout(int64_t n, int32_t d, int32_t h) {
  BwdLayout L{};
  const size_t np = (size_t)((n + 63) / 64 * 64);
  L.pt = round256((size_t)d * np * 2);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round256(bytes);
    return at;
  };
  L.y = take(L.pt);
  L.qkv = take(3 * L.pt);
  L.o = take(L.pt);
  L.zd = take(L.pt);
  L.dz = take(L.pt);
  L.t1 = take(L.pt);
  L.t2 = take(L.pt);
  L.dqkv = take(3 * L.pt);
  L.lse = take((size_t)h * (size_t)n * 4);
  L.delta = take((size_t)h * (size_t)n * 4);
  L.wt = take((size_t)3 * d * d * 2);
  L.stats = take((size_t)n * 8);
  L.part = take(std::max(colsum_partial_bytes(n, 3 * d, 1), colsum_partial_bytes(n, d, 3)));
  L.total = off;
  return L;
}
}  // namespace

extern "C" size_t dit_block_backward_workspace_bytes(const dit_block_desc* d, int64_t n_tokens) {
  if (!d || d->dtype != DIT_BF16 || d->d_model < 1 || d->n_heads < 1 || n_tokens < 0) return 0;
  return bwd_layout(n_tokens, d->d_model, d->n_heads).total;
}

extern "C" dit_status dit_block_backward(
    const dit_block_desc* d, const void* x, const void* dout, const uint8_t* modality,
    const int32_t* pos_thw, const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
    int64_t n_tokens, const float* ada_table, const void* w_qkv, const void* b_qkv,
    const void* w_o, const void* b_o, void* dx, float* dtable, void* dw_qkv, float* db_qkv,
    void* dw_o, float* db_o, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  const char* who = "dit_block_backward";
  if (!d) return fail(DIT_EINVAL, "%s: null descriptor", who);
  if (d->dtype != DIT_BF16)
    return fail(DIT_EUNSUPPORTED, "%s: bf16 only (dtype %d)", who, (int)d->dtype);
  const int32_t D = d->d_model, H = d->n_heads, Dh = d->head_dim;
  if (D < 1 || H < 1 || Dh < 1 || (int64_t)H * Dh != D)
    return fail(DIT_EINVAL, "%s: d_model %d != n_heads %d * head_dim %d", who, D, H, Dh);
  if (!x || !dout || !modality || !pos_thw || !cu_seqlens || !ada_table || !w_qkv || !w_o ||
      !dx || !dtable || !dw_qkv || !dw_o)
    return fail(DIT_EINVAL, "%s: null pointer", who);
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  if (D % 64 != 0) return fail(DIT_EUNSUPPORTED, "%s: d_model %d not a multiple of 64", who, D);
  const BwdLayout L = bwd_layout(n_tokens, D, H);
  if (!workspace || workspace_bytes < L.total)
    return fail(DIT_EWORKSPACE, "%s: workspace %zu bytes, need %zu", who, workspace_bytes,
                L.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(DIT_EUNSUPPORTED, "%s: workspace must be 256-byte aligned", who);
  char* ws = static_cast<char*>(workspace);
  char *Y = ws + L.y, *Q = ws + L.qkv, *K = Q + L.pt, *V = K + L.pt, *O = ws + L.o;
  char *ZD = ws + L.zd, *DZ = ws + L.dz, *T1 = ws + L.t1, *T2 = ws + L.t2, *DQKV = ws + L.dqkv;
  float* LSE = reinterpret_cast<float*>(ws + L.lse);
  float* DELTA = reinterpret_cast<float*>(ws + L.delta);
  char* WT = ws + L.wt;
  float* STATS = reinterpret_cast<float*>(ws + L.stats);
  float* PART = reinterpret_cast<float*>(ws + L.part);
  const int64_t np = (n_tokens + 63) / 64 * 64;

  // The stages' own checks, before anything is enqueued.
  if (dit_status st = adaln_check(DIT_BF16, x, D, modality, ada_table, Y, D, n_tokens, D,
                                  d->ln_eps))
    return st;
  if (dit_status st = proj_check("qkv_project", DIT_BF16, Y, D, w_qkv, Q, D, n_tokens, D, D))
    return st;
  if (dit_status st = rope_check(DIT_BF16, Q, D, K, D, pos_thw, n_tokens, H, Dh,
                                 d->rope_sections, d->rope_theta))
    return st;
  if (dit_status st = attn_check(DIT_BF16, Q, D, K, D, V, D, O, D, cu_seqlens, n_seqs, max_seqlen,
                                 n_tokens, H, Dh, d->softmax_scale))
    return st;
  if (!aligned16(x) || !aligned16(dout) || !aligned16(dx) || !aligned16(dw_qkv) ||
      !aligned16(dw_o) || !aligned16(dtable) || (b_qkv && !aligned16(b_qkv)) ||
      (b_o && !aligned16(b_o)) || !aligned16(w_o))
    return fail(DIT_EUNSUPPORTED, "%s: pointers must be 16-byte aligned", who);
  if (spans_overlap(dx, D, x, D, n_tokens, D, 2))
    return fail(DIT_EINVAL, "%s: dx overlaps x", who);
  if (n_tokens == 0) return DIT_OK;

  if (validate_on()) {
    if (dit_status st = validate_segments("dit_block_backward", cu_seqlens, n_seqs, max_seqlen,
                                          n_tokens, stream))
      return st;
    if (dit_status st = validate_modality("dit_block_backward", modality, n_tokens, stream))
      return st;
  }
  hipStream_t s = (hipStream_t)stream;
  const float scale = d->softmax_scale > 0.0f ? d->softmax_scale : 1.0f / std::sqrt((float)Dh);
  double freq[64], nfreq[64];
  rope_freqs(d->rope_sections, (double)d->rope_theta, Dh, freq);
  for (int i = 0; i < Dh / 2; ++i) nfreq[i] = -freq[i];
  const int causal = d->causal != 0;
  const int s_t = d->rope_sections[0], s_h = d->rope_sections[1];
  hipError_t e;
#define DIT_BWD(call, what)                                          \
  e = (call);                                                        \
  if (e != hipSuccess) return hip_fail(e, "dit_block_backward: " what)
  // forward stages, recomputed (nothing is saved between the calls)
  DIT_BWD(launch_adaln(1, x, D, modality, ada_table, Y, D, n_tokens, D, d->ln_eps, s), "adaln");
  GemmEpilogue ep_qkv{0, b_qkv, nullptr, 0, nullptr, nullptr, D, (int64_t)(L.pt / 2)};
  DIT_BWD(launch_gemm(1, Y, D, w_qkv, Q, D, n_tokens, 3 * D, D, ep_qkv, s), "qkv");
  DIT_BWD(launch_rope(1, Q, D, K, D, Q, D, K, D, pos_thw, n_tokens, H, Dh, s_t, s_h, freq, s),
          "rope");
  DIT_BWD(launch_attn(1, Q, D, K, D, V, D, O, D, cu_seqlens, n_seqs, max_seqlen, n_tokens, H, Dh,
                      scale, causal, LSE, s),
          "attention");
  GemmEpilogue ep_z{0, b_o, nullptr, 0, nullptr, nullptr};
  DIT_BWD(launch_gemm(1, O, D, w_o, ZD, D, n_tokens, D, D, ep_z, s), "z");
  // out = x + gate * z: dz, the gate rows, db_o
  DIT_BWD(launch_gate_scale(dout, D, modality, ada_table, DZ, D, n_tokens, D, s), "gate");
  DIT_BWD(launch_colsum(1, dout, D, ZD, D, nullptr, modality, n_tokens, D, PART, dtable + 2 * D,
                        3 * D, s),
          "gate rows");
  if (db_o)
    DIT_BWD(launch_colsum(0, DZ, D, nullptr, 0, nullptr, nullptr, n_tokens, D, PART, db_o, 0, s),
            "db_o");
  // z = o W_o^T + b_o: do = dz W_o, dW_o = dz^T o
  GemmEpilogue plain{0, nullptr, nullptr, 0, nullptr, nullptr};
  DIT_BWD(launch_transpose(w_o, D, D, D, WT, D, s), "W_o^T");
  DIT_BWD(launch_gemm(1, DZ, D, WT, ZD, D, n_tokens, D, D, plain, s), "do");
  DIT_BWD(launch_transpose(DZ, D, n_tokens, D, T1, np, s), "dz^T");
  DIT_BWD(launch_transpose(O, D, n_tokens, D, T2, np, s), "o^T");
  DIT_BWD(launch_gemm(1, T1, np, T2, dw_o, D, D, D, (int)np, plain, s), "dW_o");
  // attention, then the rotation's transpose (the rotation by the negated angle)
  DIT_BWD(launch_attn_bwd(Q, D, K, D, V, D, O, D, ZD, D, LSE, DQKV, 3 * D, DQKV + 2 * D, 3 * D,
                          DQKV + 4 * D, 3 * D, cu_seqlens, n_seqs, max_seqlen, n_tokens, H, scale,
                          causal, DELTA, s),
          "attention backward");
  DIT_BWD(launch_rope(1, DQKV, 3 * D, DQKV + 2 * D, 3 * D, DQKV, 3 * D, DQKV + 2 * D, 3 * D,
                      pos_thw, n_tokens, H, Dh, s_t, s_h, nfreq, s),
          "rope backward");
  if (db_qkv)
    DIT_BWD(launch_colsum(0, DQKV, 3 * D, nullptr, 0, nullptr, nullptr, n_tokens, 3 * D, PART,
                          db_qkv, 0, s),
            "db_qkv");
  // [q k v] = y W_qkv^T + b: dy = dqkv W_qkv, dW_qkv = dqkv^T y
  char* DY = O;
  char* DQKVT = Q;
  DIT_BWD(launch_transpose(w_qkv, D, 3 * D, D, WT, 3 * D, s), "W_qkv^T");
  DIT_BWD(launch_gemm(1, DQKV, 3 * D, WT, DY, D, n_tokens, D, 3 * D, plain, s), "dy");
  DIT_BWD(launch_transpose(DQKV, 3 * D, n_tokens, 3 * D, DQKVT, np, s), "dqkv^T");
  DIT_BWD(launch_transpose(Y, D, n_tokens, D, T1, np, s), "y^T");
  DIT_BWD(launch_gemm(1, DQKVT, np, T1, dw_qkv, D, 3 * D, D, (int)np, plain, s), "dW_qkv");
  // AdaLN: dx, then the shift and scale rows
  DIT_BWD(launch_adaln_bwd(x, D, DY, D, dout, D, modality, ada_table, dx, D, STATS, n_tokens, D,
                           d->ln_eps, s),
          "adaln backward");
  DIT_BWD(launch_colsum(0, DY, D, nullptr, 0, nullptr, modality, n_tokens, D, PART, dtable, 3 * D,
                        s),
          "shift rows");
  DIT_BWD(launch_colsum(2, DY, D, x, D, STATS, modality, n_tokens, D, PART, dtable + D, 3 * D, s),
          "scale rows");
#undef DIT_BWD
  return DIT_OK;
}

// ---------------------------------------------------------------------------
// Backward pass of the feed-forward half.
//
// Workspace (Np = n_tokens rounded up to 64; PD = round256(D Np 2), PF =
// round256(F Np 2)): Y [N][D] | A (pre-activation) [N][F] | H = gelu(A) |
// ZD (z, then dy) | DZ | DH (dh, then da in place) | TS (dz^T, then y^T)
// [D][Np] | TB (h^T, then da^T) [F][Np] | WT (W2^T, then W1^T) | STATS |
// column-sum partials.
namespace {
struct FfnBwdLayout {
  size_t pd, pf, y, a, h, zd, dz, dh, ts, tb, wt, stats, part, total;
};
FfnBwdLayout ffn_bwd_layout(int64_t n, int32_t d, int32_t f) {
  FfnBwdLayout L{};
  const size_t np = (size_t)((n + 63) / 64 * 64);
  L.pd = round256((size_t)d * np * 2);
  L.pf = round256((size_t)f * np * 2);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round256(bytes);
    return at;
  };
  L.y = take(L.pd);
  L.a = take(L.pf);
  L.h = take(L.pf);
  L.zd = take(L.pd);
  L.dz = take(L.pd);
  L.dh = take(L.pf);
  L.ts = take(L.pd);
  L.tb = take(L.pf);
  L.wt = take((size_t)f * d * 2);
  L.stats = take((size_t)n * 8);
  L.part = take(std::max(colsum_partial_bytes(n, f, 1), colsum_partial_bytes(n, d, 3)));
  L.total = off;
  return L;
}
}  // namespace

extern "C" size_t dit_ffn_backward_workspace_bytes(const dit_ffn_desc* d, int64_t n_tokens) {
  if (!d || d->dtype != DIT_BF16 || d->d_model < 1 || d->d_ff < 1 || n_tokens < 0) return 0;
  return ffn_bwd_layout(n_tokens, d->d_model, d->d_ff).total;
}

extern "C" dit_status dit_ffn_backward(const dit_ffn_desc* d, const void* x, const void* dout,
                                       const uint8_t* modality, int64_t n_tokens,
                                       const float* ada_table, const void* w1, const void* b1,
                                       const void* w2, const void* b2, void* dx, float* dtable,
                                       void* dw1, float* db1, void* dw2, float* db2,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  const char* who = "dit_ffn_backward";
  if (!d) return fail(DIT_EINVAL, "%s: null descriptor", who);
  if (d->dtype != DIT_BF16)
    return fail(DIT_EUNSUPPORTED, "%s: bf16 only (dtype %d)", who, (int)d->dtype);
  const int32_t D = d->d_model, F = d->d_ff;
  if (D < 1 || F < 1) return fail(DIT_EINVAL, "%s: d_model/d_ff < 1", who);
  if (!x || !dout || !modality || !ada_table || !w1 || !w2 || !dx || !dtable || !dw1 || !dw2)
    return fail(DIT_EINVAL, "%s: null pointer", who);
  if (dit_status st = check_stream_rows(n_tokens)) return st;
  if (D % 64 != 0 || F % 64 != 0)
    return fail(DIT_EUNSUPPORTED, "%s: d_model %d and d_ff %d must be multiples of 64", who, D,
                F);
  const FfnBwdLayout L = ffn_bwd_layout(n_tokens, D, F);
  if (!workspace || workspace_bytes < L.total)
    return fail(DIT_EWORKSPACE, "%s: workspace %zu bytes, need %zu", who, workspace_bytes,
                L.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(DIT_EUNSUPPORTED, "%s: workspace must be 256-byte aligned", who);
  char* ws = static_cast<char*>(workspace);
  char *Y = ws + L.y, *A = ws + L.a, *Hh = ws + L.h, *ZD = ws + L.zd, *DZ = ws + L.dz;
  char *DH = ws + L.dh, *TS = ws + L.ts, *TB = ws + L.tb, *WT = ws + L.wt;
  float* STATS = reinterpret_cast<float*>(ws + L.stats);
  float* PART = reinterpret_cast<float*>(ws + L.part);
  const int64_t np = (n_tokens + 63) / 64 * 64;
  if (dit_status st = adaln_check(DIT_BF16, x, D, modality, ada_table, Y, D, n_tokens, D,
                                  d->ln_eps))
    return st;
  if (!aligned16(dout) || !aligned16(dx) || !aligned16(w1) || !aligned16(w2) ||
      !aligned16(dw1) || !aligned16(dw2) || !aligned16(dtable) || (b1 && !aligned16(b1)) ||
      (b2 && !aligned16(b2)))
    return fail(DIT_EUNSUPPORTED, "%s: pointers must be 16-byte aligned", who);
  if (spans_overlap(dx, D, x, D, n_tokens, D, 2))
    return fail(DIT_EINVAL, "%s: dx overlaps x", who);
  if (n_tokens == 0) return DIT_OK;

  if (validate_on()) {
    if (dit_status st = validate_modality("dit_ffn_backward", modality, n_tokens, stream))
      return st;
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
#define DIT_FBWD(call, what)                                         \
  e = (call);                                                        \
  if (e != hipSuccess) return hip_fail(e, "dit_ffn_backward: " what)
  GemmEpilogue plain{0, nullptr, nullptr, 0, nullptr, nullptr};
  // forward stages, recomputed
  DIT_FBWD(launch_adaln(1, x, D, modality, ada_table, Y, D, n_tokens, D, d->ln_eps, s), "adaln");
  GemmEpilogue ep_b1{0, b1, nullptr, 0, nullptr, nullptr};
  DIT_FBWD(launch_gemm(1, Y, D, w1, A, F, n_tokens, F, D, ep_b1, s), "pre-activation");
  DIT_FBWD(launch_gelu(0, A, F, Hh, F, n_tokens, F, s), "gelu");
  GemmEpilogue ep_b2{0, b2, nullptr, 0, nullptr, nullptr};
  DIT_FBWD(launch_gemm(1, Hh, F, w2, ZD, D, n_tokens, D, F, ep_b2, s), "z");
  // out = x + gate * z: dz, the gate rows, db2
  DIT_FBWD(launch_gate_scale(dout, D, modality, ada_table, DZ, D, n_tokens, D, s), "gate");
  DIT_FBWD(launch_colsum(1, dout, D, ZD, D, nullptr, modality, n_tokens, D, PART, dtable + 2 * D,
                         3 * D, s),
           "gate rows");
  if (db2)
    DIT_FBWD(launch_colsum(0, DZ, D, nullptr, 0, nullptr, nullptr, n_tokens, D, PART, db2, 0, s),
             "db2");
  // z = h W2^T + b2: dh = dz W2, dW2 = dz^T h
  DIT_FBWD(launch_transpose(w2, F, D, F, WT, D, s), "W2^T");
  DIT_FBWD(launch_gemm(1, DZ, D, WT, DH, F, n_tokens, F, D, plain, s), "dh");
  DIT_FBWD(launch_transpose(DZ, D, n_tokens, D, TS, np, s), "dz^T");
  DIT_FBWD(launch_transpose(Hh, F, n_tokens, F, TB, np, s), "h^T");
  DIT_FBWD(launch_gemm(1, TS, np, TB, dw2, F, D, F, (int)np, plain, s), "dW2");
  // h = gelu(a): da = dh * gelu'(a), in place
  DIT_FBWD(launch_gelu(1, A, F, DH, F, n_tokens, F, s), "gelu backward");
  if (db1)
    DIT_FBWD(launch_colsum(0, DH, F, nullptr, 0, nullptr, nullptr, n_tokens, F, PART, db1, 0, s),
             "db1");
  // a = y W1^T + b1: dy = da W1, dW1 = da^T y
  char* DY = ZD;
  DIT_FBWD(launch_transpose(w1, D, F, D, WT, F, s), "W1^T");
  DIT_FBWD(launch_gemm(1, DH, F, WT, DY, D, n_tokens, D, F, plain, s), "dy");
  DIT_FBWD(launch_transpose(DH, F, n_tokens, F, TB, np, s), "da^T");
  DIT_FBWD(launch_transpose(Y, D, n_tokens, D, TS, np, s), "y^T");
  DIT_FBWD(launch_gemm(1, TB, np, TS, dw1, D, F, D, (int)np, plain, s), "dW1");
  // AdaLN: dx, then the shift and scale rows
  DIT_FBWD(launch_adaln_bwd(x, D, DY, D, dout, D, modality, ada_table, dx, D, STATS, n_tokens, D,
                            d->ln_eps, s),
           "adaln backward");
  DIT_FBWD(launch_colsum(0, DY, D, nullptr, 0, nullptr, modality, n_tokens, D, PART, dtable,
                         3 * D, s),
           "shift rows");
  DIT_FBWD(launch_colsum(2, DY, D, x, D, STATS, modality, n_tokens, D, PART, dtable + D, 3 * D,
                         s),
           "scale rows");
#undef DIT_FBWD
  return DIT_OK;
}

// ---------------------------------------------------------------------------

extern "C" dit_status dit_profile_enable(int32_t max_calls) {
  clear_error();
  if (max_calls < 0) return fail(DIT_EINVAL, "dit_profile_enable: max_calls < 0");
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
  p.ev.clear();
  p.max_calls = 0;
  p.used = 0;
  if (max_calls == 0) return DIT_OK;
  p.ev.resize((size_t)max_calls * (DIT_NUM_STAGES + 1));
  for (auto& e : p.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      for (auto& e2 : p.ev)
        if (e2) (void)hipEventDestroy(e2);
      p.ev.clear();
      return hip_fail(r, "dit_profile_enable: hipEventCreate");
    }
  }
  p.max_calls = max_calls;
  return DIT_OK;
}

extern "C" dit_status dit_profile_read(float* stage_ms, int32_t* n_calls) {
  clear_error();
  if (!stage_ms || !n_calls) return fail(DIT_EINVAL, "dit_profile_read: null pointer");
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (int s = 0; s < DIT_NUM_STAGES; ++s) stage_ms[s] = 0.0f;
  for (int c = 0; c < p.used; ++c) {
    hipEvent_t* ev = &p.ev[(size_t)c * (DIT_NUM_STAGES + 1)];
    hipError_t r = hipEventSynchronize(ev[DIT_NUM_STAGES]);
    if (r != hipSuccess) return hip_fail(r, "dit_profile_read: hipEventSynchronize");
    for (int s = 0; s < DIT_NUM_STAGES; ++s) {
      float ms = 0.0f;
      r = hipEventElapsedTime(&ms, ev[s], ev[s + 1]);
      if (r != hipSuccess) return hip_fail(r, "dit_profile_read: hipEventElapsedTime");
      stage_ms[s] += ms;
    }
  }
  *n_calls = p.used;
  p.used = 0;
  return DIT_OK;
}
