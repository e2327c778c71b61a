// Internal helpers shared by the libdit kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte global access (non-temporal hint) for data touched once:
// rows that are read or written exactly once per launch should not displace
// reused lines (tables, weights) from the caches.
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void* p, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, static_cast<u32x4*>(p));
}

// bf16 storage is raw 16-bit patterns; widening is exact.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
  return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// Sum / max over all 64 lanes of a wave (result in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Value pair {v[l], v[l ^ 32]} via v_permlane32_swap; combining the two
// results with a commutative op gives the same value in lanes l and l ^ 32.
__device__ __forceinline__ float half_swap_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// tanh-form GELU: 0.5 z (1 + tanh u) with u = sqrt(2/pi) (z + 0.044715 z^3),
// evaluated as z / (1 + exp(-2u)) (the same function; one exp and one
// reciprocal).  Large |z| saturate to z and -0.
__device__ __forceinline__ float gelu_tanh_fast(float z) {
  const float u2 = 1.5957691216057308f * fmaf(0.044715f * z, z * z, z);   // 2u
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-u2));
}
__device__ __forceinline__ float gelu_tanh_exact(float z) {
  const float u2 = 1.5957691216057308f * fmaf(0.044715f * z, z * z, z);
  return z / (1.0f + expf(-u2));
}

// Four e4m3 codes of four float32 values in one word (value j in byte j):
// nearest, ties to the even code (v_cvt_pk_fp8_f32, which rounds exactly so
// for |v| <= 464: checked against the float64 oracle on every code, every
// midpoint and its float32 neighbours and 2e5 random values), saturating at
// +-448 (the conversion gives NaN beyond 464, so values are clamped first),
// NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_pack4(float f0, float f1, float f2, float f3) {
  auto clamp = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(f0), clamp(f1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(f2), clamp(f3), w, true);
  uint32_t u = (uint32_t)w;
  if (__builtin_isnan(f0) | __builtin_isnan(f1) | __builtin_isnan(f2) | __builtin_isnan(f3)) {
    if (__builtin_isnan(f0)) u = (u & 0xffffff00u) | 0x7fu;
    if (__builtin_isnan(f1)) u = (u & 0xffff00ffu) | 0x7f00u;
    if (__builtin_isnan(f2)) u = (u & 0xff00ffffu) | 0x7f0000u;
    if (__builtin_isnan(f3)) u = (u & 0x00ffffffu) | 0x7f000000u;
  }
  return u;
}

// Rows [r0, r1) of a bf16 [n_rows][ld] array, columns [col0, col0 + ncols)
// (ncols a multiple of 8, 16-byte aligned), set to NaN, clamped to
// [0, n_rows): the workgroups part = 0 .. parts-1 of one launch share the rows.
// The attention kernels' answer to a segment longer than the max_seqlen their
// grid was sized for: its rows become NaN instead of being left unwritten.
__device__ __forceinline__ void poison_rows_bf16(uint16_t* a, int64_t ld, int col0, int ncols,
                                                 int64_t r0, int64_t r1, int64_t n_rows,
                                                 int part, int parts) {
  const int64_t lo = r0 < 0 ? 0 : r0, hi = r1 > n_rows ? n_rows : r1;
  const int vpr = ncols / 8;
  const uint4 nan4 = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
  for (int64_t i = (int64_t)part * blockDim.x + threadIdx.x; lo + i / vpr < hi;
       i += (int64_t)parts * blockDim.x) {
    const int64_t row = lo + i / vpr;
    const int c = (int)(i % vpr);
    *reinterpret_cast<uint4*>(a + row * ld + col0 + 8 * c) = nan4;
  }
}

}  // namespace dit

// Launchers implemented in the .hip files; all return hipGetLastError() of the launch.
namespace dit {

hipError_t launch_adaln(int bf16, const void* x, int64_t ld_x, const uint8_t* mod,
                        const float* table, void* y, int64_t ld_y, int64_t n, int d,
                        float eps, hipStream_t s);

// freq_d: host array of head_dim/2 pair frequencies theta^(-2j/s_axis), in double.
// Rotates q into q_out and k into k_out (k, k_out null: q only); in place when
// the outputs are the inputs; k_out may be q (each vector is loaded before the
// same thread stores over it).
hipError_t launch_rope(int bf16, const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                       void* q_out, int64_t ld_qo, void* k_out, int64_t ld_ko,
                       const int32_t* pos, int64_t n, int n_heads, int head_dim,
                       int s_t, int s_h, const double* freq_d, hipStream_t s);

// lse (bf16 only, may be null): float [n_heads][n_tokens], the natural
// log-sum-exp of each row's scaled scores.
hipError_t launch_attn(int bf16, const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                       const void* v, int64_t ld_v, void* o, int64_t ld_o,
                       const int32_t* cu, int n_seqs, int max_seqlen, int64_t n_tokens,
                       int n_heads, int head_dim, float scale, int causal, float* lse,
                       hipStream_t s);

// FP8 attention operands (head_dim 128): e4m3 codes of q and k [token][head][128]
// (ld8 bytes per token), q's per-row scales sq [head][token], the per-head
// scales sk, sv, and v's codes transposed to vt [head][d][column] (ld_vt bytes
// per d row; segment s starts at column roundup64(cu[s]) + 128 s).  amax:
// [2][head] scratch.
struct AttnFp8Ops {
  uint8_t* q8;
  uint8_t* k8;
  uint8_t* vt;
  float* sq;
  float* sk;
  float* sv;
  uint32_t* amax;
  int64_t ld8;
  int64_t ld_vt;
};
// q, k, v bf16 [token][head][128] (row strides in elements) -> ops.
hipError_t launch_attn_fp8_prepare(const uint16_t* q, int64_t ld_q, const uint16_t* k,
                                   int64_t ld_k, const uint16_t* v, int64_t ld_v,
                                   const int32_t* cu, int n_seqs, int max_seqlen,
                                   int64_t n_tokens, int n_heads, const AttnFp8Ops& ops,
                                   hipStream_t s);
// o bf16 [token][head][128] from prepared operands.
hipError_t launch_attn_fp8(const AttnFp8Ops& ops, uint16_t* o, int64_t ld_o, const int32_t* cu,
                           int n_seqs, int max_seqlen, int64_t n_tokens, int n_heads, float scale,
                           int causal, hipStream_t s);

// Attention backward (bf16, head_dim 128): delta[h][row] = sum_d do * o, then
// dk, dv (one pass over the queries per key block) and dq (one pass over the
// keys per query block), recomputing P = exp(s scale - lse).  delta: float
// [n_heads][n_tokens] scratch.
hipError_t launch_attn_bwd(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                           const void* v, int64_t ld_v, const void* o, int64_t ld_o,
                           const void* dout, int64_t ld_do, const float* lse, void* dq,
                           int64_t ld_dq, void* dk, int64_t ld_dk, void* dv, int64_t ld_dv,
                           const int32_t* cu, int n_seqs, int max_seqlen, int64_t n_tokens,
                           int n_heads, float scale, int causal, float* delta, hipStream_t s);

// C = A B^T (+ bias), A [M][K], B [N][K]; epilogue 0: store C; 1: gated residual
// out = x + table[mod][GATE] * C; 2: store gelu_tanh(C).
// Planes (kinds 0 and 3): with plane_cols > 0, output column j goes to plane
// j / plane_cols, column j % plane_cols, planes plane_stride elements apart
// (row stride ldc inside a plane); plane_cols must be a multiple of 32.
// Kind 3 (bf16 only) is kind 0 with the 3D rotary embedding applied to planes
// 0 and 1 (q and k) before the store: pos [M][3] (t, h, w) per row, rope_freq
// the rope_dh / 2 pair frequencies (rope_freqs), pairs below rope_pair_h on
// the t axis, below rope_pair_w on h, the rest on w; plane_cols and n must be
// multiples of rope_dh (64 or 128).
struct GemmEpilogue {
  int kind;                 // 0 plain, 1 gated residual, 2 GELU, 3 planes + RoPE
  const void* bias;         // [N] or null
  const void* x;            // residual input (kind 1)
  int64_t ld_x;
  const uint8_t* mod;       // modality ids (kind 1)
  const float* gate;        // table + GATE row offset; row stride 3*N floats (kind 1)
  int plane_cols = 0;       // 0: one [M][ldc] output
  int64_t plane_stride = 0;
  const int32_t* pos = nullptr;       // kind 3
  const double* rope_freq = nullptr;  // kind 3: [rope_dh / 2], host memory
  int rope_dh = 0;                    // kind 3: head_dim, 64 or 128
  int rope_pair_h = 0, rope_pair_w = 0;
};
hipError_t launch_gemm(int bf16, const void* a, int64_t lda, const void* b, void* c,
                       int64_t ldc, int64_t m, int n, int k, const GemmEpilogue& ep,
                       hipStream_t s);

// FP8 projection: a, w e4m3 codes [m][k] / [n][k] (row strides lda, k bytes),
// sa [m], sw [n] float32 row scales; c bf16; epilogues as launch_gemm.
hipError_t launch_gemm_fp8(const uint8_t* a, int64_t lda, const float* sa, const uint8_t* w,
                           const float* sw, void* c, int64_t ldc, int64_t m, int n, int k,
                           const GemmEpilogue& ep, hipStream_t s);
// Per-row e4m3 quantization of bf16 (or float32) rows: codes [n][ld_q], scales [n].
// launch_adaln_fp8: AdaLN whose output is written as such codes and scales.
hipError_t launch_adaln_fp8(int bf16, const void* x, int64_t ld_x, const uint8_t* mod,
                            const float* table, uint8_t* q, int64_t ld_q, float* scales,
                            int64_t n, int d, float eps, hipStream_t s);
hipError_t launch_quant_rows_fp8(int bf16, const void* x, int64_t ld_x, uint8_t* q, int64_t ld_q,
                                 float* scales, int64_t n, int d, hipStream_t s);

// Workspace of launch_nft_loss: a loss-bearing row count per sample (int32)
// and two squared-error sums (float) per (sample, 32-row chunk), each region
// 256-byte aligned.
size_t nft_workspace_layout(int n_samples, int max_rows, size_t* partials_offset);
hipError_t launch_nft_loss(int bf16, const void* v_theta, int64_t ld_vt, const void* v_old,
                           int64_t ld_vo, const float* v_target, int64_t ld_t,
                           const uint8_t* mask, const int32_t* cu, int n_samples, int max_rows,
                           int channels, const float* reward, float beta, float sign,
                           float scale, float* grad, int64_t ld_g, float* loss_out,
                           void* workspace, hipStream_t s);

// Backward-pass helpers (bf16).  Transpose: dst [cols][ld_dst] = src^T, zero
// in columns rows..ld_dst-1; cols, ld_dst multiples of 64.
hipError_t launch_transpose(const void* src, int64_t ld_src, int64_t rows, int cols, void* dst,
                            int64_t ld_dst, hipStream_t s);
// out = table[mod][GATE] * g (row-wise), d a multiple of 8.
hipError_t launch_gate_scale(const void* g, int64_t ld_g, const uint8_t* mod, const float* table,
                             void* out, int64_t ld_out, int64_t n, int d, hipStream_t s);
// io = gelu(a), or (backward) io = io * gelu'(a); [n][f] bf16, f a multiple of 8.
hipError_t launch_gelu(int backward, const void* a, int64_t lda, void* io, int64_t ld_io,
                       int64_t n, int f, hipStream_t s);
// Column sums over n rows (deterministic): mode 0 sums a, 1 a * b, 2
// a * (b - mean) * rstd with stats float2 [n] (mean, rstd); per modality into
// out[m * out_gstride + j] (m = 0..2) when mod is given, else into out[j].
// partial: colsum_partial_bytes(n, c, groups) bytes of scratch.
constexpr int kColsumRows = 256;
size_t colsum_partial_bytes(int64_t n, int c, int groups);
hipError_t launch_colsum(int mode, const void* a, int64_t lda, const void* b, int64_t ldb,
                         const float* stats, const uint8_t* mod, int64_t n, int c, float* partial,
                         float* out, int64_t out_gstride, hipStream_t s);
// AdaLN backward: dx = dres + rstd (dxh - mean(dxh) - xhat mean(dxh xhat)) with
// dxh = dy (1 + table[mod][SCALE]); stats float2 [n] (mean, rstd) out.
// dx may be dres.
hipError_t launch_adaln_bwd(const void* x, int64_t ld_x, const void* dy, int64_t ld_dy,
                            const void* dres, int64_t ld_dres, const uint8_t* mod,
                            const float* table, void* dx, int64_t ld_dx, float* stats, int64_t n,
                            int d, float eps, hipStream_t s);

// sigmas: host {video, video_next, audio, audio_next}; sign +1 or -1.
hipError_t launch_denoise(int bf16, float* z, int64_t ld_z, const void* v, int64_t ld_v,
                          float* x0, int64_t ld_x0, const uint8_t* mod, const uint8_t* anchor,
                          const float* anchor_vals, int64_t ld_a, int64_t n_rows, int channels,
                          const float sigmas[4], float sign, hipStream_t s);

}  // namespace dit
