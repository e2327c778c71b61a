// Softmax attention over a packed sequence, per cu_seqlens segment and head.
//
// [vLLM-Omni] section 3 "Packed Sequences and Modality Identity Preservation":
// the kernel takes its mask from cu_seqlens, so every query normalises only
// over keys of its own segment; section 1: audio and video share one
// attention context over the whole pack; section 6: rows past the effective
// length never enter the softmax.  Causal (key <= query inside the segment)
// is a variant ([VeRL-Omni] section 3 mentions causal attention).
//
// bf16 path (head_dim 128): flash-style forward on CDNA4 bf16 MFMA.
//   * Workgroup = 4 waves = 128 queries of one (segment, head); each wave owns
//     32 queries and walks the segment's keys in tiles of 64.
//   * The products are computed transposed, S^T = K Q^T and O^T = V^T P^T,
//     with v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane
//     then holds one query column and 16 key (or head-dim) rows, so the
//     softmax row max/sum is lane-local over 32 scores plus one exchange
//     between lanes l and l^32 (v_permlane32_swap), and the online-softmax
//     rescale of O is a per-lane scalar.
//   * Q stays in registers for the whole key loop.  K tiles ([key][d]) and
//     transposed V tiles ([d][key]) are double-buffered in LDS (64 KB per
//     workgroup, two workgroups per CU) with XOR-swizzled chunk indices; the
//     next tile's global loads are issued before the current tile's MFMAs.
//   * exp2 with log2(e) folded into the scale; P is rounded to bf16 for the
//     PV product; accumulation in float32.
//   * Masking (segment tail, causal diagonal) runs only on tiles that need
//     it; out-of-segment K/V rows are zero-filled, never read, so padding rows
//     holding NaN cannot leak in.  Causal launches longest q-tiles first.
//   * Grid = (q-tiles of the longest segment, segments, heads): consecutive
//     workgroups share one head's K/V, which stays hot in L2 / MALL.
//
// f32 path: one wave per (query, head), online softmax in float32 over key
// chunks of 64 (exactness for the small float32 workload, not speed).
#include <cmath>

#include "common.h"

namespace dit {
namespace {

constexpr int DH = 128;
constexpr int QB = 128;   // queries per workgroup
constexpr int KB = 64;    // keys per tile
constexpr int kThreads = 256;

// 32-bit word w (0..3) of a 16-byte vector.
__device__ __forceinline__ uint32_t word_of(const uint4& r, int w) {
  return w < 2 ? (w == 0 ? r.x : r.y) : (w == 2 ? r.z : r.w);
}

__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, int64_t ld_q, const uint16_t* __restrict__ k, int64_t ld_k,
    const uint16_t* __restrict__ v, int64_t ld_v, uint16_t* __restrict__ o, int64_t ld_o,
    const int32_t* __restrict__ cu, float scale_log2, int causal) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KB * DH];   // [key][d]
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][DH * KB];   // [d][key]

  const int h = blockIdx.z, seq = blockIdx.y;
  const int seg0 = cu[seq], seg1 = cu[seq + 1];
  const int nqt = (seg1 - seg0 + QB - 1) / QB;
  if ((int)blockIdx.x >= nqt) return;
  const int qt = causal ? nqt - 1 - (int)blockIdx.x : (int)blockIdx.x;
  const int q0 = seg0 + qt * QB;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const bool qvalid = qrow < seg1;

  // Q^T fragments (B operand of S^T = K Q^T): lane (query l32, half g) holds
  // d = 16*ks + 8*g .. +7.
  bf16x8 qf[DH / 16];
  {
    const uint16_t* qp = q + (int64_t)qrow * ld_q + h * DH + g * 8;
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks) {
      uint4 r = qvalid ? *reinterpret_cast<const uint4*>(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, r);
    }
  }

  const int kend = causal ? min(seg1, q0 + QB) : seg1;
  const int nkt = (kend - seg0 + KB - 1) / KB;

  // Staging: K tile = 64 rows x 16 chunks of 16 B (4 per thread); V tile =
  // thread (key quad kq = tid/16, d chunk tid%16) loads 4 keys x 8 d.
  uint4 rk[4], rv[4];
  const int vkq = tid >> 4, vd0 = (tid & 15) * 8;
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx >> 4, ch = idx & 15;
      const int key = kb + row;
      rk[i] = key < seg1 ? *reinterpret_cast<const uint4*>(k + (int64_t)key * ld_k + h * DH + ch * 8)
                         : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kb + vkq * 4 + i;
      rv[i] = key < seg1 ? *reinterpret_cast<const uint4*>(v + (int64_t)key * ld_v + h * DH + vd0)
                         : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx >> 4, ch = idx & 15;
      *reinterpret_cast<uint4*>(&Ks[buf][row * DH + ((ch ^ (row & 7)) * 8)]) = rk[i];
    }
    // transpose 4 keys x 8 d into 8 rows of V^T, 4 keys (8 bytes) each
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int sh = (dd & 1) * 16;
      const uint32_t a0 = (word_of(rv[0], dd >> 1) >> sh) & 0xffffu;
      const uint32_t a1 = (word_of(rv[1], dd >> 1) >> sh) & 0xffffu;
      const uint32_t a2 = (word_of(rv[2], dd >> 1) >> sh) & 0xffffu;
      const uint32_t a3 = (word_of(rv[3], dd >> 1) >> sh) & 0xffffu;
      const int row = vd0 + dd;
      const int chunk = vkq ^ (row & 15);
      *reinterpret_cast<uint2*>(&Vt[buf][row * KB + chunk * 4]) =
          make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 oacc[DH / 32];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;

  gload(seg0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int buf = j & 1;
    const int kb = seg0 + j * KB;
    if (j + 1 < nkt) gload(kb + KB);

    // S^T[key][query] for the tile's 64 keys: two 32-key blocks.
    f32x16 sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[b][e] = 0.0f;
      const int krow = 32 * b + l32;
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            &Ks[buf][krow * DH + (((2 * ks + g) ^ (krow & 7)) * 8)]);
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[b], 0, 0, 0);
      }
    }

    // Element e of block b is key kb + 32b + (e/4)*8 + 4g + e%4.
    const bool need_mask = (kb + KB > seg1) || (causal && kb + KB - 1 > qw0);
    if (need_mask) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb + 32 * b + (e >> 2) * 8 + g * 4 + (e & 3);
          if (key >= seg1 || (causal && key > qrow)) sacc[b][e] = -INFINITY;
        }
    }

    float mx = sacc[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[b][e]);
    mx = half_swap_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * scale_log2);
    const float nms = -m_use * scale_log2;
    float rs = 0.0f;
    bf16x8 pf[4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[b][e], scale_log2, nms));
        rs += p;
        pf[2 * b + (e >> 3)][e & 7] = (__bf16)p;
      }
    l_run = fmaf(l_run, alpha, rs);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;

    // O^T += V^T P^T.  Step s covers S^T block b = s/2, elements 8(s%2)..+7,
    // i.e. keys base..base+3 and base+8..base+11 with base = 32b + 16(s%2) + 4g.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c1 = 8 * (s >> 1) + 4 * (s & 1) + g;   // 8-byte chunk (4 keys)
      const int c2 = c1 + 2;
#pragma unroll
      for (int db = 0; db < DH / 32; ++db) {
        const int drow = 32 * db + l32;
        const uint2 lo = *reinterpret_cast<const uint2*>(&Vt[buf][drow * KB + ((c1 ^ (drow & 15)) * 4)]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&Vt[buf][drow * KB + ((c2 ^ (drow & 15)) * 4)]);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s], oacc[db], 0, 0, 0);
      }
    }

    if (j + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = half_swap_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    uint16_t* op = o + (int64_t)qrow * ld_o + h * DH;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d = 32 * db + qd * 8 + g * 4;
        const uint2 w = make_uint2(pack_bf16x2(oacc[db][4 * qd + 0] * inv, oacc[db][4 * qd + 1] * inv),
                                   pack_bf16x2(oacc[db][4 * qd + 2] * inv, oacc[db][4 * qd + 3] * inv));
        *reinterpret_cast<uint2*>(op + d) = w;
      }
  }
}

// ---- float32 path: one wave per (query, head) ----
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ q, int64_t ld_q,
                                                      const float* __restrict__ k, int64_t ld_k,
                                                      const float* __restrict__ v, int64_t ld_v,
                                                      float* __restrict__ o, int64_t ld_o,
                                                      const int32_t* __restrict__ cu, int n_seqs,
                                                      float scale, int causal) {
  constexpr int PER = D / 64;
  __shared__ float qs[D];
  const int row = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  // segment of this row: last s with cu[s] <= row
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int seg0 = cu[lo], seg1 = cu[lo + 1];
  const int kend = causal ? row + 1 : seg1;
  for (int d = lane; d < D; d += 64) qs[d] = q[(int64_t)row * ld_q + h * D + d];
  __syncthreads();

  float m = -INFINITY, l = 0.0f, acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  for (int kb = seg0; kb < kend; kb += 64) {
    const int key = kb + lane;
    float sc = -INFINITY;
    if (key < kend) {
      const float* kr = k + (int64_t)key * ld_k + h * D;
      float dot = 0.0f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], kr[d], dot);
      sc = dot * scale;
    }
    const float mx = wave_max(sc);
    const float m_new = fmaxf(m, mx);
    const float alpha = expf(m - m_new);
    const float p = key < kend ? expf(sc - m_new) : 0.0f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] *= alpha;
    const int cnt = min(64, kend - kb);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pj = __shfl(p, jj, 64);
      const float* vr = v + (int64_t)(kb + jj) * ld_v + h * D;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(pj, vr[lane + 64 * i], acc[i]);
    }
    m = m_new;
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[(int64_t)row * ld_o + h * D + lane + 64 * i] = acc[i] * inv;
}

}  // namespace

hipError_t launch_attn(int bf16, const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                       const void* v, int64_t ld_v, void* o, int64_t ld_o, const int32_t* cu,
                       int n_seqs, int max_seqlen, int64_t n_tokens, int n_heads, int head_dim,
                       float scale, int causal, hipStream_t s) {
  if (n_seqs > 65535 || n_heads > 65535 || n_tokens > INT32_MAX) return hipErrorInvalidValue;
  if (bf16) {
    if (head_dim != DH) return hipErrorInvalidValue;
    const dim3 grid((max_seqlen + QB - 1) / QB, n_seqs, n_heads);
    attn_bf16_kernel<<<grid, dim3(kThreads), 0, s>>>(
        static_cast<const uint16_t*>(q), ld_q, static_cast<const uint16_t*>(k), ld_k,
        static_cast<const uint16_t*>(v), ld_v, static_cast<uint16_t*>(o), ld_o, cu,
        scale * 1.4426950408889634f, causal);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)n_tokens, n_heads);
  const float* qf = static_cast<const float*>(q);
  const float* kf = static_cast<const float*>(k);
  const float* vf = static_cast<const float*>(v);
  float* of = static_cast<float*>(o);
  if (head_dim == 64)
    attn_f32_kernel<64><<<grid, dim3(64), 0, s>>>(qf, ld_q, kf, ld_k, vf, ld_v, of, ld_o, cu,
                                                  n_seqs, scale, causal);
  else if (head_dim == 128)
    attn_f32_kernel<128><<<grid, dim3(64), 0, s>>>(qf, ld_q, kf, ld_k, vf, ld_v, of, ld_o, cu,
                                                   n_seqs, scale, causal);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dit
