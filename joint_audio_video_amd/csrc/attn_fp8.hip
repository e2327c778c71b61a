// Packed softmax attention with FP8 (e4m3) products, head_dim 128.
//
// [vLLM-Omni] section 5 ("Distributed Layerwise Offload") runs the active DiT
// layers in FP8 and gives no scaling recipe; the attention of [vLLM-Omni]
// section 3 (cu_seqlens segments, full or causal) is the operation.  Reading:
// q carries one float32 scale per (token, head) row, k and v one per
// (segment, head) (amax / 448 over the segment's tokens of the head; the
// requests of a pack are independent, so one request's codes do not depend on
// the others'), so every scale factors out of its product: q's and k's out of
// s = q k^T, v's out of o = P v (a sum over one segment's keys).  Scores, softmax and the output stay float32; the probabilities
// enter the second product as e4m3 codes of 2^8 times their value relative to
// the row's running maximum (at most 2^8.75 < 448, so no code saturates).
//
// Operand preparation (four small launches, all HBM-bound):
//   * seg_amax_kernel: amax |k| and |v| per (segment, head) (a block max over
//     256 of the segment's rows, then one vector atomic max per block on the
//     float bits, which order like unsigned integers for non-negative values).
//   * seg_scale_kernel: the scales amax / 448 (1 for zero).
//   * quant_qk_kernel: q codes with per-row scales, k codes with the scale of
//     the row's segment; sixteen lanes per (token, head) row.
//   * quant_vt_kernel: v codes transposed to [head][d][key] through LDS, so
//     that a V^T fragment is a plain row read.  Segment s occupies columns
//     from vt_col0 = roundup64(cu[s]) + 128 s (aligned; the tile ends and the
//     gaps between segments never overlap), its last tile zero-padded.
//
// attn_fp8_kernel: the bf16 kernel's organisation with FP8 operands.  A
// workgroup owns 384 queries of one (segment, head), 12 waves of 32 (three
// per SIMD: the FP8 products leave the matrix pipe idle more often, so more
// waves hide the latency; 168 registers each); Q codes
// stay in registers, K tiles [64 keys][128 B] and V^T tiles [128 d][64 B]
// are double-buffered in LDS (32 KB), filled by buffer loads that write
// straight into LDS.  Per 64-key tile a wave issues 8
// v_mfma_scale_f32_32x32x64_f8f6f4 (S^T = K Q^T: two key blocks x two
// 64-deep d steps; O^T += V^T P^T: four d blocks x one 64-key step).  The
// probabilities leave the S^T accumulators as four e4m3 words per key block
// per lane; one v_permlane32_swap per word pair hands each lane half the 32
// consecutive keys the B operand of the second product expects.  Waves 4-7
// (the middle wave of each SIMD) run half a phase behind the others
// (ping-pong), as in the bf16 kernel.
#include <cmath>

#include "common.h"

namespace dit {
namespace {

constexpr int DH = 128;
constexpr int KB = 64;                    // keys per tile
// Waves per workgroup: 12 (three per SIMD; measured 2-9% faster than 8, two
// per SIMD, across one segment, four segments and causal).
#ifndef DIT_ATTN_FP8_WAVES
#define DIT_ATTN_FP8_WAVES 12
#endif
constexpr int kWaves = DIT_ATTN_FP8_WAVES;
static_assert(kWaves == 8 || kWaves == 12, "8 or 12 waves per workgroup");
constexpr int kThreads = 64 * kWaves;
constexpr int QBLK = 32 * kWaves;         // queries per workgroup
// A tile may exceed the running maximum by this much (log2 units) before the
// maximum moves: probabilities times 2^8 then stay below 2^8.75 < 448.
constexpr float kSlack = 0.75f;
constexpr float kPScale = 8.0f;           // log2 of the probability scale
typedef int v8i32 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ int vt_col0(int seg0, int s) { return ((seg0 + 63) & ~63) + 128 * s; }

__device__ __forceinline__ v8i32 cat8(const uint4& a, const uint4& b) {
  return v8i32{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// ---- operand preparation ----

__global__ void zero_u32_kernel(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// amax[(z * n_seqs + s) * n_heads + h] = max |x| over the head's columns of
// segment s's rows [seg0 + 256 bx, +256), combined over blocks; blockIdx.y = s,
// blockIdx.z = 2 h + z with z = 0: k, 1: v.
__global__ __launch_bounds__(256) void seg_amax_kernel(const uint16_t* __restrict__ k,
                                                       int64_t ld_k,
                                                       const uint16_t* __restrict__ v,
                                                       int64_t ld_v, const int32_t* __restrict__ cu,
                                                       int n_seqs, int n_heads,
                                                       uint32_t* __restrict__ amax) {
  const int s = blockIdx.y, h = blockIdx.z >> 1, z = blockIdx.z & 1, tid = threadIdx.x;
  const int seg0 = cu[s], seg1 = cu[s + 1];
  const int64_t r0 = (int64_t)seg0 + (int64_t)blockIdx.x * 256;
  if (r0 >= seg1) return;
  const uint16_t* src = z ? v : k;
  const int64_t ld = z ? ld_v : ld_k;
  float m = 0.0f;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int64_t r = r0 + 16 * i + (tid >> 4);
    if (r < seg1) {
      const uint4 w = ld_stream(src + r * ld + h * DH + 8 * (tid & 15));
      m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16lo(w.x)), fabsf(bf16hi(w.x))),
                         fmaxf(fabsf(bf16lo(w.y)), fabsf(bf16hi(w.y)))));
      m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16lo(w.z)), fabsf(bf16hi(w.z))),
                         fmaxf(fabsf(bf16lo(w.w)), fabsf(bf16hi(w.w)))));
    }
  }
  m = wave_max(m);
  __shared__ float red[4];
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    const float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(amax + ((int64_t)z * n_seqs + s) * n_heads + h, __float_as_uint(a));
  }
}

// sk[s * n_heads + h], sv[...] = amax / 448 (1 for zero) of k's and v's blocks.
__global__ void seg_scale_kernel(const uint32_t* __restrict__ amax, float* __restrict__ sk,
                                 float* __restrict__ sv, int count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 2 * count) return;
  const float a = __uint_as_float(amax[i]);
  const float s = a > 0.0f ? a / 448.0f : 1.0f;
  if (i < count) sk[i] = s;
  else sv[i - count] = s;
}

// Row (token, head) = 16 lanes x 8 values.  blockIdx.y = 0: q (own scale,
// written to sq[h][token]), 1: k (the scale of the token's segment, the last
// s with cu[s] <= token).
__global__ __launch_bounds__(256) void quant_qk_kernel(
    const uint16_t* __restrict__ q, int64_t ld_q, const uint16_t* __restrict__ k, int64_t ld_k,
    int n, int n_heads, const int32_t* __restrict__ cu, int n_seqs,
    const float* __restrict__ sk, uint8_t* __restrict__ q8, uint8_t* __restrict__ k8,
    int64_t ld8, float* __restrict__ sq) {
  const int row = (int)(((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4);
  const int c = threadIdx.x & 15;
  const bool live = row < n * n_heads;      // the same for the 16 lanes of a row
  const int tok = row / n_heads, h = row - tok * n_heads;
  const bool isk = blockIdx.y == 1;
  float x[8];
  if (live) {
    const uint16_t* src = isk ? k + (int64_t)tok * ld_k : q + (int64_t)tok * ld_q;
    const uint4 w = ld_stream(src + h * DH + 8 * c);
    x[0] = bf16lo(w.x); x[1] = bf16hi(w.x); x[2] = bf16lo(w.y); x[3] = bf16hi(w.y);
    x[4] = bf16lo(w.z); x[5] = bf16hi(w.z); x[6] = bf16lo(w.w); x[7] = bf16hi(w.w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.0f;
  }
  float inv;
  if (!isk) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    const float sc = a > 0.0f ? a / 448.0f : 1.0f;
    inv = 1.0f / sc;
    if (live && c == 0) sq[(int64_t)h * n + tok] = sc;
  } else {
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= tok) lo = mid;
      else hi = mid - 1;
    }
    inv = 1.0f / sk[lo * n_heads + h];
  }
  if (live) {
    const uint2 w = make_uint2(e4m3_pack4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv),
                               e4m3_pack4(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv));
    *reinterpret_cast<uint2*>((isk ? k8 : q8) + (int64_t)tok * ld8 + h * DH + 8 * c) = w;
  }
}

// One 64-key tile of segment blockIdx.y, head blockIdx.z: codes with the
// (segment, head) scale, written transposed (d rows of 64 key bytes); keys
// past the segment end are zero codes.
__global__ __launch_bounds__(256) void quant_vt_kernel(const uint16_t* __restrict__ v,
                                                       int64_t ld_v,
                                                       const int32_t* __restrict__ cu,
                                                       const float* __restrict__ sv,
                                                       uint8_t* __restrict__ vt, int64_t ld_vt) {
  __shared__ __attribute__((aligned(16))) uint8_t T[DH][KB + 4];   // [d][key], 68-byte rows
  const int j = blockIdx.x, s = blockIdx.y, h = blockIdx.z, tid = threadIdx.x;
  const int seg0 = cu[s], seg1 = cu[s + 1];
  if (j * KB >= seg1 - seg0) return;
  const float inv = 1.0f / sv[s * gridDim.z + h];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cidx = tid + 256 * i;         // key row cidx / 16, d chunk cidx % 16
    const int r = cidx >> 4, cc = cidx & 15;
    const int key = seg0 + j * KB + r;
    uint32_t w0 = 0u, w1 = 0u;
    if (key < seg1) {
      const uint4 w = ld_stream(v + (int64_t)key * ld_v + h * DH + 8 * cc);
      w0 = e4m3_pack4(bf16lo(w.x) * inv, bf16hi(w.x) * inv, bf16lo(w.y) * inv, bf16hi(w.y) * inv);
      w1 = e4m3_pack4(bf16lo(w.z) * inv, bf16hi(w.z) * inv, bf16lo(w.w) * inv, bf16hi(w.w) * inv);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      T[8 * cc + x][r] = (uint8_t)(w0 >> (8 * x));
      T[8 * cc + 4 + x][r] = (uint8_t)(w1 >> (8 * x));
    }
  }
  __syncthreads();
  uint8_t* dst = vt + (int64_t)h * DH * ld_vt + vt_col0(seg0, s) + j * KB;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int cidx = tid + 256 * i;         // d row cidx / 4, 16-key chunk cidx % 4
    const int d = cidx >> 2, kc = cidx & 3;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&T[d][16 * kc]);
    *reinterpret_cast<uint4*>(dst + (int64_t)d * ld_vt + 16 * kc) =
        make_uint4(src[0], src[1], src[2], src[3]);
  }
}

// ---- attention ----

__global__ __launch_bounds__(kThreads, kWaves / 4) void attn_fp8_kernel(
    const uint8_t* __restrict__ q8, int64_t ld_q8, const float* __restrict__ sq, int64_t ld_sq,
    const uint8_t* __restrict__ k8, int64_t ld_k8, const float* __restrict__ sk,
    const uint8_t* __restrict__ vt, int64_t ld_vt, const float* __restrict__ sv,
    uint16_t* __restrict__ o, int64_t ld_o, const int32_t* __restrict__ cu, float scale_log2,
    int causal, int max_seqlen, int64_t n_tokens) {
  __shared__ __attribute__((aligned(16))) uint8_t Ks0[KB * DH];
  __shared__ __attribute__((aligned(16))) uint8_t Ks1[KB * DH];
  __shared__ __attribute__((aligned(16))) uint8_t Vs0[DH * KB];
  __shared__ __attribute__((aligned(16))) uint8_t Vs1[DH * KB];

  const int h = blockIdx.z, seq = blockIdx.y;
  const int seg0 = cu[seq], seg1 = cu[seq + 1];
  if (seg1 - seg0 > max_seqlen) {
    // a segment longer than max_seqlen (cu_seqlens breaks its contract): the
    // grid and the operand preparation do not cover it; its rows become NaN
    poison_rows_bf16(o, ld_o, h * DH, DH, seg0, seg1, n_tokens, blockIdx.x, gridDim.x);
    return;
  }
  const int nqt = (seg1 - seg0 + QBLK - 1) / QBLK;
  if ((int)blockIdx.x >= nqt) return;
  const int qt = causal ? nqt - 1 - (int)blockIdx.x : (int)blockIdx.x;
  const int q0 = seg0 + qt * QBLK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int l32 = lane & 31, g = lane >> 5;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const bool qlive = qrow < seg1;

  // Q^T codes (B operand of S^T = K Q^T): lane (query l32, half g) holds
  // d = 64 ks + 32 g .. +31.
  v8i32 qf[2];
  {
    const uint8_t* qp = q8 + (int64_t)qrow * ld_q8 + h * DH + 32 * g;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 a = qlive ? *reinterpret_cast<const uint4*>(qp + 64 * ks) : make_uint4(0, 0, 0, 0);
      const uint4 b = qlive ? *reinterpret_cast<const uint4*>(qp + 64 * ks + 16) : make_uint4(0, 0, 0, 0);
      qf[ks] = cat8(a, b);
    }
  }
  // S^T holds code products; times q's row scale, k's head scale and the
  // softmax scale (log2 units) it is the exponent.  One factor per lane.
  const int sh = seq * (int)gridDim.z + h;     // this (segment, head)'s k and v scales
  const float cq = scale_log2 * (qlive ? sq[(int64_t)h * ld_sq + qrow] : 1.0f) * sk[sh];
  const float vscale = sv[sh];

  const int kend = causal ? min(seg1, q0 + QBLK) : seg1;
  const int nkt = (kend - seg0 + KB - 1) / KB;

  // Global -> LDS, 16 bytes per lane, 1 KB (64 slots) per wave and load: slot
  // s of a K tile is key row s/8, physical chunk s%8 holding logical chunk
  // (s%8) ^ ((row >> 1) & 7); of a V^T tile d row s/4, physical chunk s%4
  // holding (s%4) ^ ((d >> 2) & 3).  With 8 waves wave w loads K and V slots
  // 64w..64w+63; with 12, waves 0-7 load K and waves 8-11 two kilobytes of V.
  // With 64 four-byte banks a fragment read (16 consecutive rows per cycle)
  // then touches 16 distinct 16-byte slots.  K rows past the segment end lie
  // outside the buffer range and arrive as zeros; V^T columns past it are
  // zero codes.
  const uint32_t seg_rows = (uint32_t)(seg1 - seg0);
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(k8 + (int64_t)seg0 * ld_k8 + h * DH, seg_rows * (uint32_t)ld_k8);
  const int col0 = vt_col0(seg0, seq);
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(vt + (int64_t)h * DH * ld_vt + col0, (uint32_t)(DH * ld_vt - col0));
  constexpr int kVLoads = kWaves == 8 ? 1 : 2;         // V loads per V-loading wave
  const bool k_loader = wave < 8;
  const bool v_loader = kWaves == 8 || wave >= 8;
  const int kslot = 64 * wave + lane;                   // K: waves 0-7
  const int vbase = kWaves == 8 ? 64 * wave : 128 * (wave - 8);
  const int krow = kslot >> 3;
  const uint32_t koff = (uint32_t)krow * (uint32_t)ld_k8 + (uint32_t)(((kslot & 7) ^ ((krow >> 1) & 7)) * 16);
  uint32_t voff[kVLoads];
#pragma unroll
  for (int i = 0; i < kVLoads; ++i) {
    const int vslot = vbase + 64 * i + lane;
    const int vrow = vslot >> 2;
    voff[i] = (uint32_t)vrow * (uint32_t)ld_vt + (uint32_t)(((vslot & 3) ^ ((vrow >> 2) & 3)) * 16);
  }
  const uint32_t k_tstep = (uint32_t)KB * (uint32_t)ld_k8;
  auto issue_k = [&](uint8_t* dst, int tile) {
    if (k_loader)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, dst + 64 * wave * 16, 16, koff,
                                               (int)(tile * k_tstep), 0, 0);
  };
  auto issue_v = [&](uint8_t* dst, int tile) {
    if (v_loader) {
#pragma unroll
      for (int i = 0; i < kVLoads; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, dst + (vbase + 64 * i) * 16, 16, voff[i],
                                                 tile * KB, 0, 0);
    }
  };

  // Fragment byte offsets.  K (A of S^T): lane (key 32 b + l32, half g) reads
  // logical chunks 4 ks + 2 g + x (x = 0, 1) of its row.  V^T (A of O^T):
  // lane (d = 32 db + l32, half g) reads chunks 2 g + x of its row, keys
  // 32 g .. +31.  Block b / d block db only add a constant.
  int kofs[2][2], vofs[2];
  {
    const int ksw = (l32 >> 1) & 7, vsw = (l32 >> 2) & 3;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int x = 0; x < 2; ++x) kofs[ks][x] = l32 * DH + 16 * ((4 * ks + 2 * g + x) ^ ksw);
#pragma unroll
    for (int x = 0; x < 2; ++x) vofs[x] = l32 * KB + 16 * ((2 * g + x) ^ vsw);
  }
  auto kfrag = [&](const uint8_t* t, int b, int ks) {
    return cat8(*reinterpret_cast<const uint4*>(t + 4096 * b + kofs[ks][0]),
                *reinterpret_cast<const uint4*>(t + 4096 * b + kofs[ks][1]));
  };
  auto vfrag = [&](const uint8_t* t, int db) {
    return cat8(*reinterpret_cast<const uint4*>(t + 2048 * db + vofs[0]),
                *reinterpret_cast<const uint4*>(t + 2048 * db + vofs[1]));
  };

  float m_run = -INFINITY, l_run = 0.0f;    // m_run: running max of score * cq
  f32x16 oacc[DH / 32];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
  const f32x16 zero16 = {};
  f32x16 sacc[2];
  v8i32 pf;

  // S^T[key][query] of one tile: element e of block b is key
  // 32 b + 8 (e / 4) + 4 g + e % 4 of the tile, column query l32.
  // With three waves per SIMD the fragments of one d step (both key blocks)
  // are in flight at a time; the second step's reads follow the first step's
  // MFMAs.
  auto compute_s = [&](const uint8_t* ks_t) __attribute__((always_inline)) {
    if constexpr (kWaves == 8) {
      v8i32 kf[2][2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) kf[b][ks] = kfrag(ks_t, b, ks);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          sacc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              kf[b][ks], qf[ks], ks == 0 ? zero16 : sacc[b], 0, 0, 0, 0, 0, 0);
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v8i32 kf[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) kf[b] = kfrag(ks_t, b, ks);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 2; ++b)
          sacc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              kf[b], qf[ks], ks == 0 ? zero16 : sacc[b], 0, 0, 0, 0, 0, 0);
      }
    }
  };

  // Online softmax of tile j into the e4m3 operand pf (keys 32 g .. +31 of
  // the tile, four per word, in order).
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int kb = seg0 + j * KB;
    if ((kb + KB > seg1) || (causal && kb + KB - 1 > qw0)) {
      // key kb + 32 b + 8 (e >> 2) + 4 g + (e & 3) is visible below lim =
      // min(seg1, qrow + 1 if causal): compare the element's constant part
      // with one per-lane value and select (per-element key conditions kept
      // a 64-bit compare mask per element live in scalar registers)
      const int lim = causal ? min(seg1, qrow + 1) : seg1;
      const int rel = lim - kb - 4 * g;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          sacc[b][e] = 32 * b + 8 * (e >> 2) + (e & 3) < rel ? sacc[b][e] : -INFINITY;
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[b][e]);
    mx = half_swap_max(mx) * cq;
    if (j == 0) {
      m_run = mx;
    } else if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DH / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      m_run = m_new;
    }
    const float nb = kPScale - m_run;
    float rs = 0.0f;
    int pk[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[b][4 * w + 0], cq, nb));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[b][4 * w + 1], cq, nb));
        const float p2 = __builtin_amdgcn_exp2f(fmaf(sacc[b][4 * w + 2], cq, nb));
        const float p3 = __builtin_amdgcn_exp2f(fmaf(sacc[b][4 * w + 3], cq, nb));
        rs += (p0 + p1) + (p2 + p3);
        int c = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
        pk[b][w] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, c, true);
      }
    l_run += rs;
    // Word w of block b holds keys 32 b + 8 w + 4 g + 0..3.  The swap leaves
    // lanes g = 0 with block 0's words of both halves and lanes g = 1 with
    // block 1's, so words (2w, 2w + 1) are keys 32 g + 8 w + 0..7.
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const auto r = __builtin_amdgcn_permlane32_swap(pk[0][w], pk[1][w], false, false);
      pf[2 * w] = (int)r[0];
      pf[2 * w + 1] = (int)r[1];
    }
  };

  // O^T[d][query] += V^T P^T: one 64-key step per d block.
  auto pv = [&](const uint8_t* vs_t) __attribute__((always_inline)) {
    constexpr int kAhead = kWaves == 8 ? DH / 32 : 2;     // fragments in flight
#pragma unroll
    for (int d0 = 0; d0 < DH / 32; d0 += kAhead) {
      v8i32 vf[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) vf[i] = vfrag(vs_t, d0 + i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kAhead; ++i)
        oacc[d0 + i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[i], pf, oacc[d0 + i], 0,
                                                                       0, 0, 0, 0, 0);
    }
  };

  // Ping-pong as in the bf16 kernel: phase t runs PV of tile t-1 and S^T of
  // tile t; the leading half of the waves does the softmax of tile t after
  // its products, the lagging half that of tile t-1 before them.  Phase t
  // reads K(t) and V(t-1) and loads K(t+1) and V(t); its closing barrier
  // frees both buffers.
  const bool lagging = ((wave >> 2) & 1) != 0;   // waves 4-7: the second of their SIMD
  auto phase = [&](const uint8_t* kcur, const uint8_t* vprev, uint8_t* knext, uint8_t* vnext,
                   int t) __attribute__((always_inline)) {
    if (t + 1 < nkt) issue_k(knext, t + 1);
    if (t < nkt) issue_v(vnext, t);
    if (lagging && t >= 1) softmax(t - 1);
    __builtin_amdgcn_s_setprio(1);
    // The leading waves issue S^T(t) before PV(t-1), so their softmax of tile
    // t starts while their own PV products still run (measured 3% faster);
    // the lagging waves need P(t-1) first and keep the bf16 kernel's order.
    if (!lagging && t < nkt) compute_s(kcur);
    if (t >= 1) pv(vprev);
    if (lagging && t < nkt) compute_s(kcur);
    __builtin_amdgcn_s_setprio(0);
    if (!lagging && t < nkt) softmax(t);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  issue_k(Ks0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t <= nkt; t += 2) {
    phase(Ks0, Vs1, Ks1, Vs0, t);
    if (t + 1 <= nkt) phase(Ks1, Vs0, Ks0, Vs1, t + 1);
  }

  // o = sum_k p'_k v_k / sum_k p'_k with p' = 2^8 p on both sides.
  const float f = vscale / half_swap_sum(l_run);
  if (qlive) {
    uint16_t* op = o + (int64_t)qrow * ld_o + h * DH;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d = 32 * db + qd * 8 + g * 4;
        const uint2 w = make_uint2(pack_bf16x2(oacc[db][4 * qd + 0] * f, oacc[db][4 * qd + 1] * f),
                                   pack_bf16x2(oacc[db][4 * qd + 2] * f, oacc[db][4 * qd + 3] * f));
        *reinterpret_cast<uint2*>(op + d) = w;
      }
  }
}

}  // namespace

hipError_t launch_attn_fp8_prepare(const uint16_t* q, int64_t ld_q, const uint16_t* k,
                                   int64_t ld_k, const uint16_t* v, int64_t ld_v,
                                   const int32_t* cu, int n_seqs, int max_seqlen,
                                   int64_t n_tokens, int n_heads, const AttnFp8Ops& ops,
                                   hipStream_t s) {
  if (n_tokens <= 0) return hipSuccess;
  if (n_tokens * n_heads > INT32_MAX / 16 || n_seqs > 65535 || n_heads > 32767 ||
      (int64_t)n_seqs * n_heads > INT32_MAX / 2)
    return hipErrorInvalidValue;
  const int n = (int)n_tokens;
  const int count = n_seqs * n_heads;
  zero_u32_kernel<<<(2 * count + 255) / 256, 256, 0, s>>>(ops.amax, 2 * count);
  seg_amax_kernel<<<dim3((unsigned)((max_seqlen + 255) / 256), n_seqs, 2 * n_heads), 256, 0, s>>>(
      k, ld_k, v, ld_v, cu, n_seqs, n_heads, ops.amax);
  seg_scale_kernel<<<(2 * count + 255) / 256, 256, 0, s>>>(ops.amax, ops.sk, ops.sv, count);
  const int64_t rows = n_tokens * n_heads;
  quant_qk_kernel<<<dim3((unsigned)((rows + 15) / 16), 2), 256, 0, s>>>(
      q, ld_q, k, ld_k, n, n_heads, cu, n_seqs, ops.sk, ops.q8, ops.k8, ops.ld8, ops.sq);
  quant_vt_kernel<<<dim3((unsigned)((max_seqlen + KB - 1) / KB), n_seqs, n_heads), 256, 0, s>>>(
      v, ld_v, cu, ops.sv, ops.vt, ops.ld_vt);
  return hipGetLastError();
}

hipError_t launch_attn_fp8(const AttnFp8Ops& ops, uint16_t* o, int64_t ld_o, const int32_t* cu,
                           int n_seqs, int max_seqlen, int64_t n_tokens, int n_heads, float scale,
                           int causal, hipStream_t s) {
  if (n_tokens <= 0) return hipSuccess;
  if (n_seqs > 65535 || n_heads > 65535) return hipErrorInvalidValue;
  const dim3 grid((max_seqlen + QBLK - 1) / QBLK, n_seqs, n_heads);
  attn_fp8_kernel<<<grid, dim3(kThreads), 0, s>>>(
      ops.q8, ops.ld8, ops.sq, n_tokens, ops.k8, ops.ld8, ops.sk, ops.vt, ops.ld_vt, ops.sv, o,
      ld_o, cu, scale * 1.4426950408889634f, causal, max_seqlen, n_tokens);
  return hipGetLastError();
}

}  // namespace dit
