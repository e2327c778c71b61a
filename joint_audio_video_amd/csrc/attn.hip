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
//   * Workgroup = 8 waves = 256 queries of one (segment, head), two waves per
//     SIMD; each wave owns 32 queries (two blocks of 16) and walks the
//     segment's keys in tiles of 64.
//   * The products are computed transposed, S^T = K Q^T and O^T = V^T P^T,
//     with v_mfma_f32_16x16x32_bf16 (16 x 16 blocks, 32 deep).  Under a
//     sustained MFMA load the chip is power-limited, and this instruction
//     draws less power per FLOP than 32x32x16: the kernel runs at about
//     2.09 GHz against 1.69 GHz, though its matrix pipe is busy a smaller
//     share of the cycles (0.58 against 0.71), so it is 0-2% faster.  In the
//     16x16 accumulator layout a lane holds, for each of its two queries, 4
//     consecutive keys of every 16-key block; a query's 64 scores of a tile
//     are spread over lanes l, l^16, l^32, l^48 (two lane exchanges give a
//     row max; row sums stay per lane until the end), and the online-softmax
//     rescale of O is a per-lane scalar per query.
//   * P needs no lane exchange: the B operand of O^T += V^T P^T gives lane
//     group g the key slots 8g .. 8g+7, mapped to keys 4g .. 4g+3 of one
//     16-key block and of the next, which are the lane's own S^T values; the
//     V^T fragment reads the same keys.
//   * Q stays in registers for the whole key loop.  K tiles and V tiles (both
//     [key][d], 256 B rows) are double-buffered in LDS (64 KB per workgroup)
//     with XOR-swizzled 16-byte chunks, filled by buffer loads that write
//     straight into LDS; V^T fragments come from transposing LDS reads.
//   * Ping-pong: the two waves sharing a SIMD run half a phase apart, so one
//     wave's softmax (exp, convert: plain VALU) overlaps the other's MFMAs.
//     Row sums are fp32 adds, not v_dot2 (which shares the matrix pipe and
//     would serialise with the other wave's MFMAs).
//   * Softmax without a per-tile max: the first key tile sets each row's
//     reference max and later tiles exponentiate against it; only a tile whose
//     probabilities would leave range moves the reference (rare).
//   * exp2 with log2(e) folded into the scale; P is rounded to bf16 for the
//     PV product, its row sum is taken over the fp32 values; accumulation in
//     float32.
//   * Masking (segment tail, causal diagonal) runs only on tiles that need
//     it; out-of-segment K/V rows are zero-filled, never read, so padding rows
//     holding NaN cannot leak in.  Causal launches longest q-tiles first.
//   * Grid = (q-tiles of the longest segment, segments, heads): consecutive
//     workgroups share one head's K/V, which stays hot in L2 / MALL.
//   * Optionally each row's log-sum-exp, lse[h][row] = log sum_j exp(s_j
//     scale), for the backward pass.
//
// f32 path: one wave per (query, head), online softmax in float32 over key
// chunks of 64 (exactness for the small float32 workload, not speed).
#include <cmath>

#include "common.h"

namespace dit {
namespace {

constexpr int DH = 128;
#ifndef DIT_ATTN_KB
#define DIT_ATTN_KB 64
#endif
constexpr int KB = DIT_ATTN_KB;   // keys per tile (a multiple of 32)
constexpr int NKB = KB / 32;      // 32-key blocks per tile
constexpr int kThreads = 256;

// Buffer resource over [base, base + bytes): raw (unstrided) addressing with
// the hardware range check, so a load at or past `bytes` reads zero (also
// when it writes straight into LDS).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposed 8-byte LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, if lane 4k'+q supplies the address of V[K0 + k'][D0 + 4q .. +3], lane j
// receives V[K0 + k][D0 + j] for k = 0..3: four consecutive keys of one column.
typedef __attribute__((address_space(3))) uint16_t lds_u16;
__device__ __forceinline__ v4i16 lds_read_tr16(const lds_u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
}

// Bound on a lane's partial row sum of one tile (so on every p) before the
// reference max is moved: 2^32.
constexpr float kRefBound = 4294967296.0f;

// LDS fragment reads are issued this many k-steps (S^T) or MFMAs (PV) ahead of
// the MFMA that consumes them; scheduling fences keep the compiler from
// sinking them next to their use, which would expose the LDS latency.
constexpr int kKAhead = 2;
constexpr int kVAhead = 2;

// Wave = 32 queries; workgroup = 8 waves = 256 queries, two waves per SIMD
// (waves w and w + 4 share one).
#ifndef DIT_ATTN_WAVES
#define DIT_ATTN_WAVES 8
#endif
constexpr int kWaves = DIT_ATTN_WAVES;
constexpr int kAttnThreads = 64 * kWaves;
constexpr int QBLK = 32 * kWaves;                  // queries per workgroup
constexpr int kTileLoads = KB * DH * 2 / 16 / kAttnThreads;   // 16-byte loads per thread per tile

// LDS tiles, row-major [key][d] (256 B per key row), 16-byte chunks XOR-swizzled.
// The LDS has 64 four-byte banks (256 B per sweep), so one key row covers every
// bank once and rows that a read serves together must sit in different chunks.
// K: chunk ^ (row & 15): a 16-byte fragment read is served 16 lanes (16
//    consecutive rows) at a time, which then touch 16 distinct chunks;
// V: chunk ^ 2*(row & 7): a transposed 8-byte read is served 32 lanes at a
//    time, eight consecutive rows of 32 contiguous bytes each, which then
//    touch eight distinct 32-byte slots of the sweep.
__device__ __forceinline__ int k_chunk(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int v_chunk(int row, int c) { return c ^ (2 * (row & 7)); }

constexpr int NKB2 = KB / 16;     // 16-key blocks per tile

// Max / sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes holding one
// query's scores), the same value in all four.
__device__ __forceinline__ float quad_max(float v) {
  v = half_swap_max(v);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quad_sum(float v) {
  v = half_swap_sum(v);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(kAttnThreads, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, int64_t ld_q, const uint16_t* __restrict__ k, int64_t ld_k,
    const uint16_t* __restrict__ v, int64_t ld_v, uint16_t* __restrict__ o, int64_t ld_o,
    const int32_t* __restrict__ cu, float scale_log2, int causal, float* __restrict__ lse,
    int64_t ld_lse, int max_seqlen, int64_t n_tokens) {
  // Two LDS buffers per tensor as distinct objects: with the key loop unrolled
  // by two, every access names its buffer at compile time, so the compiler can
  // tell the prefetch into one buffer from the reads of the other and does not
  // wait for the prefetch before reading.
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[KB * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[KB * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[KB * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[KB * DH];

  const int h = blockIdx.z, seq = blockIdx.y;
  const int seg0 = cu[seq], seg1 = cu[seq + 1];
  if (seg1 - seg0 > max_seqlen) {
    // cu_seqlens breaks its contract (a segment longer than max_seqlen): the
    // grid does not cover the segment and its byte span may pass the buffer
    // range's 4 GiB, so its rows of this head become NaN (and its lse).
    poison_rows_bf16(o, ld_o, h * DH, DH, seg0, seg1, n_tokens, blockIdx.x, gridDim.x);
    if (lse != nullptr)
      for (int64_t r = (int64_t)seg0 + blockIdx.x * kAttnThreads + threadIdx.x;
           r < seg1 && r < n_tokens; r += (int64_t)gridDim.x * kAttnThreads)
        if (r >= 0) lse[(int64_t)h * ld_lse + r] = __builtin_nanf("");
    return;
  }
  const int nqt = (seg1 - seg0 + QBLK - 1) / QBLK;
  if ((int)blockIdx.x >= nqt) return;
  const int qt = causal ? nqt - 1 - (int)blockIdx.x : (int)blockIdx.x;
  const int q0 = seg0 + qt * QBLK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform in an SGPR: the lagging/leading branches are then scalar
  // branches, with no exec-mask bookkeeping
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;
  const int qw0 = q0 + wave * 32;

  // Q^T fragments (B operand of S^T = K Q^T, 16x16x32): lane (query l16 of
  // query block qb, k group q4) holds d = 32*ds + 8*q4 .. +7.
  bf16x8 qf[2][DH / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qw0 + qb * 16 + l16;
    const uint16_t* qp = q + (int64_t)qrow * ld_q + h * DH + q4 * 8;
#pragma unroll
    for (int ds = 0; ds < DH / 32; ++ds) {
      uint4 r = qrow < seg1 ? *reinterpret_cast<const uint4*>(qp + ds * 32) : make_uint4(0, 0, 0, 0);
      qf[qb][ds] = __builtin_bit_cast(bf16x8, r);
    }
  }

  const int kend = causal ? min(seg1, q0 + QBLK) : seg1;
  const int nkt = (kend - seg0 + KB - 1) / KB;

  // Global -> LDS, 16 bytes per lane straight into LDS: slot s = threads*i + tid
  // of a tile is key row s/16, physical chunk s%16; the swizzle is applied on the
  // global side.  Offsets are bytes from key row seg0 of this head; rows past
  // the segment end fall outside the buffer range and arrive as zeros.
  const uint32_t seg_rows = (uint32_t)(seg1 - seg0);
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(k + (int64_t)seg0 * ld_k + h * DH, seg_rows * (uint32_t)ld_k * 2u);
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(v + (int64_t)seg0 * ld_v + h * DH, seg_rows * (uint32_t)ld_v * 2u);
  const int srow = tid >> 4, pch = tid & 15;
  uint32_t koff[kTileLoads], voff[kTileLoads];
#pragma unroll
  for (int i = 0; i < kTileLoads; ++i) {
    const int row = (kAttnThreads / 16) * i + srow;
    koff[i] = (uint32_t)row * (uint32_t)ld_k * 2u + (uint32_t)k_chunk(row, pch) * 16u;
    voff[i] = (uint32_t)row * (uint32_t)ld_v * 2u + (uint32_t)v_chunk(row, pch) * 16u;
  }
  const uint32_t k_tstep = (uint32_t)KB * (uint32_t)ld_k * 2u;
  const uint32_t v_tstep = (uint32_t)KB * (uint32_t)ld_v * 2u;
  auto issue_k = [&](uint16_t* kdst, int tile) {
#pragma unroll
    for (int i = 0; i < kTileLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, kdst + (kAttnThreads * i + 64 * wave) * 8, 16,
                                               koff[i], (int)(tile * k_tstep), 0, 0);
  };
  auto issue_v = [&](uint16_t* vdst, int tile) {
#pragma unroll
    for (int i = 0; i < kTileLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, vdst + (kAttnThreads * i + 64 * wave) * 8, 16,
                                               voff[i], (int)(tile * v_tstep), 0, 0);
  };

  // K fragment (A operand, 16 keys x 32 d) of key block kb and d step ds:
  // lane (key l16, k group q4) reads row 16 kb + l16, logical chunk 4 ds + q4,
  // physical chunk (4 ds + q4) ^ l16.
  int k_lane_off[DH / 32];
#pragma unroll
  for (int ds = 0; ds < DH / 32; ++ds) k_lane_off[ds] = l16 * DH + ((4 * ds + q4) ^ l16) * 8;
  // V^T fragment (A operand of O^T += V^T P^T, 16 d x 32 key slots) of d
  // block db and key step ks: lane group q4 holds slots 8 q4 .. 8 q4 + 7 =
  // keys 32 ks + 4 q4 + k, then 32 ks + 16 + 4 q4 + k (k < 4), the keys its
  // own S^T accumulators hold, so P needs no lane exchange.  Two transposed
  // reads; lane 4k' + qq of the group points at key row 4 q4 + k' (plus
  // 32 ks, plus 16 for the second read), d = 16 db + 4 qq, whose physical
  // chunk under c ^ 2 (row & 7) is 2 (db ^ rr) + (qq >> 1) with rr = row & 7.
  int v_lane_off[DH / 16];
  {
    const int vrow = 4 * q4 + (l16 >> 2), rr = vrow & 7;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) v_lane_off[db] = vrow * DH + 16 * (db ^ rr) + 4 * (l16 & 3);
  }

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};
  f32x4 oacc[DH / 16][2];
#pragma unroll
  for (int db = 0; db < DH / 16; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const f32x4 zero4 = {};

  // Ping-pong: the two waves sharing a SIMD (w and w + kWaves/2) are half a
  // phase apart.  In phase t every wave runs PV of tile t-1 and S^T of tile t;
  // the leading half does the softmax of tile t after its MFMAs, the lagging
  // half the softmax of tile t-1 before them, so one wave's exp/convert work
  // overlaps the other's MFMAs (raised wave priority during the MFMA run
  // keeps the matrix pipe fed first).  Phase t reads K(t) and V(t-1) and
  // loads K(t+1) and V(t); the barrier ending it frees both buffers.
  const bool lagging = wave >= kWaves / 2;
  f32x4 sacc[NKB2][2];     // [key block of 16][query block of 16]
  bf16x8 pf[KB / 32][2];   // [key step of 32][query block]

  // S^T[key][query] of one tile: 4 key blocks x 2 query blocks, 4 d steps.
  auto compute_s = [&](const uint16_t* ks_t) __attribute__((always_inline)) {
    auto kfrag = [&](int kb, int ds) {
      return *reinterpret_cast<const bf16x8*>(ks_t + k_lane_off[ds] + 16 * DH * kb);
    };
    bf16x8 kf[DH / 32][NKB2];
#pragma unroll
    for (int ds = 0; ds < kKAhead; ++ds)
#pragma unroll
      for (int kb = 0; kb < NKB2; ++kb) kf[ds][kb] = kfrag(kb, ds);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ds = 0; ds < DH / 32; ++ds) {
#pragma unroll
      for (int kb = 0; kb < NKB2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kf[ds][kb], qf[qb][ds], ds == 0 ? zero4 : sacc[kb][qb], 0, 0, 0);
      if (ds + kKAhead < DH / 32) {
#pragma unroll
        for (int kb = 0; kb < NKB2; ++kb) kf[ds + kKAhead][kb] = kfrag(kb, ds + kKAhead);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Online softmax of tile j (scores in sacc) into the bf16 operand pf.
  // Element r of sacc[kb][qb] is key kb0 + 16 kb + 4 q4 + r of query
  // qw0 + 16 qb + l16; a query's 64 scores sit in lanes l16 + 16 q (q < 4),
  // so a row max takes two lane exchanges and the row sums stay per lane
  // until the end.  The first key tile sets each row's reference max; later
  // tiles exponentiate against it without taking their own max.  Only when a
  // tile's probabilities could leave range (a lane's partial row sum above
  // 2^32, or not finite) does the rare path take that tile's max, move the
  // reference and rescale O and l.  o = sum p v / sum p does not depend on the
  // reference.
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int kb0 = seg0 + j * KB;
    if ((kb0 + KB > seg1) || (causal && kb0 + KB - 1 > qw0)) {
      // Key kb0 + 16 kb + 4 q4 + r is visible to query row qrow when it lies
      // below lim = min(seg1, qrow + 1 if causal): each element compares its
      // constant part 16 kb + r with one per-lane value, lim - kb0 - 4 q4, and
      // selects.  (Written as per-element conditions on the key, the compiler
      // kept 64-bit compare masks for all 32 elements live, ran out of scalar
      // registers and spilled them into vector lanes on every phase.)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qrow = qw0 + 16 * qb + l16;
        const int lim = causal ? min(seg1, qrow + 1) : seg1;
        const int rel = lim - kb0 - 4 * q4;
#pragma unroll
        for (int kb = 0; kb < NKB2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sacc[kb][qb][r] = 16 * kb + r < rel ? sacc[kb][qb][r] : -INFINITY;
      }
    }
    auto tile_max = [&](int qb) __attribute__((always_inline)) {
      float mx = sacc[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < NKB2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
      return quad_max(mx);
    };
    float rs[2];
    auto exps = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float nms = -(m_run[qb] == -INFINITY ? 0.0f : m_run[qb]) * scale_log2;
        float acc_rs = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KB / 32; ++ks)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * ks + hf][qb][r], scale_log2, nms));
              const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * ks + hf][qb][r + 1], scale_log2, nms));
              acc_rs += p0 + p1;
              pf[ks][qb][4 * hf + r] = (__bf16)p0;
              pf[ks][qb][4 * hf + r + 1] = (__bf16)p1;
            }
        rs[qb] = acc_rs;
      }
    };
    if (j == 0) {
      m_run[0] = tile_max(0);
      m_run[1] = tile_max(1);
    }
    exps();
    if (__builtin_amdgcn_ballot_w64(!(rs[0] <= kRefBound && rs[1] <= kRefBound)) != 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float m_new = fmaxf(m_run[qb], tile_max(qb));
        const float alpha = m_run[qb] == -INFINITY ? 0.0f
                                                   : __builtin_amdgcn_exp2f((m_run[qb] - m_new) * scale_log2);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DH / 16; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[db][qb][e] *= alpha;
        m_run[qb] = m_new;
      }
      exps();
    }
    l_run[0] += rs[0];
    l_run[1] += rs[1];
  };

  // O^T += V^T P^T: fragment i = 8 ks + db (key step ks, d block db) feeds
  // the two query blocks' MFMAs.
  auto pv = [&](const uint16_t* vs_t) __attribute__((always_inline)) {
    auto vread = [&](int i) __attribute__((always_inline)) {
      const int ks = i >> 3, db = i & 7;
      const lds_u16* p = (const lds_u16*)vs_t + v_lane_off[db] + 32 * ks * DH;
      const v4i16 lo = lds_read_tr16(p);
      const v4i16 hi = lds_read_tr16(p + 16 * DH);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int kN = (KB / 32) * (DH / 16);
    bf16x8 vf[kN];
#pragma unroll
    for (int i = 0; i < kVAhead; ++i) vf[i] = vread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        oacc[i & 7][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[i], pf[i >> 3][qb],
                                                                  oacc[i & 7][qb], 0, 0, 0);
      if (i + kVAhead < kN) vf[i + kVAhead] = vread(i + kVAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto phase = [&](const uint16_t* kcur, const uint16_t* vprev, uint16_t* knext, uint16_t* vnext,
                   int t) __attribute__((always_inline)) {
    if (t + 1 < nkt) issue_k(knext, t + 1);
    if (t < nkt) issue_v(vnext, t);
    if (lagging && t >= 1) softmax(t - 1);
    __builtin_amdgcn_s_setprio(1);
    if (t >= 1) pv(vprev);
    if (t < nkt) compute_s(kcur);
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

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qw0 + 16 * qb + l16;
    const float l_tot = quad_sum(l_run[qb]);
    const float inv = 1.0f / l_tot;
    // log sum_j exp(s_j scale) = ln2 (m scale_log2 + log2 l), m the row's reference max
    if (lse != nullptr && q4 == 0 && qrow < seg1)
      lse[(int64_t)h * ld_lse + qrow] = (m_run[qb] * scale_log2 + log2f(l_tot)) * 0.69314718055994531f;
    if (qrow < seg1) {
      uint16_t* op = o + (int64_t)qrow * ld_o + h * DH;
#pragma unroll
      for (int db = 0; db < DH / 16; ++db) {
        const int d = 16 * db + 4 * q4;
        const uint2 w = make_uint2(pack_bf16x2(oacc[db][qb][0] * inv, oacc[db][qb][1] * inv),
                                   pack_bf16x2(oacc[db][qb][2] * inv, oacc[db][qb][3] * inv));
        *reinterpret_cast<uint2*>(op + d) = w;
      }
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
                       float scale, int causal, float* lse, hipStream_t s) {
  if (n_seqs > 65535 || n_heads > 65535 || n_tokens > INT32_MAX) return hipErrorInvalidValue;
  if (lse != nullptr && !bf16) return hipErrorInvalidValue;
  if (bf16) {
    if (head_dim != DH) return hipErrorInvalidValue;
    const dim3 grid((max_seqlen + QBLK - 1) / QBLK, n_seqs, n_heads);
    attn_bf16_kernel<<<grid, dim3(kAttnThreads), 0, s>>>(
        static_cast<const uint16_t*>(q), ld_q, static_cast<const uint16_t*>(k), ld_k,
        static_cast<const uint16_t*>(v), ld_v, static_cast<uint16_t*>(o), ld_o, cu,
        scale * 1.4426950408889634f, causal, lse, n_tokens, max_seqlen, n_tokens);
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
