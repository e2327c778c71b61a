// Backward pass of the packed softmax attention (bf16, head_dim 128).
//
// The gradient of o = softmax(q k^T scale) v inside each cu_seqlens segment
// (the chain rule through the forward of this library's attention; the
// pages print no backward pass, the DiffusionNFT objective of [H3-NFT]
// section "DiffusionNFT: Skipping the Reverse Chain Entirely" trains the
// DiT through it).  With P = exp(s scale - lse) recomputed from the
// forward's per-row log-sum-exp and delta = rowsum(do * o):
//   dv = P^T do,  dS = P * (do v^T - delta),  dq = scale dS k,  dk = scale dS^T q.
//
// Three launches, no atomics, deterministic:
//   * attn_delta_kernel: delta[h][row], sixteen lanes per (row, head).
//   * attn_bwd_dkdv_kernel: a workgroup owns 256 keys of one (segment,
//     head) (32 per wave, their K in registers, the block's V rows in LDS;
//     8 waves, two per SIMD, share every streamed tile) and streams the
//     segment's queries in tiles of 64 (q, do, lse, delta double-buffered in
//     LDS).  Per tile a wave computes S = q k^T and dP = do v^T (rows =
//     queries, so the 32x32 accumulator gives each lane one key column), P
//     and dS elementwise, then dv^T += do^T P and dk^T += q^T dS with the
//     transposed operand read from LDS by ds_read_b64_tr_b16 and P / dS as
//     the bf16 B operand in the accumulator's own row order (the k index of
//     a product can be permuted as long as both operands agree).
//   * attn_bwd_dq_kernel: a workgroup owns 256 queries (q, do, lse, delta of
//     its 32 per wave in registers; 8 waves, the two of a SIMD in ping-pong)
//     and streams the keys in tiles of 64 (triple-buffered):
//     S^T = k q^T and dP^T = v do^T (rows = keys), dS^T, then
//     dq^T += k^T dS^T, as the forward kernel computes O^T.
// All products are v_mfma_f32_32x32x16_bf16 with float32 accumulation, their
// LDS fragments read one or two products ahead; P and dS are rounded to bf16
// as MFMA operands.  Rows past a segment's end
// load as zeros (buffer range checks) and get P = 0.
#include <cmath>

#include "common.h"

namespace dit {
namespace {

constexpr int DH = 128;
constexpr int TB = 64;                 // streamed rows per tile
// dq: 8 waves (256 queries) per workgroup, two per SIMD in ping-pong.
constexpr int kThreadsQ = 512;
constexpr int BLKQ = kThreadsQ / 2;
// dk, dv: 8 waves (256 keys) per workgroup, two waves per SIMD sharing each
// streamed tile.
constexpr int kThreadsKV = 512;
constexpr int BLKKV = kThreadsKV / 2;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// LDS tiles are [row][d] with 256-byte rows; 16-byte chunk c of row r sits at
// physical chunk c ^ f(r), f(r) = (4 (r & 3) + ((r >> 1) & 3)) ^ 8 ((r >> 3) & 1).
// The tiles are read both as rows (16 consecutive rows, one chunk each, per
// cycle of a 16-byte read) and transposed (four consecutive rows, four
// adjacent chunks, per cycle of an 8-byte transposing read).  The LDS has 64
// four-byte banks, one sweep per 256-byte row, so a read is conflict-free
// when its 16 chunks land on 16 distinct physical chunks: f is one-to-one on
// r & 15 (row reads), and f >> 2 differs on every aligned four rows
// (transposed reads).  f (r + 8) = f (r) ^ 8, so the second half of a
// transposed fragment (rows + 8) is the first half's address with db ^ 2.
__device__ __forceinline__ int swz_f(int row) {
  return (4 * (row & 3) + ((row >> 1) & 3)) ^ (8 * ((row >> 3) & 1));
}
__device__ __forceinline__ int swz(int row, int c) { return c ^ swz_f(row); }

// Fragment reads.  Each lane keeps one byte offset per fragment kind; the
// offset of a given k-slice or d block is that base with a few bits flipped
// (the swizzle is an XOR on the chunk index, and row and tile bases have none
// of those bits), computed next to its reads by one XOR in inline assembly.
// Left to itself the compiler hoists every (offset, tile) combination out of
// the tile loop into registers; at 256 registers that spilled, or left no
// room to read fragments ahead of their products.  Tile bases and row blocks
// go into the LDS instructions' immediate offset.
//
// Row fragment: lane (l32, g) reads tile row rb + l32 (rb a multiple of 16),
// d = 16 ks + 8 g .. +7, i.e. logical chunk 2 ks + g, at physical chunk
// (2 ks + g) ^ f(l32) = 2 ks ^ (g ^ f(l32)): byte offset base ^ 32 ks.
struct RowFrag {
  int base;   // bytes: row l32, chunk g ^ f(l32)
  __device__ void init(int lane) {
    const int l32 = lane & 31, g = lane >> 5;
    base = 2 * (l32 * DH + 8 * (g ^ swz_f(l32)));
  }
  // byte offset of k-slice ks
  __device__ __forceinline__ int at(int ks) const {
    if (ks == 0) return base;
    int r;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "i"(32 * ks), "v"(base));
    return r;
  }
  __device__ __forceinline__ bf16x8 read_at(const uint16_t* t, int rb, int o) const {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(t) + o + rb * DH * 2);
  }
};

// Transposed fragment: 32 rows d = 32 db + l32, 8 k values = tile rows
// b0 + 4g + {0..3} and b0 + 4g + 8 + {0..3} (b0 a multiple of 16), two
// ds_read_b64_tr_b16.  In each 16-lane group (t = (lane >> 4) & 1) lane i
// supplies row b0 + y, y = 4 g + (i >> 2), columns 32 db + 16 t + 4 (i & 3)
// .. +3 and receives column 32 db + l32 of the four rows.  The column's
// chunk 4 db + x (x = 2 t + ((i & 3) >> 1)) sits at physical chunk
// 4 (db ^ (f(y) >> 2)) + (x ^ (f(y) & 3)): byte offset base ^ 64 db, and for
// rows y + 8, where f flips bit 3, base ^ 64 (db ^ 2) one 8-row step on.
struct TrFrag {
  int base;   // bytes: the lane's half-chunk of row y for d block 0
  __device__ void init(int lane) {
    const int i = lane & 15, t = (lane >> 4) & 1, g = lane >> 5;
    const int y = 4 * g + (i >> 2), x = 2 * t + ((i & 3) >> 1);
    const int f = swz_f(y);
    base = 2 * (y * DH + 8 * (x ^ (f & 3)) + 4 * (i & 1) + 32 * (f >> 2));
  }
  __device__ __forceinline__ int xr(int c) const {
    if (c == 0) return base;
    int r;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "i"(c), "v"(base));
    return r;
  }
  // byte offsets of d block db in the rows b0 + y and b0 + 8 + y
  __device__ __forceinline__ int2 at(int db) const {
    return make_int2(xr(64 * db), xr(64 * (db ^ 2)));
  }
  __device__ __forceinline__ bf16x8 read_at(const uint16_t* tile, int b0, int2 o) const {
    const lds_u16* p = (const lds_u16*)((const char*)tile + o.x + b0 * DH * 2);
    const lds_u16* p2 = (const lds_u16*)((const char*)tile + o.y + (b0 + 8) * DH * 2);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p2);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// Accumulator element e of a 32x32 block lies in row 8 (e / 4) + 4 g + e % 4.
__device__ __forceinline__ int acc_row(int e, int g) { return 8 * (e >> 2) + 4 * g + (e & 3); }

// Global -> LDS tile loader for a workgroup of THREADS threads: slot
// s = THREADS * i + tid is tile row s / 16, physical chunk s % 16 (the
// swizzle applied on the global side).
template <int THREADS>
struct TileLoader {
  static constexpr int kLoads = TB * DH * 2 / 16 / THREADS;   // 16-byte loads per thread
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off[kLoads];
  uint32_t tstep;
  __device__ void init(const uint16_t* base, int64_t ld, uint32_t rows, int tid) {
    rs = make_rsrc(base, rows * (uint32_t)ld * 2u);
    const int srow = tid >> 4, pch = tid & 15;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int row = (THREADS / 16) * i + srow;
      off[i] = (uint32_t)row * (uint32_t)ld * 2u + (uint32_t)swz(row, pch) * 16u;
    }
    tstep = (uint32_t)TB * (uint32_t)ld * 2u;
  }
  __device__ void issue(uint16_t* dst, int tile, int wave) const {
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + (THREADS * i + 64 * wave) * 8, 16,
                                               off[i], (int)(tile * tstep), 0, 0);
  }
};

// delta[h][row] = sum_d do[row][h d] o[row][h d].  Sixteen lanes share one
// (row, head): each reads 16 bytes of o and of do, so a wave reads 1 KB of
// contiguous row per instruction, and the group sums over shuffles.
__global__ __launch_bounds__(256) void attn_delta_kernel(const uint16_t* __restrict__ o,
                                                         int64_t ld_o,
                                                         const uint16_t* __restrict__ dout,
                                                         int64_t ld_do, float* __restrict__ delta,
                                                         int64_t n, int n_heads) {
  const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;   // (row, head) pair
  const int part = threadIdx.x & 15;
  const bool live = idx < n * n_heads;
  const int64_t row = live ? idx / n_heads : 0;
  const int h = live ? (int)(idx - row * n_heads) : 0;
  float s = 0.0f;
  if (live) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + row * ld_o + h * DH + 8 * part);
    const uint4 b = *reinterpret_cast<const uint4*>(dout + row * ld_do + h * DH + 8 * part);
    s = fmaf(bf16lo(a.x), bf16lo(b.x), s); s = fmaf(bf16hi(a.x), bf16hi(b.x), s);
    s = fmaf(bf16lo(a.y), bf16lo(b.y), s); s = fmaf(bf16hi(a.y), bf16hi(b.y), s);
    s = fmaf(bf16lo(a.z), bf16lo(b.z), s); s = fmaf(bf16hi(a.z), bf16hi(b.z), s);
    s = fmaf(bf16lo(a.w), bf16lo(b.w), s); s = fmaf(bf16hi(a.w), bf16hi(b.w), s);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (live && part == 0) delta[(int64_t)h * n + row] = s;
}

// Stores a 32x32 accumulator block transposed into rows of out: lane (key or
// query l32) writes d = 32 db + 8 j + 4 g .. +3 for j = 0..3.
__device__ __forceinline__ void store_rows(uint16_t* rowp, const f32x16& acc, int db, int g,
                                           float mul) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = 32 * db + 8 * j + 4 * g;
    *reinterpret_cast<uint2*>(rowp + d) =
        make_uint2(pack_bf16x2(acc[4 * j] * mul, acc[4 * j + 1] * mul),
                   pack_bf16x2(acc[4 * j + 2] * mul, acc[4 * j + 3] * mul));
  }
}

__global__ __launch_bounds__(kThreadsKV, 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, int64_t ld_q, const uint16_t* __restrict__ k, int64_t ld_k,
    const uint16_t* __restrict__ v, int64_t ld_v, const uint16_t* __restrict__ dout,
    int64_t ld_do, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, int64_t ld_dk, uint16_t* __restrict__ dv, int64_t ld_dv,
    const int32_t* __restrict__ cu, int64_t n, float scale, float scale_log2, int causal,
    int max_seqlen) {
  // The streamed tiles are aligned so that they are laid out first, below
  // 64 KB: their addresses then fit the LDS instructions' 16-bit offset.
  __shared__ __attribute__((aligned(4096))) uint16_t Qs0[TB * DH];
  __shared__ __attribute__((aligned(4096))) uint16_t Qs1[TB * DH];
  __shared__ __attribute__((aligned(4096))) uint16_t Ds0[TB * DH];
  __shared__ __attribute__((aligned(4096))) uint16_t Ds1[TB * DH];
  __shared__ float Ls0[TB], Ls1[TB], Es0[TB], Es1[TB];   // lse * log2(e), delta
  __shared__ __attribute__((aligned(16))) uint16_t Vb[BLKKV * DH];   // this block's V rows

  const int h = blockIdx.z, seq = blockIdx.y;
  const int seg0 = cu[seq], seg1 = cu[seq + 1];
  if (seg1 - seg0 > max_seqlen) {
    // a segment longer than max_seqlen (cu_seqlens breaks its contract): the
    // grid does not cover it; its dk and dv rows of this head become NaN
    poison_rows_bf16(dk, ld_dk, h * DH, DH, seg0, seg1, n, blockIdx.x, gridDim.x);
    poison_rows_bf16(dv, ld_dv, h * DH, DH, seg0, seg1, n, blockIdx.x, gridDim.x);
    return;
  }
  const int kb0 = seg0 + (int)blockIdx.x * BLKKV;
  if (kb0 >= seg1) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int l32 = lane & 31, g = lane >> 5;
  const int key = kb0 + 32 * wave + l32;
  RowFrag rf;
  TrFrag tf;
  rf.init(lane);
  tf.init(lane);

  // K^T operand of this wave's 32 keys in registers: lane (key l32, half g)
  // holds d = 16 ks + 8 g .. +7.  V's rows of the whole block wait in LDS
  // (the same operand read per tile), which keeps a wave within 256
  // registers, so two waves share each SIMD.
  bf16x8 kf[DH / 16];
  {
    const bool live = key < seg1;
    const uint16_t* kp = k + (int64_t)key * ld_k + h * DH + 8 * g;
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks) {
      const uint4 a = live ? *reinterpret_cast<const uint4*>(kp + 16 * ks) : make_uint4(0, 0, 0, 0);
      kf[ks] = __builtin_bit_cast(bf16x8, a);
    }
    TileLoader<kThreadsKV> lvb;
    lvb.init(v + (int64_t)kb0 * ld_v + h * DH, ld_v, (uint32_t)(seg1 - kb0), tid);
#pragma unroll
    for (int j = 0; j < BLKKV / TB; ++j) lvb.issue(Vb + j * TB * DH, j, wave);
  }
  const int vrb = 32 * wave;

  // Query tiles: causal attention reaches this block's keys only from queries >= kb0.
  const int qt0 = causal ? (kb0 - seg0) / TB : 0;
  const int nqt = (seg1 - seg0 + TB - 1) / TB;
  const uint32_t seg_rows = (uint32_t)(seg1 - seg0);
  TileLoader<kThreadsKV> lq, ld;
  lq.init(q + (int64_t)seg0 * ld_q + h * DH, ld_q, seg_rows, tid);
  ld.init(dout + (int64_t)seg0 * ld_do + h * DH, ld_do, seg_rows, tid);
  const float* lse_h = lse + (int64_t)h * n;
  const float* del_h = delta + (int64_t)h * n;
  // lse / delta of a tile: threads 0..63 fetch lse, 64..127 delta (registers,
  // stored to LDS after the current tile's reads).
  auto fetch_ld = [&](int t) -> float {
    const int r = seg0 + t * TB + (tid & 63);
    if (tid < 64) return r < seg1 ? lse_h[r] * 1.4426950408889634f : INFINITY;
    if (tid < 128) return r < seg1 ? del_h[r] : 0.0f;
    return 0.0f;
  };
  auto put_ld = [&](float* L, float* E, float val) {
    if (tid < 64) L[tid] = val;
    else if (tid < 128) E[tid - 64] = val;
  };

  f32x16 dka[DH / 32], dva[DH / 32];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dka[db][e] = 0.0f, dva[db][e] = 0.0f;
  const f32x16 zero16 = {};

  auto step = [&](const uint16_t* Qs, const uint16_t* Ds, const float* Ls, const float* Es,
                  uint16_t* Qn, uint16_t* Dn, float* Ln, float* En, int t)
      __attribute__((always_inline)) {
    float nxt = 0.0f;
    if (t + 1 < nqt) {
      lq.issue(Qn, t + 1, wave);
      ld.issue(Dn, t + 1, wave);
      nxt = fetch_ld(t + 1);
    }
    const int qbase = seg0 + t * TB;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 sacc = zero16, pacc = zero16;
      // fragments of k-slice ks + 1 are read while the products of ks run
      bf16x8 fq, fd, fv;
      {
        const int ro = rf.at(0);
        fq = rf.read_at(Qs, 32 * qb, ro);
        fd = rf.read_at(Ds, 32 * qb, ro);
        fv = rf.read_at(Vb, vrb, ro);
      }
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) {
        bf16x8 nq = fq, nd = fd, nv = fv;
        if (ks + 1 < DH / 16) {
          const int ro = rf.at(ks + 1);
          nq = rf.read_at(Qs, 32 * qb, ro);
          nd = rf.read_at(Ds, 32 * qb, ro);
          nv = rf.read_at(Vb, vrb, ro);
        }
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq, kf[ks], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fd, fv, pacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        fq = nq; fd = nd; fv = nv;
      }
      // some query of the block precedes some key of the wave (wave-uniform);
      // then query qbase + 32 qb + 8 (e >> 2) + 4 g + (e & 3) of element e
      // precedes this lane's key when its constant part is below rel
      const bool diag = causal && qbase + 32 * qb < kb0 + 32 * wave + 31;
      const int rel = key - qbase - 32 * qb - 4 * g;
      bf16x8 pf[2], sf[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * qb + acc_row(e, g);
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[e], scale_log2, -Ls[r]));
        if (diag) p = 8 * (e >> 2) + (e & 3) < rel ? 0.0f : p;
        const float ds = p * (pacc[e] - Es[r]);
        pf[e >> 3][e & 7] = (__bf16)p;
        sf[e >> 3][e & 7] = (__bf16)ds;
      }
      __builtin_amdgcn_sched_barrier(0);
      // the next d block's transposed fragments are read during this one's products
      bf16x8 td, tq;
      {
        const int2 to = tf.at(0);
        td = tf.read_at(Ds, 32 * qb, to);
        tq = tf.read_at(Qs, 32 * qb, to);
      }
#pragma unroll
      for (int it = 0; it < 2 * DH / 32; ++it) {
        const int u = it >> 2, db = it & 3;
        bf16x8 nd = td, nq = tq;
        if (it + 1 < 2 * DH / 32) {
          const int b1 = 32 * qb + 16 * ((it + 1) >> 2);
          const int2 to = tf.at((it + 1) & 3);
          nd = tf.read_at(Ds, b1, to);
          nq = tf.read_at(Qs, b1, to);
        }
        dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(td, pf[u], dva[db], 0, 0, 0);
        dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq, sf[u], dka[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        td = nd; tq = nq;
      }
    }
    if (t + 1 < nqt) put_ld(Ln, En, nxt);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if (qt0 < nqt) {
    lq.issue(Qs0, qt0, wave);
    ld.issue(Ds0, qt0, wave);
    put_ld(Ls0, Es0, fetch_ld(qt0));
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = qt0; t < nqt; t += 2) {
    step(Qs0, Ds0, Ls0, Es0, Qs1, Ds1, Ls1, Es1, t);
    if (t + 1 < nqt) step(Qs1, Ds1, Ls1, Es1, Qs0, Ds0, Ls0, Es0, t + 1);
  }

  if (key < seg1) {
    uint16_t* kr = dk + (int64_t)key * ld_dk + h * DH;
    uint16_t* vr = dv + (int64_t)key * ld_dv + h * DH;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db) {
      store_rows(kr, dka[db], db, g, scale);
      store_rows(vr, dva[db], db, g, 1.0f);
    }
  }
}

__global__ __launch_bounds__(kThreadsQ, 1) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, int64_t ld_q, const uint16_t* __restrict__ k, int64_t ld_k,
    const uint16_t* __restrict__ v, int64_t ld_v, const uint16_t* __restrict__ dout,
    int64_t ld_do, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dq, int64_t ld_dq, const int32_t* __restrict__ cu, int64_t n,
    float scale, float scale_log2, int causal, int max_seqlen) {
  // Key and value tiles, three buffers each as distinct objects (the main loop
  // is unrolled by three, so every access names its buffer at compile time and
  // the compiler can tell a prefetch from the reads of another buffer).
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[TB * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[TB * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Ks2[TB * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[TB * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[TB * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Vs2[TB * DH];

  const int h = blockIdx.z, seq = blockIdx.y;
  const int seg0 = cu[seq], seg1 = cu[seq + 1];
  if (seg1 - seg0 > max_seqlen) {
    // as in the key kernel: the segment's dq rows of this head become NaN
    poison_rows_bf16(dq, ld_dq, h * DH, DH, seg0, seg1, n, blockIdx.x, gridDim.x);
    return;
  }
  const int q0 = seg0 + (int)blockIdx.x * BLKQ;
  if (q0 >= seg1) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int l32 = lane & 31, g = lane >> 5;
  const int qrow = q0 + 32 * wave + l32;
  const bool live = qrow < seg1;
  RowFrag rf;
  TrFrag tf;
  rf.init(lane);
  tf.init(lane);

  // Q^T and dO^T operands (B of S^T = K Q^T and dP^T = V dO^T): lane (query
  // l32, half g) holds d = 16 ks + 8 g .. +7.
  bf16x8 qf[DH / 16], df[DH / 16];
  {
    const uint16_t* qp = q + (int64_t)qrow * ld_q + h * DH + 8 * g;
    const uint16_t* dp = dout + (int64_t)qrow * ld_do + h * DH + 8 * g;
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks) {
      const uint4 a = live ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
      const uint4 b = live ? *reinterpret_cast<const uint4*>(dp + 16 * ks) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, a);
      df[ks] = __builtin_bit_cast(bf16x8, b);
    }
  }
  const float lse2 = live ? lse[(int64_t)h * n + qrow] * 1.4426950408889634f : INFINITY;
  const float dlt = live ? delta[(int64_t)h * n + qrow] : 0.0f;

  const int kend = causal ? min(seg1, q0 + BLKQ) : seg1;
  const int nkt = (kend - seg0 + TB - 1) / TB;
  const uint32_t seg_rows = (uint32_t)(seg1 - seg0);
  TileLoader<kThreadsQ> lk, lv;
  lk.init(k + (int64_t)seg0 * ld_k + h * DH, ld_k, seg_rows, tid);
  lv.init(v + (int64_t)seg0 * ld_v + h * DH, ld_v, seg_rows, tid);

  f32x16 dqa[DH / 32];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqa[db][e] = 0.0f;
  const f32x16 zero16 = {};
  f32x16 sacc[2], pacc[2];
  bf16x8 sf[4];

  // Tile t's products S^T = K Q^T and dP^T = V dO^T (two 32-key blocks).
  auto products = [&](const uint16_t* Ks, const uint16_t* Vs) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sacc[b] = zero16;
      pacc[b] = zero16;
      // fragments of k-slice ks + 1 are read while the products of ks run
      bf16x8 fk, fv;
      {
        const int ro = rf.at(0);
        fk = rf.read_at(Ks, 32 * b, ro);
        fv = rf.read_at(Vs, 32 * b, ro);
      }
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) {
        bf16x8 nk = fk, nv = fv;
        if (ks + 1 < DH / 16) {
          const int ro = rf.at(ks + 1);
          nk = rf.read_at(Ks, 32 * b, ro);
          nv = rf.read_at(Vs, 32 * b, ro);
        }
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk, qf[ks], sacc[b], 0, 0, 0);
        pacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv, df[ks], pacc[b], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        fk = nk; fv = nv;
      }
    }
  };
  // Tile t's P^T and dS^T (VALU) into the bf16 operand sf.
  auto grads = [&](int t) __attribute__((always_inline)) {
    const int kbase = seg0 + t * TB;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int kb = kbase + 32 * b;
      const bool edge = kb + 32 > seg1 || (causal && kb + 31 > q0 + 32 * wave);
      // key kb + 8 (e >> 2) + 4 g + (e & 3) of element e is visible below
      // lim = min(seg1, qrow + 1 if causal): its constant part against rel
      const int rel = (causal ? min(seg1, qrow + 1) : seg1) - kb - 4 * g;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[b][e], scale_log2, -lse2));
        if (edge) p = 8 * (e >> 2) + (e & 3) < rel ? p : 0.0f;
        sf[2 * b + (e >> 3)][e & 7] = (__bf16)(p * (pacc[b][e] - dlt));
      }
    }
  };
  // dq^T += K^T dS^T with tile t's K read transposed.
  auto accumulate = [&](const uint16_t* Ks) __attribute__((always_inline)) {
    // K^T fragments are read two products ahead
    bf16x8 t0 = tf.read_at(Ks, 0, tf.at(0)), t1 = tf.read_at(Ks, 0, tf.at(1));
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      bf16x8 t2 = t1;
      if (it + 2 < 16) t2 = tf.read_at(Ks, 16 * ((it + 2) >> 2), tf.at((it + 2) & 3));
      dqa[it & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t0, sf[it >> 2], dqa[it & 3], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      t0 = t1; t1 = t2;
    }
  };

  // Ping-pong between the two waves of a SIMD (w and w + 4), as in the
  // forward kernel: in phase t every wave runs the dq product of tile t-1 and
  // the S^T, dP^T products of tile t; the leading half computes P and dS of
  // tile t after its MFMAs, the lagging half those of tile t-1 before them,
  // so one wave's exponentials overlap the other's MFMAs.  Phase t reads K of
  // tiles t-1 and t and V of tile t, and loads tile t+1 into the third buffer.
  const bool lagging = wave >= kThreadsQ / 128;
  auto phase = [&](const uint16_t* Kprev, const uint16_t* Kcur, const uint16_t* Vcur,
                   uint16_t* Knext, uint16_t* Vnext, int t) __attribute__((always_inline)) {
    if (t + 1 < nkt) {
      lk.issue(Knext, t + 1, wave);
      lv.issue(Vnext, t + 1, wave);
    }
    if (lagging && t >= 1) grads(t - 1);
    __builtin_amdgcn_s_setprio(1);
    if (t >= 1) accumulate(Kprev);
    if (t < nkt) products(Kcur, Vcur);
    __builtin_amdgcn_s_setprio(0);
    if (!lagging && t < nkt) grads(t);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if (nkt > 0) {
    lk.issue(Ks0, 0, wave);
    lv.issue(Vs0, 0, wave);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t <= nkt; t += 3) {
    phase(Ks2, Ks0, Vs0, Ks1, Vs1, t);
    if (t + 1 <= nkt) phase(Ks0, Ks1, Vs1, Ks2, Vs2, t + 1);
    if (t + 2 <= nkt) phase(Ks1, Ks2, Vs2, Ks0, Vs0, t + 2);
  }

  if (live) {
    uint16_t* qr = dq + (int64_t)qrow * ld_dq + h * DH;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db) store_rows(qr, dqa[db], db, g, scale);
  }
}

}  // namespace

hipError_t launch_attn_bwd(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                           const void* v, int64_t ld_v, const void* o, int64_t ld_o,
                           const void* dout, int64_t ld_do, const float* lse, void* dq,
                           int64_t ld_dq, void* dk, int64_t ld_dk, void* dv, int64_t ld_dv,
                           const int32_t* cu, int n_seqs, int max_seqlen, int64_t n_tokens,
                           int n_heads, float scale, int causal, float* delta, hipStream_t s) {
  if (n_seqs > 65535 || n_heads > 65535 || n_tokens > INT32_MAX) return hipErrorInvalidValue;
  // the buffer resources address a segment's rows with 32-bit byte offsets
  for (int64_t ld : {ld_q, ld_k, ld_v, ld_do})
    if ((uint64_t)max_seqlen * (uint64_t)ld * 2u > 0xFFFFFFFFull) return hipErrorInvalidValue;
  if (n_tokens == 0) return hipSuccess;
  const int64_t lanes = n_tokens * n_heads * 16;
  attn_delta_kernel<<<dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s>>>(
      static_cast<const uint16_t*>(o), ld_o, static_cast<const uint16_t*>(dout), ld_do, delta,
      n_tokens, n_heads);
  const float sl2 = scale * 1.4426950408889634f;
  const dim3 grid_kv((max_seqlen + BLKKV - 1) / BLKKV, n_seqs, n_heads);
  attn_bwd_dkdv_kernel<<<grid_kv, dim3(kThreadsKV), 0, s>>>(
      static_cast<const uint16_t*>(q), ld_q, static_cast<const uint16_t*>(k), ld_k,
      static_cast<const uint16_t*>(v), ld_v, static_cast<const uint16_t*>(dout), ld_do, lse, delta,
      static_cast<uint16_t*>(dk), ld_dk, static_cast<uint16_t*>(dv), ld_dv, cu, n_tokens, scale,
      sl2, causal, max_seqlen);
  const dim3 grid_q((max_seqlen + BLKQ - 1) / BLKQ, n_seqs, n_heads);
  attn_bwd_dq_kernel<<<grid_q, dim3(kThreadsQ), 0, s>>>(
      static_cast<const uint16_t*>(q), ld_q, static_cast<const uint16_t*>(k), ld_k,
      static_cast<const uint16_t*>(v), ld_v, static_cast<const uint16_t*>(dout), ld_do, lse, delta,
      static_cast<uint16_t*>(dq), ld_dq, cu, n_tokens, scale, sl2, causal, max_seqlen);
  return hipGetLastError();
}

}  // namespace dit
