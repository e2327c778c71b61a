// Projections of the block: C = A B^T (+ bias), with four epilogues.
//   plain:          qkv = y W_qkv^T + b          (fused to_q | to_k | to_v)
//   gated residual: out = x + gate[m] * (o W_o^T + b)   (to_out.0, ff.net.2)
//   GELU:           h = gelu_tanh(y W_1^T + b)   (ff.net.0.proj)
//   planes + RoPE:  q', k', v = rotate(y W_qkv^T + b) into three planes, the
//                   3D rotation applied to q and k before the single bf16
//                   rounding ([H3-NFT] section "MiniMax H3 and Why Joint
//                   Audio-Video Generation Complicates RL Training": RoPE over
//                   time, height and width).  Each lane holds 4 consecutive
//                   columns of one row, i.e. 2 pairs of one head; the row's
//                   (t, h, w) positions are loaded after the k loop, and a
//                   pair's angle is pos * omega in turns, reduced to [-1/2, 1/2]
//                   exactly, then sin and cos in float32 (the hardware's
//                   turn-based sine and cosine).  A zero position leaves the
//                   pair's bits as they are.
// [VeRL-Omni] section 5.2 (Q, K, V packed into one matrix on the rollout
// side); [H3-NFT] section "How VeRL-Omni's Adapter Architecture Keeps
// H3-Specific Logic Contained" (projection names to_q, to_k, to_v, to_out.0,
// ff.net.0.proj, ff.net.2); the feed-forward activation, tanh-form GELU, is a
// reading (the pages name none).
//
// bf16 path: CDNA4 bf16 MFMA (v_mfma_f32_16x16x32_bf16), float32 accumulate.
// Workgroup tile 256x256x64, four waves in a 2x2 arrangement, each owning a
// 128x128 sub-tile as 8x8 MFMA blocks of 16x16 (256 accumulators per lane,
// held in the AGPR half of the register file).  A and B tiles are staged through LDS
// (double-buffered, 128 KB): global loads into registers a step ahead, then
// LDS writes, with an XOR swizzle of the 16-byte chunk index so the rows an MFMA fragment
// read touches spread over the banks.  The LDS has 64 four-byte banks, so a
// 16-byte read is served 16 lanes at a time; a tile row is 128 bytes, so
// those 16 rows must land on 16 distinct 16-byte slots of a 256-byte sweep,
// which chunk ^ ((row>>1) & 7) gives (row pairs share a chunk pattern and
// differ by the 128-byte half).  Both operands are K-contiguous
// ([rows][K]), so every fragment is one 16-byte LDS read.
// With one wave per SIMD nothing else hides latency, so each k-step is laid
// out by hand as 32 fenced groups of four independent MFMAs; one fragment
// read of the next sub-step rides in each group's shadow, and one LDS write
// of the next tile and one global load of the tile after it in every second.
// 16x16x32 rather than 32x32x16: the chip is power-limited under sustained
// MFMA load, and the smaller instruction draws less power per FLOP.  A
// register-only probe (independent MFMAs on every CU for tens of ms) keeps
// the matrix pipe 93-95% busy with either, but at about 1.78 GHz with
// 32x32x16 (69% of the 2.4 GHz peak rate) against 2.07 GHz with 16x16x32
// (82%).  In this kernel the clock rises from 1.66 to 1.90 GHz while the
// matrix pipe's busy share falls from 0.73 to 0.65 (memory latency is fixed
// in time, so it costs more cycles, and a step issues twice the MFMAs).  Net,
// in two same-process A/B runs on two boxes (rotated order, medians of six
// rounds): QKV -1.2% / +1.4%, to_out.0 -1.6% / -1.5%, ff.net.0.proj -2.0% /
// -0.2%, ff.net.2 -0.7% / -0.6% in time, bit-identical results.  Loading through
// registers gives every global load a full step to land; loads that wrote
// straight into LDS (buffer_load ... lds) had to wait for the barrier that
// freed their stage and had half a step to a step.  Same-process A/B on the
// block's shapes (58,758 tokens), four runs on different boxes: 0.5-3.8%
// faster per product, about 2% on average (last run: QKV 7.46 -> 7.40 ms,
// to_out.0 2.68 -> 2.65, ff.net.0.proj 10.23 -> 10.06, ff.net.2 9.83 ->
// 9.77), bit-identical results.  Counters on the QKV product: the clock
// under this load is about 1.72 GHz (0.72 of the 2.4 GHz peak rate is the
// ceiling) and the MFMA pipe is busy 73% of cycles (70% before); the rest is
// issue stalls behind memory instructions that one wave per SIMD cannot
// cover.  Tried and slower: five 32-k LDS stages with direct-to-LDS loads
// (two to three steps of cover, but 64-byte row segments cost more in the
// load path than the cover gains), two staging register sets (two steps of
// cover), and running the last sub-step after the barrier.
// Tile order.  The hardware deals consecutive workgroups to the 8 XCDs (one
// L2 each) round-robin, and an XCD runs about 32 of them at once (one per CU).
// Workgroup pid = 8 j + x becomes the j-th tile of XCD x's contiguous share of
// a linear order in which 32 consecutive tiles form a block of 4 M-tiles by 8
// N-tiles, so the 32 workgroups an XCD runs together read 4 A and 8 B panels
// (12 k-slices per k-step) instead of one A panel against 32 B panels (33);
// the last T mod 8 workgroups keep their index.  Measured on one box: the
// QKV product's L2 fills drop from 40 to 16 GB (FP8), and same-process A/B
// times fall for bf16 QKV (7.73 -> 7.58 ms), to_out.0 (2.72 -> 2.63) and
// ff.net.0.proj (10.52 -> 10.42) and for the FP8 products by 4-5%.
//
// float32 path: a plain LDS-tiled VALU kernel (the tiny float32 workload only
// needs to be exact, not fast).
#include "common.h"

namespace dit {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kXcds = 8;

struct EpiArgs {
  int kind;
  const uint16_t* bias;
  const uint16_t* x;
  int64_t ld_x;
  const uint8_t* mod;
  const float* gate;
  int64_t gate_stride;      // floats between the gate rows of two modalities
  int plane_cols;           // kinds 0, 3: output split into planes of this many columns (0: none)
  int64_t plane_stride;     // elements between planes
  // kinds 3 (head_dim 128) and 4 (head_dim 64): 3D RoPE on planes 0 and 1
  const int32_t* pos;       // [M][3] (t, h, w) per row
  int pair_h, pair_w;       // first pair of the h and of the w section
  float rope_rev[64];       // per pair: omega / (2 pi), turns per unit of position
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Tile of this workgroup (the XCD-blocked order above): linear index L in
// groups of 4 M-tiles, each walked in chunks of 8 N-tiles, M fastest inside a
// chunk.  A bijection from workgroup ids onto the tiles_m x tiles_n tiles for
// any tile counts: pid -> L permutes the first 8 * per_xcd ids (x-major to
// XCD-contiguous) and fixes the rest, and L -> (group, chunk, r) covers each
// group's gsize x tiles_n tiles once, the last group and chunk partial (the
// GPU tests' ragged shapes exercise both).
__device__ __forceinline__ void tile_coords_xcd(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int pid = blockIdx.x;
  const int per_xcd = (tiles_m * tiles_n) / kXcds;
  const int L = pid < kXcds * per_xcd ? (pid % kXcds) * per_xcd + pid / kXcds : pid;
  const int group = L / (4 * tiles_n);
  const int idx = L - group * 4 * tiles_n;
  const int gsize = min(4, tiles_m - 4 * group);
  const int chunk = idx / (gsize * 8);
  const int r = idx - chunk * gsize * 8;
  tm = 4 * group + r % gsize;
  tn = 8 * chunk + r / gsize;
}

template <int KIND>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B,
    uint16_t* C, int64_t ldc, int M, int N, int K, EpiArgs ep) {
  // Two LDS stages per operand.
  __shared__ __attribute__((aligned(16))) uint16_t As0[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t As1[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs0[BN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs1[BN * BK];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords_xcd(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int wm = wave >> 1, wn = wave & 1;

  constexpr bool kRope = KIND == 3 || KIND == 4;

  // Global -> registers -> LDS: lane slot s = 256*i + tid of a tile is a
  // 16-byte global load that is written to LDS element 8*s, i.e. row s/8,
  // physical chunk s%8 (so each wave's LDS write is 1 KB contiguous).  The
  // swizzle is applied on the global side: that slot holds logical chunk
  // (s%8) ^ ((row>>1) & 7).  For this thread the row is 32*i + tid/8 and the
  // logical chunk (tid&7) ^ ((tid>>4)&7) for every i.  Rows past M (N) are
  // clamped to the last valid row: their results are never stored.  Offsets
  // are bytes from the tile's first row; the k offset is a scalar.
  const int lrow = tid >> 3;
  const int lchunk = (tid & 7) ^ ((tid >> 4) & 7);
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A + (int64_t)m0 * lda), 0, (int)((uint32_t)rows_a * (uint32_t)lda * 2u),
      0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(B + (int64_t)n0 * K), 0, (int)((uint32_t)rows_b * (uint32_t)K * 2u),
      0x00020000);
  uint32_t aoff[8], boff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    aoff[i] = ((uint32_t)min(32 * i + lrow, rows_a - 1) * (uint32_t)lda + lchunk * 8) * 2u;
    boff[i] = ((uint32_t)min(32 * i + lrow, rows_b - 1) * (uint32_t)K + lchunk * 8) * 2u;
  }
  // Slot i (0..15: A rows 32i.., then B): its global load, and its write
  // into an LDS stage.
  auto gload = [&](int k0, int i) -> uint4 {
    const i32x4 v = i < 8 ? __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[i], k0 * 2, 0)
                          : __builtin_amdgcn_raw_buffer_load_b128(rb, boff[i - 8], k0 * 2, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  auto lput = [&](uint16_t* adst, uint16_t* bdst, int i, uint4 v) {
    uint16_t* d = i < 8 ? adst + (256 * i + tid) * 8 : bdst + (256 * (i - 8) + tid) * 8;
    *reinterpret_cast<uint4*>(d) = v;
  };
  // LDS barrier: orders this workgroup's LDS writes and reads (waits only for
  // this wave's LDS operations, not for its global loads in flight).
  auto lds_barrier = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  typedef float f32x4 __attribute__((ext_vector_type(4)));
  f32x4 acc[8][8];   // [token block][feature block], 16 x 16 each
  const f32x4 zero4 = {};
  const int l16 = lane & 15, q4 = lane >> 4;

  // Pipeline.  Step t multiplies LDS stage t%2.  Tile t+1 waits in the
  // staging registers st[] (loaded during step t-1); step t writes it into
  // the idle stage (t+1)%2, slot by slot, and reloads each slot with tile t+2
  // right after writing it, so every global load has one full step to land.
  // The products are v_mfma_f32_16x16x32_bf16 (two 32-deep sub-steps per
  // step, 8 x 8 blocks per wave): under a sustained load on this chip they
  // keep the matrix pipe at 81% of the peak rate against 69% for
  // 32x32x16 (a register-only probe, one launch of each filling every CU for
  // tens of milliseconds).  Each sub-step is 16 fenced groups of four
  // independent MFMAs; after each come one fragment read of the next
  // sub-step and, after every second group, one slot's LDS write and reload.
  const int nk = K / BK;
  // 16 rows x 32 k: lane (row l16, k chunk 4 ks + q4) of sub-step ks.
  auto frag = [&](const uint16_t* base, int row, int ks) {
    return *reinterpret_cast<const bf16x8*>(&base[row * BK + swz(row, 4 * ks + q4) * 8]);
  };
  uint4 st[16];
  auto k_step = [&](const uint16_t* as, const uint16_t* bs, uint16_t* an, uint16_t* bn, int kt,
                    bool first) {
    const int kload = min(kt + 2, nk - 1) * BK;   // past the end: reload the last tile
    bf16x8 af[8], bfr[8], an_[8], bn_[8];
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) af[tb] = frag(as, wm * 128 + tb * 16 + l16, 0);
#pragma unroll
    for (int fb = 0; fb < 8; ++fb) bfr[fb] = frag(bs, wn * 128 + fb * 16 + l16, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
#pragma unroll
      for (int gi = 0; gi < 16; ++gi) {
        const int tb = gi >> 1, fb0 = (gi & 1) * 4;
#pragma unroll
        for (int f = 0; f < 4; ++f)
          acc[tb][fb0 + f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              bfr[fb0 + f], af[tb], (first && ks == 0) ? zero4 : acc[tb][fb0 + f], 0, 0, 0);
        if (ks + 1 < BK / 32) {
          if (gi < 8) an_[gi] = frag(as, wm * 128 + gi * 16 + l16, ks + 1);
          else bn_[gi - 8] = frag(bs, wn * 128 + (gi - 8) * 16 + l16, ks + 1);
        }
        if (gi & 1) {
          const int i = 8 * ks + (gi >> 1);
          lput(an, bn, i, st[i]);
          st[i] = gload(kload, i);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ks + 1 < BK / 32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          af[i] = an_[i];
          bfr[i] = bn_[i];
        }
      }
    }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

#pragma unroll
  for (int i = 0; i < 16; ++i) st[i] = gload(0, i);
#pragma unroll
  for (int i = 0; i < 16; ++i) lput(As0, Bs0, i, st[i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) st[i] = gload(min(1, nk - 1) * BK, i);
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  k_step(As0, Bs0, As1, Bs1, 0, true);
  for (int kt = 1; kt < nk; kt += 2) {
    k_step(As1, Bs1, As0, Bs0, kt, false);
    if (kt + 1 < nk) k_step(As0, Bs0, As1, Bs1, kt + 1, false);
  }

  // the lane's row and quarter again, from the lane id (kept from before the
  // k loop they are registers held through it)
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int qe = lane_e >> 4, le16 = lane_e & 15;

  // Epilogue.  The MFMAs computed C^T: acc[tb][fb][r] is token row
  // m0 + wm*128 + tb*16 + l16 and feature column n0 + wn*128 + fb*16 +
  // 4*q4 + r, so each lane holds 4 consecutive features of one token and
  // stores them as 8 bytes.  What depends on the column only is set up once
  // for the tile: each feature block's plane (a 16-column block never
  // straddles two: plane_cols is a multiple of 32), whether RoPE rotates it,
  // and the lane's RoPE pair frequencies and axes.
  const int ncol0 = n0 + wn * 128;   // wave-uniform
  int64_t fb_off[8];                 // element offset of the block's plane: p (plane_stride - plane_cols)
  bool fb_rot[8];
#pragma unroll
  for (int fb = 0; fb < 8; ++fb) {
    fb_off[fb] = 0;
    fb_rot[fb] = false;
    if ((KIND == 0 || kRope) && ep.plane_cols > 0) {
      const int plane = (ncol0 + fb * 16) / ep.plane_cols;
      fb_off[fb] = (int64_t)plane * (ep.plane_stride - ep.plane_cols);
      fb_rot[fb] = kRope && plane < 2;
    }
  }
  const bool has_bias = ep.bias != nullptr;
  // RoPE (kinds 3, 4): the lane's 4 columns of block fb are pairs j and j + 1
  // of a head, j = 8 (fb mod DH/16) + 2 qe (plane bases and n0 are multiples
  // of the head width); slot jj = 2 (fb mod DH/16) + t holds pair j + t.
  constexpr int kRopeDH = KIND == 4 ? 64 : 128;
  constexpr int kNJ = kRope ? kRopeDH / 8 : 1;
  float rrev[kNJ];
  int rax[kNJ];
#pragma unroll
  for (int jj = 0; jj < kNJ; ++jj) {
    rrev[jj] = 0.0f;
    rax[jj] = 0;
    if constexpr (kRope) {
      const int j0 = 8 * (jj >> 1) + (jj & 1);   // qe = 0
      const float r0 = ep.rope_rev[j0], r1 = ep.rope_rev[j0 + 2];
      const float r2 = ep.rope_rev[j0 + 4], r3 = ep.rope_rev[j0 + 6];
      rrev[jj] = qe == 0 ? r0 : (qe == 1 ? r1 : (qe == 2 ? r2 : r3));
      const int j = j0 + 2 * qe;
      rax[jj] = j < ep.pair_h ? 0 : (j < ep.pair_w ? 1 : 2);
    }
  }

  // Every global input of the epilogue is loaded ahead of the stores that
  // precede its use in program order (left in place, each load waits behind
  // the previous block's stores, which may alias it, and its latency is
  // paid once per 16x16 block): the bias of the lane's columns and the rows'
  // modality once, the residual, gate and positions of token block tb + 1
  // while block tb is computed.  The x elements a lane uses are exactly the
  // ones it later writes, so an output written over x stays correct.
  // (An opaque copy of the bias pointer keeps its loads after the k loop:
  // issued before it, their registers are held through it and spill.)
  const uint16_t* bias_p = ep.bias;
  asm volatile("" : "+s"(bias_p));
  // Loads past the last row or column read the last one instead (no
  // branch around them; their values go unused).
  uint2 bv[8];
  if (has_bias) {
#pragma unroll
    for (int fb = 0; fb < 8; ++fb)
      bv[fb] = *reinterpret_cast<const uint2*>(bias_p + min(ncol0 + fb * 16 + 4 * qe, N - 4));
  }
  int mrow[8];
  if constexpr (KIND == 1) {
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) mrow[tb] = ep.mod[min(m0 + wm * 128 + tb * 16 + le16, M - 1)];
  }
  constexpr int kNX = KIND == 1 ? 8 : 1;
  uint2 xin[2][kNX];
  float4 gin[2][kNX];
  float rp[2][3];
  auto load_tb = [&](int tb, int sl) __attribute__((always_inline)) {
    const int row = min(m0 + wm * 128 + tb * 16 + le16, M - 1);
    if constexpr (KIND == 1) {
      const uint16_t* xrow = ep.x + (int64_t)row * ep.ld_x;
      const float* grow = ep.gate + mrow[tb] * ep.gate_stride;
#pragma unroll
      for (int fb = 0; fb < 8; ++fb) {
        const int col = min(ncol0 + fb * 16 + 4 * qe, N - 4);
        xin[sl][fb] = *reinterpret_cast<const uint2*>(xrow + col);
        gin[sl][fb] = *reinterpret_cast<const float4*>(grow + col);
      }
    }
    if constexpr (kRope) {
#pragma unroll
      for (int a = 0; a < 3; ++a) rp[sl][a] = (float)ep.pos[3 * (int64_t)row + a];
    }
  };
  load_tb(0, 0);
#pragma unroll
  for (int tb = 0; tb < 8; ++tb) {
    const int sl = tb & 1;
    if (tb + 1 < 8) load_tb(tb + 1, sl ^ 1);
    const int row = m0 + wm * 128 + tb * 16 + le16;
    if (row >= M) continue;
    uint16_t* crow = C + (int64_t)row * ldc;
#pragma unroll
    for (int fb = 0; fb < 8; ++fb) {
      const int col = ncol0 + fb * 16 + 4 * qe;
      if (col >= N) continue;
      // The block's accumulators move to VGPRs here, one block at a time
      // (left alone the compiler copies all 256 out of the AGPRs at once and
      // spills).
      f32x4 blk = acc[tb][fb];
      asm volatile("" : "+v"(blk));
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = blk[e];
      if (has_bias) {
        const uint2 b = bv[fb];
        v[0] += bf16lo(b.x); v[1] += bf16hi(b.x); v[2] += bf16lo(b.y); v[3] += bf16hi(b.y);
      }
      if constexpr (KIND == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = gelu_tanh_fast(v[e]);
      }
      if constexpr (KIND == 1) {
        const uint2 xv = xin[sl][fb];
        const float4 gt = gin[sl][fb];
        v[0] = fmaf(gt.x, v[0], bf16lo(xv.x));
        v[1] = fmaf(gt.y, v[1], bf16hi(xv.x));
        v[2] = fmaf(gt.z, v[2], bf16lo(xv.y));
        v[3] = fmaf(gt.w, v[3], bf16hi(xv.y));
      }
      if constexpr (kRope) {
        if (fb_rot[fb]) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int jj = 2 * (fb % (kRopeDH / 16)) + t;
            const float p = rax[jj] == 0 ? rp[sl][0] : (rax[jj] == 1 ? rp[sl][1] : rp[sl][2]);
            float turns = p * rrev[jj];
            turns -= rintf(turns);                      // exact: |turns| < 2^23
            const float sn = __builtin_amdgcn_sinf(turns);
            const float cs = __builtin_amdgcn_cosf(turns);
            const float u = v[2 * t], w = v[2 * t + 1];
            // position 0 leaves the pair exactly as it is (a non-finite one too)
            v[2 * t] = p != 0.0f ? fmaf(u, cs, -w * sn) : u;
            v[2 * t + 1] = p != 0.0f ? fmaf(u, sn, w * cs) : w;
          }
        }
      }
      *reinterpret_cast<uint2*>(crow + fb_off[fb] + col) =
          make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  }
}

// ---- FP8 path: e4m3 codes with one float32 scale per row of A and of W ----
//
// C = (decode(A) decode(W)^T) * sa[row] * sw[col] (+ bias), then the same
// three epilogues.  v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, float32
// accumulate) at twice the bf16 rate.  The tile and the LDS layout are the
// bf16 kernel's in bytes: a 64-element bf16 k-step is a 128-byte row, and so
// is a 128-code FP8 k-step, so the 256x256 tiles, the XOR-swizzled 16-byte
// chunks and the direct global -> LDS loads carry over unchanged.  A k-step
// is 2 sub-steps of 64 codes; a fragment (32 codes of one row) is two chunks,
// two 16-byte LDS reads.  Each sub-step is written as 4 fenced groups of 4
// independent MFMAs, each group followed by the next sub-step's reads of one
// A and one B block and, in the first sub-step, 4 of the next tile's 16
// global loads.
typedef int v8i32 __attribute__((ext_vector_type(8)));
constexpr int BK8 = 128;   // codes per k-step

struct EpiArgs8 {
  const float* sa;          // [M] row scales of A
  const float* sw;          // [N] row scales of W (output channels)
};

template <int KIND>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B,
    uint16_t* C, int64_t ldc, int M, int N, int K, EpiArgs ep, EpiArgs8 sc) {
  __shared__ __attribute__((aligned(16))) uint8_t As0[BM * BK8];
  __shared__ __attribute__((aligned(16))) uint8_t As1[BM * BK8];
  __shared__ __attribute__((aligned(16))) uint8_t Bs0[BN * BK8];
  __shared__ __attribute__((aligned(16))) uint8_t Bs1[BN * BK8];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords_xcd(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;

  // Global -> LDS exactly as the bf16 kernel, with 128-byte rows of codes.
  const int lrow = tid >> 3;
  const int lchunk = (tid & 7) ^ ((tid >> 4) & 7);
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(A + (int64_t)m0 * lda), 0, (int)((uint32_t)rows_a * (uint32_t)lda),
      0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(B + (int64_t)n0 * K), 0, (int)((uint32_t)rows_b * (uint32_t)K),
      0x00020000);
  uint32_t aoff[8], boff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    aoff[i] = (uint32_t)min(32 * i + lrow, rows_a - 1) * (uint32_t)lda + lchunk * 16;
    boff[i] = (uint32_t)min(32 * i + lrow, rows_b - 1) * (uint32_t)K + lchunk * 16;
  }
  auto load1 = [&](uint8_t* adst, uint8_t* bdst, int k0, int i) {
    if (i < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, adst + (256 * i + 64 * wave) * 16, 16, aoff[i],
                                               k0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, bdst + (256 * (i - 8) + 64 * wave) * 16, 16,
                                               boff[i - 8], k0, 0, 0);
  };
  auto issue = [&](uint8_t* adst, uint8_t* bdst, int k0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) load1(adst, bdst, k0, i);
  };

  f32x16 acc[4][4];
  const f32x16 zero16 = {};
  const int nk = K / BK8;
  // Fragment of sub-step ks for a row: codes 64ks + 32g .. +31 = chunks
  // 4ks + 2g and 4ks + 2g + 1 of the row.
  auto frag = [&](const uint8_t* base, int row, int ks) {
    const uint4 lo = *reinterpret_cast<const uint4*>(&base[row * BK8 + swz(row, 4 * ks + 2 * g) * 16]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&base[row * BK8 + swz(row, 4 * ks + 2 * g + 1) * 16]);
    return v8i32{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
                 (int)hi.w};
  };
  auto k_step = [&](const uint8_t* as, const uint8_t* bs, uint8_t* an, uint8_t* bn, int kt,
                    bool first) {
    const int kload = min(kt + 1, nk - 1) * BK8;   // last step: reload into the idle buffer
    v8i32 af[4], bfr[4], an_[4], bn_[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) af[mb] = frag(as, wm * 128 + mb * 32 + l32, 0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) bfr[nb] = frag(bs, wn * 128 + nb * 32 + l32, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < BK8 / 64; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              bfr[nb], af[mb], (first && ks == 0) ? zero16 : acc[mb][nb], 0, 0, 0, 0, 0, 0);
        if (ks + 1 < BK8 / 64) {
          an_[mb] = frag(as, wm * 128 + mb * 32 + l32, ks + 1);
          bn_[mb] = frag(bs, wn * 128 + mb * 32 + l32, ks + 1);
        }
        if (ks == 0) {                   // the 16 loads: four per group, first sub-step
#pragma unroll
          for (int j = 0; j < 4; ++j) load1(an, bn, kload, 4 * mb + j);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ks + 1 < BK8 / 64) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          af[i] = an_[i];
          bfr[i] = bn_[i];
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  issue(As0, Bs0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  k_step(As0, Bs0, As1, Bs1, 0, true);
  for (int kt = 1; kt < nk; kt += 2) {
    k_step(As1, Bs1, As0, Bs0, kt, false);
    if (kt + 1 < nk) k_step(As0, Bs0, As1, Bs1, kt + 1, false);
  }

  // Epilogue: acc^T as in the bf16 kernel, times the row scale of A and the
  // column scales of W, then the bias and the epilogue kind.  Each 32-column
  // block's plane offset, p (plane_stride - plane_cols), is set up once.
  int64_t nb_off[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    nb_off[nb] = 0;
    if (KIND == 0 && ep.plane_cols > 0) {
      const int plane = (n0 + wn * 128 + nb * 32) / ep.plane_cols;
      nb_off[nb] = (int64_t)plane * (ep.plane_stride - ep.plane_cols);
    }
  }
  // Global inputs are loaded ahead of the stores (as in the bf16 kernel):
  // the column scales and bias of the lane's 16 column groups and every
  // row's scale and modality once, then each row's residual and gate before
  // any of that row's stores.  Past the last row or column the loads read
  // the last one (their values go unused).
  // (An opaque copy of the scale pointer keeps these loads after the k loop:
  // issued before it, their registers are held through it and spill.)
  const float* sw_p = sc.sw;
  asm volatile("" : "+s"(sw_p));
  float4 swv[4][4];
  uint2 bv[4][4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = min(n0 + wn * 128 + nb * 32 + r * 8 + g * 4, N - 4);
      swv[nb][r] = *reinterpret_cast<const float4*>(sw_p + col);
      if (ep.bias) bv[nb][r] = *reinterpret_cast<const uint2*>(ep.bias + col);
    }
  float sav[4];
  int modv[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int rowc = min(m0 + wm * 128 + mb * 32 + l32, M - 1);
    sav[mb] = sc.sa[rowc];
    if constexpr (KIND == 1) modv[mb] = ep.mod[rowc];
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int row = m0 + wm * 128 + mb * 32 + l32;
    const float sa = sav[mb];
    uint16_t* crow = C + (int64_t)row * ldc;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      // the residual and gate of this 32-column group, before its stores
      constexpr int kNX = KIND == 1 ? 4 : 1;
      uint2 xin[kNX];
      float4 gin[kNX];
      if constexpr (KIND == 1) {
        const uint16_t* xrow = ep.x + (int64_t)min(row, M - 1) * ep.ld_x;
        const float* grow = ep.gate + modv[mb] * ep.gate_stride;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int col = min(n0 + wn * 128 + nb * 32 + r * 8 + g * 4, N - 4);
          xin[r] = *reinterpret_cast<const uint2*>(xrow + col);
          gin[r] = *reinterpret_cast<const float4*>(grow + col);
        }
      }
      if (row >= M) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = n0 + wn * 128 + nb * 32 + r * 8 + g * 4;
        if (col >= N) continue;
        const float4 sw = swv[nb][r];
        float v[4] = {acc[mb][nb][4 * r + 0] * sa * sw.x, acc[mb][nb][4 * r + 1] * sa * sw.y,
                      acc[mb][nb][4 * r + 2] * sa * sw.z, acc[mb][nb][4 * r + 3] * sa * sw.w};
        if (ep.bias) {
          const uint2 b = bv[nb][r];
          v[0] += bf16lo(b.x); v[1] += bf16hi(b.x); v[2] += bf16lo(b.y); v[3] += bf16hi(b.y);
        }
        if constexpr (KIND == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = gelu_tanh_fast(v[e]);
        }
        if constexpr (KIND == 1) {
          const uint2 xv = xin[r];
          const float4 gt = gin[r];
          v[0] = fmaf(gt.x, v[0], bf16lo(xv.x));
          v[1] = fmaf(gt.y, v[1], bf16hi(xv.x));
          v[2] = fmaf(gt.z, v[2], bf16lo(xv.y));
          v[3] = fmaf(gt.w, v[3], bf16hi(xv.y));
        }
        *reinterpret_cast<uint2*>(crow + nb_off[nb] + col) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
}

// Per-row quantization: one wave per row, the row held in registers (NV
// 16-byte vectors per lane), scale = amax / 448 and inv = 1 / scale (IEEE
// divisions, once per row), codes of x * inv (one float32 product per value),
// 4-code stores.
template <typename T, int NV>
__global__ __launch_bounds__(256) void quant_rows_kernel(const T* __restrict__ x, int64_t ld_x,
                                                         uint8_t* __restrict__ q, int64_t ld_q,
                                                         float* __restrict__ scales, int64_t n,
                                                         int d) {
  constexpr int E = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const int nvec = d / E;
  uint4 raw[NV];
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * ld_x);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    raw[i] = c < nvec ? ld_stream(xr + c) : make_uint4(0, 0, 0, 0);
  }
  auto unpack = [&](const uint4& r, float* f) {
    if constexpr (E == 8) {
      f[0] = bf16lo(r.x); f[1] = bf16hi(r.x); f[2] = bf16lo(r.y); f[3] = bf16hi(r.y);
      f[4] = bf16lo(r.z); f[5] = bf16hi(r.z); f[6] = bf16lo(r.w); f[7] = bf16hi(r.w);
    } else {
      f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
      f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
    }
  };
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float f[E];
    unpack(raw[i], f);
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(f[e]));
  }
  amax = wave_max(amax);
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  const float inv = 1.0f / s;
  if (lane == 0) scales[row] = s;
  uint8_t* qr = q + row * ld_q;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c >= nvec) continue;
    float f[E];
    unpack(raw[i], f);
    uint32_t w[E / 4];
#pragma unroll
    for (int j = 0; j < E / 4; ++j)
      w[j] = e4m3_pack4(f[4 * j] * inv, f[4 * j + 1] * inv, f[4 * j + 2] * inv, f[4 * j + 3] * inv);
    if constexpr (E == 8)
      *reinterpret_cast<uint2*>(qr + c * E) = make_uint2(w[0], w[1]);
    else
      *reinterpret_cast<uint32_t*>(qr + c * E) = w[0];
  }
}

// ---- float32 path ----
constexpr int FT = 64, FK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                        const float* __restrict__ B,
                                                        float* C, int64_t ldc, int M,
                                                        int N, int K, const float* bias,
                                                        int kind, const float* x, int64_t ld_x,
                                                        const uint8_t* mod, const float* gate,
                                                        int64_t gate_stride, int plane_cols,
                                                        int64_t plane_stride) {
  __shared__ float As[FK][FT + 1];
  __shared__ float Bs[FK][FT + 1];
  const int m0 = blockIdx.y * FT, n0 = blockIdx.x * FT;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FK) {
    for (int i = threadIdx.x; i < FT * FK; i += 256) {
      const int r = i / FK, c = i % FK;
      As[c][r] = (m0 + r < M) ? A[(int64_t)(m0 + r) * lda + k0 + c] : 0.0f;
      Bs[c][r] = (n0 + r < N) ? B[(int64_t)(n0 + r) * K + k0 + c] : 0.0f;
    }
    __syncthreads();
    for (int kk = 0; kk < FK; ++kk) {
      float a[4], b[4];
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= M) continue;
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      float v = acc[i][j] + (bias ? bias[col] : 0.0f);
      if (kind == 2) v = gelu_tanh_exact(v);
      if (kind == 1) v = fmaf(gate[mod[row] * gate_stride + col], v, x[(int64_t)row * ld_x + col]);
      const int plane = plane_cols > 0 ? col / plane_cols : 0;
      C[plane * plane_stride + (int64_t)row * ldc + (col - plane * plane_cols)] = v;
    }
  }
}

}  // namespace

hipError_t launch_gemm(int bf16, const void* a, int64_t lda, const void* b, void* c, int64_t ldc,
                       int64_t m, int n, int k, const GemmEpilogue& ep, hipStream_t s) {
  if (k % BK != 0 || m > INT32_MAX) return hipErrorInvalidValue;
  const bool rope = ep.kind == 3;
  if (ep.plane_cols < 0 || ep.plane_cols % 32 != 0 ||
      (ep.plane_cols > 0 && ep.kind != 0 && !rope))
    return hipErrorInvalidValue;
  if (rope && (!bf16 || !ep.pos || !ep.rope_freq || (ep.rope_dh != 64 && ep.rope_dh != 128) ||
               ep.plane_cols <= 0 || ep.plane_cols % ep.rope_dh != 0 || n % ep.rope_dh != 0))
    return hipErrorInvalidValue;
  // gate rows of the table are 3*N floats apart (table [3][3][N], N = d_model)
  const int64_t gate_stride = 3 * (int64_t)n;
  if (bf16) {
    const int tiles = (int)((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    EpiArgs e{ep.kind, static_cast<const uint16_t*>(ep.bias), static_cast<const uint16_t*>(ep.x),
              ep.ld_x, ep.mod, ep.gate, gate_stride, ep.plane_cols, ep.plane_stride, ep.pos,
              ep.rope_pair_h, ep.rope_pair_w, {}};
    if (rope) {
      constexpr double kTwoPi = 6.283185307179586476925;
      for (int j = 0; j < 64; ++j)
        e.rope_rev[j] = j < ep.rope_dh / 2 ? (float)(ep.rope_freq[j] / kTwoPi) : 0.0f;
    }
    if (rope && ep.rope_dh == 128)
      gemm_bf16_kernel<3><<<dim3(tiles), dim3(kThreads), 0, s>>>(
          static_cast<const uint16_t*>(a), lda, static_cast<const uint16_t*>(b),
          static_cast<uint16_t*>(c), ldc, (int)m, n, k, e);
    else if (rope)
      gemm_bf16_kernel<4><<<dim3(tiles), dim3(kThreads), 0, s>>>(
          static_cast<const uint16_t*>(a), lda, static_cast<const uint16_t*>(b),
          static_cast<uint16_t*>(c), ldc, (int)m, n, k, e);
    else if (ep.kind == 1)
      gemm_bf16_kernel<1><<<dim3(tiles), dim3(kThreads), 0, s>>>(
          static_cast<const uint16_t*>(a), lda, static_cast<const uint16_t*>(b),
          static_cast<uint16_t*>(c), ldc, (int)m, n, k, e);
    else if (ep.kind == 2)
      gemm_bf16_kernel<2><<<dim3(tiles), dim3(kThreads), 0, s>>>(
          static_cast<const uint16_t*>(a), lda, static_cast<const uint16_t*>(b),
          static_cast<uint16_t*>(c), ldc, (int)m, n, k, e);
    else
      gemm_bf16_kernel<0><<<dim3(tiles), dim3(kThreads), 0, s>>>(
          static_cast<const uint16_t*>(a), lda, static_cast<const uint16_t*>(b),
          static_cast<uint16_t*>(c), ldc, (int)m, n, k, e);
  } else {
    const dim3 grid((n + FT - 1) / FT, (unsigned)((m + FT - 1) / FT));
    gemm_f32_kernel<<<grid, dim3(256), 0, s>>>(
        static_cast<const float*>(a), lda, static_cast<const float*>(b), static_cast<float*>(c),
        ldc, (int)m, n, k, static_cast<const float*>(ep.bias), ep.kind,
        static_cast<const float*>(ep.x), ep.ld_x, ep.mod, ep.gate, gate_stride, ep.plane_cols,
        ep.plane_stride);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const uint8_t* a, int64_t lda, const float* sa, const uint8_t* w,
                           const float* sw, void* c, int64_t ldc, int64_t m, int n, int k,
                           const GemmEpilogue& ep, hipStream_t s) {
  if (k % BK8 != 0 || m > INT32_MAX) return hipErrorInvalidValue;
  if (ep.plane_cols < 0 || ep.plane_cols % 32 != 0 || (ep.plane_cols > 0 && ep.kind != 0))
    return hipErrorInvalidValue;
  if (ep.kind == 3) return hipErrorInvalidValue;
  const int64_t gate_stride = 3 * (int64_t)n;
  const int tiles = (int)((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  EpiArgs e{ep.kind, static_cast<const uint16_t*>(ep.bias), static_cast<const uint16_t*>(ep.x),
            ep.ld_x, ep.mod, ep.gate, gate_stride, ep.plane_cols, ep.plane_stride, nullptr, 0, 0,
            {}};
  EpiArgs8 e8{sa, sw};
  uint16_t* cp = static_cast<uint16_t*>(c);
  if (ep.kind == 1)
    gemm_fp8_kernel<1><<<dim3(tiles), dim3(kThreads), 0, s>>>(a, lda, w, cp, ldc, (int)m, n, k, e, e8);
  else if (ep.kind == 2)
    gemm_fp8_kernel<2><<<dim3(tiles), dim3(kThreads), 0, s>>>(a, lda, w, cp, ldc, (int)m, n, k, e, e8);
  else
    gemm_fp8_kernel<0><<<dim3(tiles), dim3(kThreads), 0, s>>>(a, lda, w, cp, ldc, (int)m, n, k, e, e8);
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp8(int bf16, const void* x, int64_t ld_x, uint8_t* q, int64_t ld_q,
                                 float* scales, int64_t n, int d, hipStream_t s) {
  const int e = bf16 ? 8 : 4;
  if (d % e != 0) return hipErrorInvalidValue;
  const int need = (d / e + 63) / 64;
  const dim3 grid((unsigned)((n + 3) / 4)), block(256);
#define DIT_QUANT_CASE(NVV)                                                                     \
  if (need <= NVV) {                                                                            \
    if (bf16)                                                                                   \
      quant_rows_kernel<uint16_t, NVV><<<grid, block, 0, s>>>(                                  \
          static_cast<const uint16_t*>(x), ld_x, q, ld_q, scales, n, d);                        \
    else                                                                                        \
      quant_rows_kernel<float, NVV><<<grid, block, 0, s>>>(static_cast<const float*>(x), ld_x,  \
                                                           q, ld_q, scales, n, d);              \
    return hipGetLastError();                                                                   \
  }
  DIT_QUANT_CASE(1) DIT_QUANT_CASE(2) DIT_QUANT_CASE(4) DIT_QUANT_CASE(8) DIT_QUANT_CASE(10)
  DIT_QUANT_CASE(12)
  DIT_QUANT_CASE(16) DIT_QUANT_CASE(24) DIT_QUANT_CASE(32) DIT_QUANT_CASE(40)
#undef DIT_QUANT_CASE
  return hipErrorInvalidValue;
}

}  // namespace dit
