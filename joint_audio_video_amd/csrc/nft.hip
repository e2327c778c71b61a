// DiffusionNFT loss over a packed batch of samples, with the gradient of the
// batch objective with respect to the policy's velocity, in three
// deterministic launches (no atomics).
//
// [VeRL-Omni] section 4 (implicit policies and the scalar-reward loss):
//   v_pos = beta v_theta + (1 - beta) v_old,  v_neg = (1 + beta) v_old - beta v_theta,
//   L_s = r_s MSE(v_pos, v_target) + (1 - r_s) MSE(v_neg, v_target).
// [H3-NFT] section "FL2VA: First-Frame Conditioning With Shared
// Infrastructure": condition-frame rows are masked out of the loss.
// [VeRL-Omni] section 5.1: H3's velocity is sign-reversed (velocity_sign).
//
// With d = v_theta - v_old and a = v_old - v_target (after the sign):
//   v_pos - v_target = a + beta d,   v_neg - v_target = a - beta d,
//   dL_s/dv_theta = (2 beta / n_s) (r_s (a + beta d) - (1 - r_s)(a - beta d)),
// n_s = loss-bearing rows of sample s times the channel count.
//
// 1. count: a block per sample counts its loss-bearing rows (16-byte mask
//    reads) into the workspace.
// 2. main: a block per (32-row chunk, sample) streams its chunk once: read
//    v_theta, v_old, v_target, write the gradient, and reduce the chunk's two
//    squared-error sums into the workspace.
// 3. finalize: a block per sample adds its chunks' sums in float64 in a fixed
//    order and writes (loss, mse_pos, mse_neg).
// HBM-bound: a thread owns 4 consecutive channels of one row (16-byte float
// accesses, 8-byte bf16 loads), threads walk the chunk's flattened
// (row, 4-channel group) index.
#include "common.h"

namespace dit {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkRows = 32;   // measured best of 16..256 rows (16 packs, 96 channels)
constexpr int kUnroll = 2;       // measured best of 2, 4, 8

template <typename T>
__device__ __forceinline__ T block_sum(T v, T* red) {
  // red: LDS scratch of kThreads / 64 elements
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  T t = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) t += red[w];
  return t;
}

constexpr int kCountThreads = 1024;

// Nonzero bytes of a 32-bit word.
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  return ((w & 0xffu) != 0) + ((w & 0xff00u) != 0) + ((w & 0xff0000u) != 0) + ((w >> 24) != 0);
}

__global__ __launch_bounds__(kCountThreads) void nft_count_kernel(const uint8_t* __restrict__ mask,
                                                                  const int32_t* __restrict__ cu,
                                                                  int32_t* __restrict__ totals) {
  __shared__ int red[kCountThreads / 64];
  const int s = blockIdx.x;
  const int seg0 = cu[s], seg1 = cu[s + 1];
  int k = 0;
  if (!mask) {
    k = threadIdx.x == 0 ? seg1 - seg0 : 0;
  } else {
    // bytes up to the first 16-byte boundary, 16-byte words, then the tail
    const uintptr_t base = (uintptr_t)mask;
    const int head_end =
        min(seg1, (int)((((uintptr_t)(mask + seg0) + 15) & ~(uintptr_t)15) - base));
    const int n16 = (seg1 - head_end) / 16;
    const int tail0 = head_end + 16 * n16;
    for (int r = seg0 + (int)threadIdx.x; r < head_end; r += kCountThreads) k += mask[r] != 0;
    const uint4* m16 = reinterpret_cast<const uint4*>(mask + head_end);
    for (int i = threadIdx.x; i < n16; i += kCountThreads) {
      const uint4 w = m16[i];
      k += nonzero_bytes(w.x) + nonzero_bytes(w.y) + nonzero_bytes(w.z) + nonzero_bytes(w.w);
    }
    for (int r = tail0 + (int)threadIdx.x; r < seg1; r += kCountThreads) k += mask[r] != 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) k += __shfl_xor(k, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < kCountThreads / 64; ++w) t += red[w];
    totals[s] = t;
  }
}

template <bool kBf16>
__device__ __forceinline__ f32x4 load_v4(const void* p, int64_t off) {
  if constexpr (kBf16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + off);
    return f32x4{bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y)};
  } else {
    const uint4 w = ld_stream(static_cast<const float*>(p) + off);
    return f32x4{__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                 __uint_as_float(w.w)};
  }
}

struct NftArgs {
  const void* vt;
  int64_t ld_vt;
  const void* vo;
  int64_t ld_vo;
  const float* tg;
  int64_t ld_t;
  const uint8_t* mask;
  const int32_t* cu;
  const float* reward;
  float* grad;
  int64_t ld_g;
  const int32_t* totals;  // [S] loss-bearing rows
  float* partials;       // [S][chunks][2]
  int chunks;
  int groups;            // channels / 4
  float beta, sign, scale;
};

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void nft_main_kernel(NftArgs a) {
  __shared__ float fred[kThreads / 64];
  const int s = blockIdx.y, c = blockIdx.x;
  const int seg0 = a.cu[s], seg1 = a.cu[s + 1];
  const int r0 = seg0 + c * kChunkRows;
  if (r0 >= seg1) return;
  const int r1 = min(seg1, r0 + kChunkRows);
  const int kept = a.totals[s];
  const float r = a.reward[s];
  // gradient factor: scale * sign * 2 beta / n_s (n_s > 0 whenever a row here is kept)
  const float coef = kept > 0 ? a.scale * a.sign * 2.0f * a.beta / ((float)kept * (float)(4 * a.groups))
                              : 0.0f;
  const float wp = coef * r, wn = coef * (1.0f - r);
  float sp = 0.0f, sn = 0.0f;
  const int total = (r1 - r0) * a.groups;
  // kUnroll groups per thread per pass, all loads issued before any arithmetic
  // (memory-level parallelism for an HBM-bound pass).
  for (int base = threadIdx.x; base < total; base += kUnroll * kThreads) {
    f32x4 vt[kUnroll], vo[kUnroll], t[kUnroll];
    int64_t goff[kUnroll];
    bool live[kUnroll], keep[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int idx = base + u * kThreads;
      live[u] = idx < total;
      const int rr = live[u] ? idx / a.groups : 0;
      const int row = r0 + rr;
      const int col = (idx - rr * a.groups) * 4;
      keep[u] = live[u] && (!a.mask || a.mask[row] != 0);
      goff[u] = (int64_t)row * a.ld_g + col;
      if (keep[u]) {
        vt[u] = load_v4<kBf16>(a.vt, (int64_t)row * a.ld_vt + col);
        vo[u] = load_v4<kBf16>(a.vo, (int64_t)row * a.ld_vo + col);
        const uint4 tw = ld_stream(a.tg + (int64_t)row * a.ld_t + col);
        t[u] = f32x4{__uint_as_float(tw.x), __uint_as_float(tw.y), __uint_as_float(tw.z),
                     __uint_as_float(tw.w)};
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (!live[u]) continue;
      f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f};
      if (keep[u]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d = a.sign * (vt[u][e] - vo[u][e]);
          const float av = fmaf(a.sign, vo[u][e], -t[u][e]);
          const float ep = fmaf(a.beta, d, av);
          const float en = fmaf(-a.beta, d, av);
          sp = fmaf(ep, ep, sp);
          sn = fmaf(en, en, sn);
          g[e] = fmaf(wp, ep, -wn * en);
        }
      }
      if (a.grad)
        st_stream(a.grad + goff[u], make_uint4(__float_as_uint(g[0]), __float_as_uint(g[1]),
                                               __float_as_uint(g[2]), __float_as_uint(g[3])));
    }
  }
  sp = block_sum(sp, fred);
  sn = block_sum(sn, fred);
  if (threadIdx.x == 0) {
    float* p = a.partials + ((size_t)s * a.chunks + c) * 2;
    p[0] = sp;
    p[1] = sn;
  }
}

__global__ __launch_bounds__(64) void nft_finalize_kernel(const int32_t* __restrict__ cu,
                                                          const float* __restrict__ reward,
                                                          const int32_t* __restrict__ totals,
                                                          const float* __restrict__ partials,
                                                          int chunks, int channels,
                                                          float* __restrict__ out) {
  const int s = blockIdx.x, lane = threadIdx.x;
  const int nchunks = (cu[s + 1] - cu[s] + kChunkRows - 1) / kChunkRows;
  double sp = 0.0, sn = 0.0;
  for (int i = lane; i < nchunks; i += 64) {
    const float* p = partials + ((size_t)s * chunks + i) * 2;
    sp += (double)p[0];
    sn += (double)p[1];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sp += __shfl_xor(sp, off, 64);
    sn += __shfl_xor(sn, off, 64);
  }
  const int kept = totals[s];
  if (lane == 0) {
    const double n = (double)kept * (double)channels;
    const double mp = n > 0 ? sp / n : 0.0, mn = n > 0 ? sn / n : 0.0;
    const double r = (double)reward[s];
    out[3 * s + 0] = (float)(r * mp + (1.0 - r) * mn);
    out[3 * s + 1] = (float)mp;
    out[3 * s + 2] = (float)mn;
  }
}

}  // namespace

size_t nft_workspace_layout(int n_samples, int max_rows, size_t* partials_offset) {
  const size_t chunks = (size_t)((max_rows + kChunkRows - 1) / kChunkRows);
  const size_t totals_bytes = ((size_t)n_samples * 4 + 255) & ~size_t(255);
  const size_t partial_bytes = ((size_t)n_samples * chunks * 8 + 255) & ~size_t(255);
  if (partials_offset) *partials_offset = totals_bytes;
  return totals_bytes + partial_bytes;
}

hipError_t launch_nft_loss(int bf16, const void* v_theta, int64_t ld_vt, const void* v_old,
                           int64_t ld_vo, const float* v_target, int64_t ld_t,
                           const uint8_t* mask, const int32_t* cu, int n_samples, int max_rows,
                           int channels, const float* reward, float beta, float sign,
                           float scale, float* grad, int64_t ld_g, float* loss_out,
                           void* workspace, hipStream_t s) {
  if (channels % 4 != 0 || n_samples < 1 || n_samples > 65535 || max_rows < 1)
    return hipErrorInvalidValue;
  const int chunks = (max_rows + kChunkRows - 1) / kChunkRows;
  size_t poff = 0;
  nft_workspace_layout(n_samples, max_rows, &poff);
  int32_t* totals = static_cast<int32_t*>(workspace);
  float* partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + poff);
  const dim3 grid(chunks, n_samples);
  nft_count_kernel<<<dim3(n_samples), dim3(kCountThreads), 0, s>>>(mask, cu, totals);
  NftArgs a{v_theta, ld_vt, v_old, ld_vo, v_target, ld_t, mask, cu, reward, grad, ld_g,
            totals, partials, chunks, channels / 4, beta, sign, scale};
  if (bf16)
    nft_main_kernel<true><<<grid, dim3(kThreads), 0, s>>>(a);
  else
    nft_main_kernel<false><<<grid, dim3(kThreads), 0, s>>>(a);
  nft_finalize_kernel<<<dim3(n_samples), dim3(64), 0, s>>>(cu, reward, totals, partials, chunks,
                                                         channels, loss_out);
  return hipGetLastError();
}

}  // namespace dit
