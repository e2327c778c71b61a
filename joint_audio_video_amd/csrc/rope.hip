// 3D (time, height, width) rotary position embedding of q and k, in place.
//
// [H3-NFT] section "MiniMax H3 and Why Joint Audio-Video Generation Complicates
// RL Training": RoPE over the three axes time, height and width.  [vLLM-Omni]
// section 3: every row carries its (t, h, w) position, and the modality tag
// keeps the position spaces of the modalities independent (audio and text
// rows sit on the time axis only, so their h and w sections never turn).
//
// head_dim splits into sections (s_t, s_h, s_w); pair p = (2p, 2p+1) of a head
// belongs to one section and turns by phi = pos[axis] * theta^(-2j / s_axis).
// The angle and its cosine/sine are computed once per (token, pair) in double
// precision into LDS and reused by every head of q and k; a pair whose angle
// is zero is copied bit-identically.  HBM-bound: each q/k row is read and
// written once with 16-byte accesses.
#include "common.h"

namespace dit {
namespace {

struct Freqs {
  double f[64];
};

template <typename T> struct VecE;
template <> struct VecE<uint16_t> { static constexpr int N = 8; };
template <> struct VecE<float> { static constexpr int N = 4; };

__device__ __forceinline__ void load_vec(const uint4& r, float* f, uint16_t) {
  f[0] = bf16lo(r.x); f[1] = bf16hi(r.x); f[2] = bf16lo(r.y); f[3] = bf16hi(r.y);
  f[4] = bf16lo(r.z); f[5] = bf16hi(r.z); f[6] = bf16lo(r.w); f[7] = bf16hi(r.w);
}
__device__ __forceinline__ void load_vec(const uint4& r, float* f, float) {
  f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
  f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
}
__device__ __forceinline__ uint4 store_vec(const float* f, uint16_t) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                    pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}
__device__ __forceinline__ uint4 store_vec(const float* f, float) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                    __float_as_uint(f[2]), __float_as_uint(f[3]));
}

constexpr int kThreads = 256;

template <typename T, int DH>
__global__ __launch_bounds__(kThreads) void rope_kernel(T* __restrict__ q, int64_t ld_q,
                                                         T* __restrict__ k, int64_t ld_k,
                                                         const int32_t* __restrict__ pos,
                                                         int64_t n, int n_heads, int s_t,
                                                         int s_h, Freqs fr) {
  constexpr int P = DH / 2;             // pairs per head
  constexpr int TOK = kThreads / P;     // tokens per workgroup
  constexpr int E = VecE<T>::N;         // elements per 16-byte vector
  __shared__ float2 cs[TOK][P];

  const int64_t t0 = (int64_t)blockIdx.x * TOK;
  {
    const int tok = threadIdx.x / P, p = threadIdx.x % P;
    const int64_t row = t0 + tok;
    float c = 1.0f, s = 0.0f;
    if (row < n) {
      const int col = 2 * p;
      const int axis = col < s_t ? 0 : (col < s_t + s_h ? 1 : 2);
      const int32_t ps = pos[3 * row + axis];
      if (ps != 0) {
        double sd, cd;
        sincos((double)ps * fr.f[p], &sd, &cd);
        s = (float)sd;
        c = (float)cd;
      }
    }
    cs[tok][p] = make_float2(c, s);
  }
  __syncthreads();

  const int nv = n_heads * DH / E;                  // vectors per q (or k) row
  const int items = TOK * 2 * nv;
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int tok = it / (2 * nv);
    const int rem = it - tok * 2 * nv;
    const int which = rem / nv;                     // 0: q, 1: k
    const int v = rem - which * nv;
    const int64_t row = t0 + tok;
    if (row >= n) continue;
    if (which == 1 && k == nullptr) continue;
    T* base = which == 0 ? q + row * ld_q : k + row * ld_k;
    uint4* ptr = reinterpret_cast<uint4*>(base) + v;
    const uint4 raw = *ptr;
    float f[E];
    load_vec(raw, f, T());
    const int p0 = ((v * E) % DH) / 2;
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
      const float2 r = cs[tok][p0 + j];
      const float u = f[2 * j], w = f[2 * j + 1];
      if (r.y != 0.0f) {
        f[2 * j] = fmaf(u, r.x, -w * r.y);
        f[2 * j + 1] = fmaf(u, r.y, w * r.x);
      }
    }
    *ptr = store_vec(f, T());
  }
}

template <typename T>
hipError_t dispatch(void* q, int64_t ld_q, void* k, int64_t ld_k, const int32_t* pos, int64_t n,
                    int n_heads, int head_dim, int s_t, int s_h, const double* freq,
                    hipStream_t s) {
  Freqs fr;
  for (int p = 0; p < 64; ++p) fr.f[p] = p < head_dim / 2 ? freq[p] : 0.0;
  T* qp = static_cast<T*>(q);
  T* kp = static_cast<T*>(k);
  if (head_dim == 128) {
    constexpr int TOK = kThreads / 64;
    rope_kernel<T, 128><<<dim3((unsigned)((n + TOK - 1) / TOK)), dim3(kThreads), 0, s>>>(
        qp, ld_q, kp, ld_k, pos, n, n_heads, s_t, s_h, fr);
  } else if (head_dim == 64) {
    constexpr int TOK = kThreads / 32;
    rope_kernel<T, 64><<<dim3((unsigned)((n + TOK - 1) / TOK)), dim3(kThreads), 0, s>>>(
        qp, ld_q, kp, ld_k, pos, n, n_heads, s_t, s_h, fr);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(int bf16, void* q, int64_t ld_q, void* k, int64_t ld_k,
                       const int32_t* pos, int64_t n, int n_heads, int head_dim, int s_t,
                       int s_h, const double* freq_d, hipStream_t s) {
  return bf16 ? dispatch<uint16_t>(q, ld_q, k, ld_k, pos, n, n_heads, head_dim, s_t, s_h, freq_d,
                                   s)
              : dispatch<float>(q, ld_q, k, ld_k, pos, n, n_heads, head_dim, s_t, s_h, freq_d, s);
}

}  // namespace dit
