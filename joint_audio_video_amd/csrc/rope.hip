// 3D (time, height, width) rotary position embedding of q and k, in place or
// into separate outputs.
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
// written once with 16-byte accesses.  Writing to separate outputs avoids the
// read-modify-write of the same lines; an output may be the other input
// (the rotated k may go to q's rows): every vector is loaded and stored by
// the same thread, loads first.
// Shape: one workgroup per token, thread t holding vector t of the token's q
// and k rows, so the grid streams both arrays in address order with one
// vector per thread and row.  On one MI355X, copies of a 601 MB array
// sustain 81% of 8 TB/s with one 16-byte vector per thread against 71% with
// eight (and 68-71% for rows of ten vectors per lane); at 58,758 tokens x 40
// heads this form takes 396.5 us (75.9% of 8 TB/s) against 431.1 us (69.8%)
// for two tokens per 128-thread workgroup with five vectors per thread and
// row, bit-identical.  Rows wider than 1024 vectors keep that older form.
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

// Rows wider than 1024 vectors: 128 threads (two tokens per workgroup at
// head_dim 128) and up to five vectors per thread per row in one pass.
constexpr int kThreads = 128;

// Workgroup = TOK tokens.  Thread tid handles vector tid + kThreads*j of each
// of the 2*TOK rows (q and k of every token); since kThreads*E is a multiple
// of DH, its pairs p0..p0+E/2-1 within the head are the same for every j.
// Rows wider than kThreads*NJ vectors are walked in chunks.  The loads do not
// depend on the angles, so the first chunk's loads are issued before the
// angle table is computed.
// q, k: inputs; qo, ko: outputs (equal to q, k when in place).  The four
// pointers are not restrict-qualified: ko may be q.
template <typename T, int DH, int NJ>
__global__ __launch_bounds__(kThreads) void rope_kernel(const T* q, int64_t ld_q, const T* k,
                                                         int64_t ld_k, T* qo, int64_t ld_qo,
                                                         T* ko, int64_t ld_ko,
                                                         const int32_t* __restrict__ pos,
                                                         int64_t n, int n_heads, int s_t,
                                                         int s_h, Freqs fr) {
  constexpr int P = DH / 2;             // pairs per head
  constexpr int TOK = kThreads / P;     // tokens per workgroup
  constexpr int E = VecE<T>::N;         // elements per 16-byte vector
  static_assert((kThreads * E) % DH == 0, "a thread's pairs must not depend on j");
  __shared__ float2 cs[TOK][P];

  const int64_t t0 = (int64_t)blockIdx.x * TOK;
  const int nv = n_heads * DH / E;      // vectors per q (or k) row
  const int p0 = ((threadIdx.x * E) % DH) / 2;
  const T* base[TOK][2];
  T* obase[TOK][2];
  bool live[TOK][2];
#pragma unroll
  for (int tk = 0; tk < TOK; ++tk) {
    const int64_t row = t0 + tk;
    base[tk][0] = q + row * ld_q;
    base[tk][1] = k + row * ld_k;
    obase[tk][0] = qo + row * ld_qo;
    obase[tk][1] = ko + row * ld_ko;
    live[tk][0] = row < n;
    live[tk][1] = row < n && k != nullptr;
  }

  for (int vb = 0; vb < nv; vb += kThreads * NJ) {
    uint4 raw[TOK][2][NJ];
#pragma unroll
    for (int tk = 0; tk < TOK; ++tk)
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int v = vb + threadIdx.x + kThreads * j;
          raw[tk][w][j] = live[tk][w] && v < nv
                              ? ld_stream(reinterpret_cast<const uint4*>(base[tk][w]) + v)
                              : make_uint4(0, 0, 0, 0);
        }

    if (vb == 0) {
      // Angle table: thread (tk, p) computes pair p of token t0 + tk.
      const int tk = threadIdx.x / P, p = threadIdx.x % P;
      const int64_t row = t0 + tk;
      float c = 1.0f, sn = 0.0f;
      if (row < n) {
        const int col = 2 * p;
        const int axis = col < s_t ? 0 : (col < s_t + s_h ? 1 : 2);
        const int32_t ps = pos[3 * row + axis];
        if (ps != 0) {
          double sd, cd;
          sincos((double)ps * fr.f[p], &sd, &cd);
          sn = (float)sd;
          c = (float)cd;
        }
      }
      cs[tk][p] = make_float2(c, sn);
      __syncthreads();
    }

#pragma unroll
    for (int tk = 0; tk < TOK; ++tk)
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int v = vb + threadIdx.x + kThreads * j;
          if (!live[tk][w] || v >= nv) continue;
          float f[E];
          load_vec(raw[tk][w][j], f, T());
#pragma unroll
          for (int jj = 0; jj < E / 2; ++jj) {
            const float2 r = cs[tk][p0 + jj];
            const float u = f[2 * jj], x = f[2 * jj + 1];
            if (r.y != 0.0f) {
              f[2 * jj] = fmaf(u, r.x, -x * r.y);
              f[2 * jj + 1] = fmaf(u, r.y, x * r.x);
            }
          }
          st_stream(reinterpret_cast<uint4*>(obase[tk][w]) + v, store_vec(f, T()));
        }
  }
}

// Token-per-workgroup form (rows of at most 1024 vectors): thread t loads
// vector t of the token's q row and of its k row, the first DH/2 threads
// compute the token's angles into LDS, and thread t writes both rotated
// vectors (loads before stores in one thread, so ko may be q).
template <typename T, int DH>
__global__ __launch_bounds__(1024) void rope_row_kernel(const T* q, int64_t ld_q, const T* k,
                                                        int64_t ld_k, T* qo, int64_t ld_qo,
                                                        T* ko, int64_t ld_ko,
                                                        const int32_t* __restrict__ pos,
                                                        int64_t n, int n_heads, int s_t, int s_h,
                                                        Freqs fr) {
  constexpr int P = DH / 2;
  constexpr int E = VecE<T>::N;
  __shared__ float2 cs[P];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int nv = n_heads * DH / E;
  const bool live = t < nv, has_k = k != nullptr;
  const uint4 rq = live ? ld_stream(reinterpret_cast<const uint4*>(q + row * ld_q) + t)
                        : make_uint4(0, 0, 0, 0);
  const uint4 rk = live && has_k ? ld_stream(reinterpret_cast<const uint4*>(k + row * ld_k) + t)
                                 : make_uint4(0, 0, 0, 0);
  if (t < P) {
    const int col = 2 * t;
    const int axis = col < s_t ? 0 : (col < s_t + s_h ? 1 : 2);
    const int32_t ps = pos[3 * row + axis];
    float c = 1.0f, sn = 0.0f;
    if (ps != 0) {
      double sd, cd;
      sincos((double)ps * fr.f[t], &sd, &cd);
      sn = (float)sd;
      c = (float)cd;
    }
    cs[t] = make_float2(c, sn);
  }
  __syncthreads();
  if (!live) return;
  const int p0 = ((t * E) % DH) / 2;
  auto rotate = [&](const uint4& raw) {
    float f[E];
    load_vec(raw, f, T());
#pragma unroll
    for (int jj = 0; jj < E / 2; ++jj) {
      const float2 r = cs[p0 + jj];
      const float u = f[2 * jj], x = f[2 * jj + 1];
      if (r.y != 0.0f) {
        f[2 * jj] = fmaf(u, r.x, -x * r.y);
        f[2 * jj + 1] = fmaf(u, r.y, x * r.x);
      }
    }
    return store_vec(f, T());
  };
  const uint4 oq = rotate(rq);
  if (has_k) {
    const uint4 ok = rotate(rk);
    st_stream(reinterpret_cast<uint4*>(ko + row * ld_ko) + t, ok);
  }
  st_stream(reinterpret_cast<uint4*>(qo + row * ld_qo) + t, oq);
}

struct RopeIO {
  const void* q;
  int64_t ld_q;
  const void* k;
  int64_t ld_k;
  void* qo;
  int64_t ld_qo;
  void* ko;
  int64_t ld_ko;
};

template <typename T, int DH>
hipError_t launch_dh(const RopeIO& io, const int32_t* pos, int64_t n, int n_heads, int s_t,
                     int s_h, const Freqs& fr, hipStream_t s) {
  constexpr int TOK = kThreads / (DH / 2);
  const int nv = n_heads * DH / VecE<T>::N;
  const int nj = (nv + kThreads - 1) / kThreads;     // vectors per thread per row
  if (n == 0) return hipSuccess;
  if (nv <= 1024) {
    rope_row_kernel<T, DH><<<dim3((unsigned)n), dim3((unsigned)(64 * ((nv + 63) / 64))), 0, s>>>(
        static_cast<const T*>(io.q), io.ld_q, static_cast<const T*>(io.k), io.ld_k,
        static_cast<T*>(io.qo), io.ld_qo, static_cast<T*>(io.ko), io.ld_ko, pos, n, n_heads, s_t,
        s_h, fr);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((n + TOK - 1) / TOK)), block(kThreads);
  const T* q = static_cast<const T*>(io.q);
  const T* k = static_cast<const T*>(io.k);
  T* qo = static_cast<T*>(io.qo);
  T* ko = static_cast<T*>(io.ko);
#define DIT_ROPE_LAUNCH(NJ)                                                                  \
  rope_kernel<T, DH, NJ><<<grid, block, 0, s>>>(q, io.ld_q, k, io.ld_k, qo, io.ld_qo, ko, io.ld_ko, \
                                                pos, n, n_heads, s_t, s_h, fr)
  if (nj <= 1) DIT_ROPE_LAUNCH(1);
  else if (nj <= 2) DIT_ROPE_LAUNCH(2);
  else if (nj <= 3) DIT_ROPE_LAUNCH(3);
  else if (nj <= 4) DIT_ROPE_LAUNCH(4);
  else DIT_ROPE_LAUNCH(5);   // wider rows are walked in chunks of 5 * kThreads vectors
#undef DIT_ROPE_LAUNCH
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const RopeIO& io, const int32_t* pos, int64_t n, int n_heads, int head_dim,
                    int s_t, int s_h, const double* freq, hipStream_t s) {
  Freqs fr;
  for (int p = 0; p < 64; ++p) fr.f[p] = p < head_dim / 2 ? freq[p] : 0.0;
  if (head_dim == 128) return launch_dh<T, 128>(io, pos, n, n_heads, s_t, s_h, fr, s);
  if (head_dim == 64) return launch_dh<T, 64>(io, pos, n, n_heads, s_t, s_h, fr, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rope(int bf16, const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                       void* q_out, int64_t ld_qo, void* k_out, int64_t ld_ko,
                       const int32_t* pos, int64_t n, int n_heads, int head_dim, int s_t,
                       int s_h, const double* freq_d, hipStream_t s) {
  const RopeIO io{q, ld_q, k, ld_k, q_out, ld_qo, k_out, ld_ko};
  return bf16 ? dispatch<uint16_t>(io, pos, n, n_heads, head_dim, s_t, s_h, freq_d, s)
              : dispatch<float>(io, pos, n, n_heads, head_dim, s_t, s_h, freq_d, s);
}

}  // namespace dit
