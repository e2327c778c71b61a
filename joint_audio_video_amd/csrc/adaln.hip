// Per-modality adaptive LayerNorm: y = LN(x) * (1 + scale[m]) + shift[m].
//
// [H3-NFT] section "MiniMax H3 and Why Joint Audio-Video Generation Complicates
// RL Training": AdaLN branches are per modality and their modulation outputs
// can be cached, so the kernel reads a precomputed float32 table
// [3 modalities][shift, scale, gate][d_model]; the modality id of each token
// picks its rows.
//
// HBM-bound (about 2*d_model*elt bytes per token).  One wave per token row:
// the row is read once with 16-byte streaming loads into registers, mean and
// variance are two exact passes over the registers (wave reductions), and the
// modulated row is written with 16-byte streaming stores, so the x and y
// streams do not evict the table rows, which come from L2.
#include "common.h"

namespace dit {
namespace {

// Waves per workgroup: measured best of 1, 2, 4, 8 (2 rows per wave at d_model
// 5120: 205.5 us = 73.2% of 8 TB/s against 208.8 us for 4 waves).
constexpr int kWaves = 2;

template <typename T> struct Vec;
template <> struct Vec<uint16_t> { static constexpr int N = 8; };   // bf16 bits
template <> struct Vec<float> { static constexpr int N = 4; };

__device__ __forceinline__ void unpack(const uint4& r, float* f, uint16_t) {
  f[0] = bf16lo(r.x); f[1] = bf16hi(r.x); f[2] = bf16lo(r.y); f[3] = bf16hi(r.y);
  f[4] = bf16lo(r.z); f[5] = bf16hi(r.z); f[6] = bf16lo(r.w); f[7] = bf16hi(r.w);
}
__device__ __forceinline__ void unpack(const uint4& r, float* f, float) {
  f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
  f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
}
__device__ __forceinline__ uint4 pack(const float* f, uint16_t) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                    pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}
__device__ __forceinline__ uint4 pack(const float* f, float) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                    __float_as_uint(f[2]), __float_as_uint(f[3]));
}

// NV = 16-byte vectors per lane (row of nvec <= 64*NV vectors); each wave
// normalises R consecutive rows.  All R rows are loaded before any
// reduction, and when the R rows share one modality (the common case in a
// pack, whose modalities come in long runs) each table vector is loaded once
// for all of them, dividing the table's L2 traffic by R.
// Q8: instead of y, write its per-row e4m3 codes (q, row stride ld_y bytes)
// and float32 scales (qs), scale = amax(|y|) / 448 of the float32 y.
template <typename T, int NV, int R, bool Q8 = false>
__global__ __launch_bounds__(64 * kWaves) void adaln_kernel(
    const T* __restrict__ x, int64_t ld_x, const uint8_t* __restrict__ mod,
    const float* __restrict__ table, T* __restrict__ y, int64_t ld_y, int64_t n, int d,
    float eps, uint8_t* __restrict__ q = nullptr, float* __restrict__ qs = nullptr) {
  constexpr int E = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * R;
  if (row0 >= n) return;
  const int nvec = d / E;

  uint4 raw[R][NV];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint4* xr = reinterpret_cast<const uint4*>(x + (row0 + r) * ld_x);
    const bool live = row0 + r < n;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + 64 * i;
      raw[r][i] = live && c < nvec ? ld_stream(xr + c) : make_uint4(0, 0, 0, 0);
    }
  }
  const float inv_d = 1.0f / (float)d;
  float mean[R], rstd[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float f[E];
      unpack(raw[r][i], f, T());
#pragma unroll
      for (int e = 0; e < E; ++e) s += f[e];
    }
    mean[r] = wave_sum(s) * inv_d;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (lane + 64 * i < nvec) {
        float f[E];
        unpack(raw[r][i], f, T());
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float t = f[e] - mean[r];
          ss = fmaf(t, t, ss);
        }
      }
    }
    rstd[r] = 1.0f / sqrtf(wave_sum(ss) * inv_d + eps);
  }

  int m[R];
  bool same = true;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = row0 + r < n ? mod[row0 + r] : mod[row0];
    same = same && m[r] == m[0];
  }
  // Modulated values of row r's vector i given the table vectors of its modality.
  auto modulate = [&](int r, int i, const float* shv, const float* scv, float* o) {
    float f[E];
    unpack(raw[r][i], f, T());
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = fmaf((f[e] - mean[r]) * rstd[r], 1.0f + scv[e], shv[e]);
  };
  auto load_table = [&](int mm, int c, float* shv, float* scv) {
    const float4* shift = reinterpret_cast<const float4*>(table + (size_t)(3 * mm + 0) * d);
    const float4* scale = reinterpret_cast<const float4*>(table + (size_t)(3 * mm + 1) * d);
#pragma unroll
    for (int e4 = 0; e4 < E / 4; ++e4) {
      const float4 sh = shift[c * (E / 4) + e4];
      const float4 sc = scale[c * (E / 4) + e4];
      shv[4 * e4 + 0] = sh.x; shv[4 * e4 + 1] = sh.y; shv[4 * e4 + 2] = sh.z; shv[4 * e4 + 3] = sh.w;
      scv[4 * e4 + 0] = sc.x; scv[4 * e4 + 1] = sc.y; scv[4 * e4 + 2] = sc.z; scv[4 * e4 + 3] = sc.w;
    }
  };
  if constexpr (!Q8) {
    // Writes row r's vector i given the table vectors of its modality.
    auto emit = [&](int r, int i, const float* shv, const float* scv) {
      float o[E];
      modulate(r, i, shv, scv, o);
      st_stream(reinterpret_cast<uint4*>(y + (row0 + r) * ld_y) + lane + 64 * i, pack(o, T()));
    };
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + 64 * i;
      if (c >= nvec) continue;
      float shv[E], scv[E];
      if (same) {
        load_table(m[0], c, shv, scv);
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (row0 + r < n) emit(r, i, shv, scv);
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (row0 + r >= n) continue;
          load_table(m[r], c, shv, scv);
          emit(r, i, shv, scv);
        }
      }
    }
  } else {
    // FP8 output (one row per wave): the modulated row stays in registers
    // while the wave reduces its amax, then leaves as codes of y * (1 / scale).
    static_assert(!Q8 || R == 1, "the FP8 output takes one row per wave");
    float yv[NV][E];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + 64 * i;
#pragma unroll
      for (int e = 0; e < E; ++e) yv[i][e] = 0.0f;
      if (c >= nvec) continue;
      float shv[E], scv[E];
      load_table(m[0], c, shv, scv);
      modulate(0, i, shv, scv, yv[i]);
#pragma unroll
      for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(yv[i][e]));
    }
    const float a = wave_max(amax);
    const float sc = a > 0.0f ? a / 448.0f : 1.0f;
    const float inv = 1.0f / sc;
    if (lane == 0) qs[row0] = sc;
    uint8_t* qrow = q + row0 * ld_y;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + 64 * i;
      if (c >= nvec) continue;
      uint32_t w[E / 4];
#pragma unroll
      for (int j = 0; j < E / 4; ++j)
        w[j] = e4m3_pack4(yv[i][4 * j] * inv, yv[i][4 * j + 1] * inv, yv[i][4 * j + 2] * inv,
                          yv[i][4 * j + 3] * inv);
      if constexpr (E == 8)
        *reinterpret_cast<uint2*>(qrow + c * E) = make_uint2(w[0], w[1]);
      else
        *reinterpret_cast<uint32_t*>(qrow + c * E) = w[0];
    }
  }
}

template <typename T, bool Q8>
hipError_t dispatch(const void* x, int64_t ld_x, const uint8_t* mod, const float* table, void* y,
                    int64_t ld_y, int64_t n, int d, float eps, uint8_t* q, float* qs,
                    hipStream_t s) {
  const int nvec = d / Vec<T>::N;
  const int need = (nvec + 63) / 64;
  const T* xp = static_cast<const T*>(x);
  T* yp = static_cast<T*>(y);
  // Rows per wave: enough to share table loads, few enough to keep the raw
  // rows (R * NV * 4 registers) in registers.
  // The FP8 output keeps the modulated row in registers between its two
  // passes: one row per wave keeps the register count (and occupancy) of the
  // bf16 output's two rows.
#define DIT_ADALN_CASE(NVV, RR)                                                                 \
  if (need <= NVV) {                                                                            \
    constexpr int RQ = Q8 ? 1 : RR;                                                             \
    const dim3 grid((unsigned)((n + kWaves * RQ - 1) / (kWaves * RQ))), block(64 * kWaves);     \
    adaln_kernel<T, NVV, RQ, Q8><<<grid, block, 0, s>>>(xp, ld_x, mod, table, yp, ld_y, n, d,   \
                                                        eps, q, qs);                            \
    return hipGetLastError();                                                                   \
  }
  DIT_ADALN_CASE(1, 2) DIT_ADALN_CASE(2, 2) DIT_ADALN_CASE(3, 2) DIT_ADALN_CASE(4, 2)
  DIT_ADALN_CASE(5, 2) DIT_ADALN_CASE(6, 2) DIT_ADALN_CASE(8, 2) DIT_ADALN_CASE(10, 2)
  DIT_ADALN_CASE(12, 1)
  DIT_ADALN_CASE(16, 1) DIT_ADALN_CASE(20, 1) DIT_ADALN_CASE(24, 1) DIT_ADALN_CASE(32, 1)
#undef DIT_ADALN_CASE
  return hipErrorInvalidValue;
}

// Backward of y = xhat (1 + scale[m]) + shift[m] for one row per wave
// (bf16): with dxh = dy (1 + scale[m]), dx = dres + rstd (dxh - mean(dxh) -
// xhat mean(dxh xhat)); the row's mean and rstd go to stats for the table
// gradients.  x and dy stay in registers between the two passes.
template <int NV>
__global__ __launch_bounds__(64 * kWaves) void adaln_bwd_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, const uint16_t* __restrict__ dy, int64_t ld_dy,
    const uint16_t* dres, int64_t ld_dres, const uint8_t* __restrict__ mod,
    const float* __restrict__ table, uint16_t* dx, int64_t ld_dx, float2* __restrict__ stats,
    int64_t n, int d, float eps) {
  constexpr int E = 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= n) return;
  const int nvec = d / E;
  uint4 xr[NV], gr[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    xr[i] = c < nvec ? ld_stream(reinterpret_cast<const uint4*>(x + row * ld_x) + c)
                     : make_uint4(0, 0, 0, 0);
    gr[i] = c < nvec ? ld_stream(reinterpret_cast<const uint4*>(dy + row * ld_dy) + c)
                     : make_uint4(0, 0, 0, 0);
  }
  const float inv_d = 1.0f / (float)d;
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float f[E];
    unpack(xr[i], f, uint16_t());
#pragma unroll
    for (int e = 0; e < E; ++e) s += f[e];
  }
  const float mean = wave_sum(s) * inv_d;
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (lane + 64 * i < nvec) {
      float f[E];
      unpack(xr[i], f, uint16_t());
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float t = f[e] - mean;
        ss = fmaf(t, t, ss);
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(ss) * inv_d + eps);
  const float* scale = table + (size_t)(3 * mod[row] + 1) * d;
  // dxh and xhat of vector i
  auto terms = [&](int i, float* xh, float* g) {
    float f[E];
    unpack(xr[i], f, uint16_t());
    unpack(gr[i], g, uint16_t());
    const float4* sc = reinterpret_cast<const float4*>(scale) + 2 * (lane + 64 * i);
    const float4 s0 = sc[0], s1 = sc[1];
    const float sv[E] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int e = 0; e < E; ++e) {
      xh[e] = (f[e] - mean) * rstd;
      g[e] *= 1.0f + sv[e];
    }
  };
  float a1 = 0.0f, a2 = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (lane + 64 * i >= nvec) continue;
    float xh[E], g[E];
    terms(i, xh, g);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      a1 += g[e];
      a2 = fmaf(g[e], xh[e], a2);
    }
  }
  const float m1 = wave_sum(a1) * inv_d, m2 = wave_sum(a2) * inv_d;
  if (lane == 0) stats[row] = make_float2(mean, rstd);
  // Up to 10 vectors per lane (d_model 5,120) the row's dres vectors are all
  // loaded before the first dx store: dx may be dres, so a load placed after
  // a store waits for it and the row's latency is paid once per vector.
  // (Past the row end the last vector is loaded instead; it is not stored.)
  // Wider rows keep the loads in the loop: held, they would leave one wave
  // per SIMD.
  constexpr bool kAhead = NV <= 10;
  uint4 rr[kAhead ? NV : 1];
  if constexpr (kAhead) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      rr[i] = *(reinterpret_cast<const uint4*>(dres + row * ld_dres) + min(lane + 64 * i, nvec - 1));
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c >= nvec) continue;
    float xh[E], g[E], r[E];
    terms(i, xh, g);
    if constexpr (kAhead)
      unpack(rr[i], r, uint16_t());
    else
      unpack(*(reinterpret_cast<const uint4*>(dres + row * ld_dres) + c), r, uint16_t());
#pragma unroll
    for (int e = 0; e < E; ++e) r[e] += rstd * (g[e] - m1 - xh[e] * m2);
    *(reinterpret_cast<uint4*>(dx + row * ld_dx) + c) = pack(r, uint16_t());
  }
}

}  // namespace

hipError_t launch_adaln(int bf16, const void* x, int64_t ld_x, const uint8_t* mod,
                        const float* table, void* y, int64_t ld_y, int64_t n, int d, float eps,
                        hipStream_t s) {
  return bf16 ? dispatch<uint16_t, false>(x, ld_x, mod, table, y, ld_y, n, d, eps, nullptr,
                                         nullptr, s)
              : dispatch<float, false>(x, ld_x, mod, table, y, ld_y, n, d, eps, nullptr, nullptr,
                                       s);
}

hipError_t launch_adaln_fp8(int bf16, const void* x, int64_t ld_x, const uint8_t* mod,
                            const float* table, uint8_t* q, int64_t ld_q, float* scales,
                            int64_t n, int d, float eps, hipStream_t s) {
  return bf16 ? dispatch<uint16_t, true>(x, ld_x, mod, table, nullptr, ld_q, n, d, eps, q, scales,
                                         s)
              : dispatch<float, true>(x, ld_x, mod, table, nullptr, ld_q, n, d, eps, q, scales, s);
}

}  // namespace dit

namespace dit {

hipError_t launch_adaln_bwd(const void* x, int64_t ld_x, const void* dy, int64_t ld_dy,
                            const void* dres, int64_t ld_dres, const uint8_t* mod,
                            const float* table, void* dx, int64_t ld_dx, float* stats, int64_t n,
                            int d, float eps, hipStream_t s) {
  if (d % 8 != 0 || d > 16384) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  const int need = (d / 8 + 63) / 64;
  const dim3 grid((unsigned)((n + kWaves - 1) / kWaves)), block(64 * kWaves);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* gp = static_cast<const uint16_t*>(dy);
  const uint16_t* rp = static_cast<const uint16_t*>(dres);
  uint16_t* op = static_cast<uint16_t*>(dx);
  float2* st = reinterpret_cast<float2*>(stats);
#define DIT_ADALN_BWD_CASE(NVV)                                                                 \
  if (need <= NVV) {                                                                            \
    adaln_bwd_kernel<NVV><<<grid, block, 0, s>>>(xp, ld_x, gp, ld_dy, rp, ld_dres, mod, table,  \
                                                 op, ld_dx, st, n, d, eps);                     \
    return hipGetLastError();                                                                   \
  }
  DIT_ADALN_BWD_CASE(1) DIT_ADALN_BWD_CASE(2) DIT_ADALN_BWD_CASE(4) DIT_ADALN_BWD_CASE(6)
  DIT_ADALN_BWD_CASE(8) DIT_ADALN_BWD_CASE(10) DIT_ADALN_BWD_CASE(12) DIT_ADALN_BWD_CASE(16)
  DIT_ADALN_BWD_CASE(24) DIT_ADALN_BWD_CASE(32)
#undef DIT_ADALN_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace dit
