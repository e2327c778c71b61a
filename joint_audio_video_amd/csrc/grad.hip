// Elementwise and reduction kernels of the block's backward pass (bf16).
//
// The chain rule through the gated residual and the AdaLN modulation of the
// block ([H3-NFT] section "MiniMax H3 and Why Joint Audio-Video Generation
// Complicates RL Training": per-modality AdaLN; the gate row scales the
// branch) needs, besides the products:
//   * dz = gate[m] * dout, the gradient of the branch before its gate;
//   * sums over tokens, per modality or over all: the bias gradients (sum of
//     dz, of dqkv) and the table gradients (sum of dout * z for the gate
//     rows, of dy for the shift rows, of dy * xhat for the scale rows);
//   * transposes, so that the weight gradients (a sum over the tokens,
//     dW = dz^T o) run on the same A B^T GEMM with K = tokens.
// All HBM-bound.  Sums are deterministic: each workgroup reduces a fixed
// chunk of rows for 512 columns into a partial row, and a second pass adds
// the partials in chunk order.
#include "common.h"

namespace dit {
namespace {

__device__ __forceinline__ void unpack8(const uint4& r, float* f) {
  f[0] = bf16lo(r.x); f[1] = bf16hi(r.x); f[2] = bf16lo(r.y); f[3] = bf16hi(r.y);
  f[4] = bf16lo(r.z); f[5] = bf16hi(r.z); f[6] = bf16lo(r.w); f[7] = bf16hi(r.w);
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// dst [cols][ld_dst] = src [rows][cols]^T, with dst[c][r] = 0 for rows <= r < ld_dst.
// 64 x 64 tiles through LDS; cols and ld_dst are multiples of 64.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src,
                                                        int64_t ld_src, int64_t rows,
                                                        uint16_t* __restrict__ dst,
                                                        int64_t ld_dst) {
  __shared__ uint16_t t[64][72];
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
  {
    const int lr = tid >> 2, lc = (tid & 3) * 16;
    const int64_t r = r0 + lr;
    uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
    if (r < rows) {
      const uint4* p = reinterpret_cast<const uint4*>(src + r * ld_src + c0 + lc);
      a = p[0];
      b = p[1];
    }
    *reinterpret_cast<uint4*>(&t[lr][lc]) = a;
    *reinterpret_cast<uint4*>(&t[lr][lc + 8]) = b;
  }
  __syncthreads();
  const int orow = tid >> 2, ocol = (tid & 3) * 16;
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = (uint32_t)t[ocol + 2 * i][orow] | ((uint32_t)t[ocol + 2 * i + 1][orow] << 16);
  uint4* q = reinterpret_cast<uint4*>(dst + (c0 + orow) * ld_dst + r0 + ocol);
  q[0] = make_uint4(w[0], w[1], w[2], w[3]);
  q[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// out[i][j] = table[mod[i]][GATE][j] * g[i][j]
__global__ __launch_bounds__(256) void gate_scale_kernel(const uint16_t* __restrict__ g,
                                                         int64_t ld_g,
                                                         const uint8_t* __restrict__ mod,
                                                         const float* __restrict__ table,
                                                         uint16_t* __restrict__ out,
                                                         int64_t ld_out, int64_t n, int d) {
  const int vpr = d / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * vpr) return;
  const int64_t row = idx / vpr;
  const int c = (int)(idx - row * vpr) * 8;
  float f[8];
  unpack8(*reinterpret_cast<const uint4*>(g + row * ld_g + c), f);
  const float4* gt = reinterpret_cast<const float4*>(table + (size_t)(3 * mod[row] + 2) * d + c);
  const float4 g0 = gt[0], g1 = gt[1];
  f[0] *= g0.x; f[1] *= g0.y; f[2] *= g0.z; f[3] *= g0.w;
  f[4] *= g1.x; f[5] *= g1.y; f[6] *= g1.z; f[7] *= g1.w;
  *reinterpret_cast<uint4*>(out + row * ld_out + c) = pack8(f);
}

// io = gelu(a) (BWD false), or io = io * gelu'(a) (BWD true), elementwise over
// [n][f] bf16; gelu is the tanh form z sigma(2u), 2u = 2 sqrt(2/pi) (z +
// 0.044715 z^3), as the GEMM's GELU epilogue, and its derivative
// sigma(2u) + z sigma(2u) (1 - sigma(2u)) 2 sqrt(2/pi) (1 + 3 * 0.044715 z^2).
template <bool BWD>
__global__ __launch_bounds__(256) void gelu_kernel(const uint16_t* __restrict__ a, int64_t lda,
                                                   uint16_t* io, int64_t ld_io, int64_t n,
                                                   int f) {
  const int vpr = f / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * vpr) return;
  const int64_t row = idx / vpr;
  const int c = (int)(idx - row * vpr) * 8;
  float z[8], g[8];
  unpack8(*reinterpret_cast<const uint4*>(a + row * lda + c), z);
  uint4* out = reinterpret_cast<uint4*>(io + row * ld_io + c);
  if constexpr (BWD) unpack8(*out, g);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (BWD) {
      const float zz = z[e];
      const float s = __builtin_amdgcn_rcpf(
          1.0f + __expf(-1.5957691216057308f * fmaf(0.044715f * zz, zz * zz, zz)));
      const float dsu = 1.5957691216057308f * fmaf(0.134145f * zz, zz, 1.0f);
      g[e] *= fmaf(zz * s * (1.0f - s), dsu, s);
    } else {
      g[e] = gelu_tanh_fast(z[e]);
    }
  }
  *out = pack8(g);
}

constexpr int kColBlock = 512;   // columns per workgroup (8 per lane)

// Partial column sums over rows [chunk * rows_per_chunk, +rows_per_chunk):
// MODE 0 sums a, 1 sums a * b, 2 sums a * (b - mean) * rstd (stats per row).
// With mod, row i adds into group mod[i] (3 groups), else into group 0.
// partial: [chunks][groups][c].
template <int MODE>
__global__ __launch_bounds__(256) void colsum_kernel(const uint16_t* __restrict__ a, int64_t lda,
                                                     const uint16_t* __restrict__ b,
                                                     int64_t ldb,
                                                     const float2* __restrict__ stats,
                                                     const uint8_t* __restrict__ mod, int64_t n,
                                                     int c, int rows_per_chunk,
                                                     float* __restrict__ partial) {
  __shared__ float red[4][3][kColBlock];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int groups = mod ? 3 : 1;
  const int col = (int)blockIdx.x * kColBlock + lane * 8;
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r_end = min(n, r_begin + rows_per_chunk);
  float acc[3][8];
#pragma unroll
  for (int gi = 0; gi < 3; ++gi)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[gi][e] = 0.0f;
  if (col < c) {
    for (int64_t r = r_begin + wave; r < r_end; r += 4) {
      float v[8];
      unpack8(*reinterpret_cast<const uint4*>(a + r * lda + col), v);
      if constexpr (MODE >= 1) {
        float w[8];
        unpack8(*reinterpret_cast<const uint4*>(b + r * ldb + col), w);
        if constexpr (MODE == 2) {
          const float2 st = stats[r];
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = (w[e] - st.x) * st.y;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= w[e];
      }
      const int gi = mod ? mod[r] : 0;
      if (gi == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[0][e] += v[e];
      } else if (gi == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[1][e] += v[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[2][e] += v[e];
      }
    }
  }
#pragma unroll
  for (int gi = 0; gi < 3; ++gi)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][gi][lane * 8 + e] = acc[gi][e];
  __syncthreads();
  for (int i = tid; i < groups * kColBlock; i += 256) {
    const int gi = i / kColBlock, j = i % kColBlock;
    const int cc = (int)blockIdx.x * kColBlock + j;
    if (cc >= c) continue;
    const float s = red[0][gi][j] + red[1][gi][j] + red[2][gi][j] + red[3][gi][j];
    partial[((int64_t)blockIdx.y * groups + gi) * c + cc] = s;
  }
}

// out[g * out_gstride + j] = sum over chunks (in order) of partial[chunk][g][j]
__global__ __launch_bounds__(256) void colsum_finalize_kernel(const float* __restrict__ partial,
                                                              int chunks, int groups, int c,
                                                              float* __restrict__ out,
                                                              int64_t out_gstride) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)groups * c) return;
  const int gi = (int)(idx / c), j = (int)(idx - (int64_t)gi * c);
  float s = 0.0f;
  for (int ch = 0; ch < chunks; ++ch) s += partial[((int64_t)ch * groups + gi) * c + j];
  out[gi * out_gstride + j] = s;
}

}  // namespace

hipError_t launch_transpose(const void* src, int64_t ld_src, int64_t rows, int cols, void* dst,
                            int64_t ld_dst, hipStream_t s) {
  if (cols % 64 != 0 || ld_dst % 64 != 0 || ld_dst < rows || ld_src % 8 != 0)
    return hipErrorInvalidValue;
  if (rows == 0 && ld_dst == 0) return hipSuccess;
  const dim3 grid((unsigned)(cols / 64), (unsigned)(ld_dst / 64));
  transpose_kernel<<<grid, dim3(256), 0, s>>>(static_cast<const uint16_t*>(src), ld_src, rows,
                                              static_cast<uint16_t*>(dst), ld_dst);
  return hipGetLastError();
}

hipError_t launch_gate_scale(const void* g, int64_t ld_g, const uint8_t* mod, const float* table,
                             void* out, int64_t ld_out, int64_t n, int d, hipStream_t s) {
  if (d % 8 != 0) return hipErrorInvalidValue;
  const int64_t work = n * (d / 8);
  if (work == 0) return hipSuccess;
  gate_scale_kernel<<<dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s>>>(
      static_cast<const uint16_t*>(g), ld_g, mod, table, static_cast<uint16_t*>(out), ld_out, n,
      d);
  return hipGetLastError();
}

hipError_t launch_gelu(int backward, const void* a, int64_t lda, void* io, int64_t ld_io,
                       int64_t n, int f, hipStream_t s) {
  if (f % 8 != 0) return hipErrorInvalidValue;
  const int64_t work = n * (f / 8);
  if (work == 0) return hipSuccess;
  const dim3 grid((unsigned)((work + 255) / 256)), block(256);
  const uint16_t* ap = static_cast<const uint16_t*>(a);
  uint16_t* op = static_cast<uint16_t*>(io);
  if (backward)
    gelu_kernel<true><<<grid, block, 0, s>>>(ap, lda, op, ld_io, n, f);
  else
    gelu_kernel<false><<<grid, block, 0, s>>>(ap, lda, op, ld_io, n, f);
  return hipGetLastError();
}

size_t colsum_partial_bytes(int64_t n, int c, int groups) {
  const int64_t chunks = (n + kColsumRows - 1) / kColsumRows;
  return (size_t)(chunks > 0 ? chunks : 1) * (size_t)groups * (size_t)c * 4;
}

hipError_t launch_colsum(int mode, const void* a, int64_t lda, const void* b, int64_t ldb,
                         const float* stats, const uint8_t* mod, int64_t n, int c, float* partial,
                         float* out, int64_t out_gstride, hipStream_t s) {
  if (c % 8 != 0 || mode < 0 || mode > 2) return hipErrorInvalidValue;
  const int groups = mod ? 3 : 1;
  const int64_t chunks = (n + kColsumRows - 1) / kColsumRows;
  if (chunks > 65535) return hipErrorInvalidValue;
  if (chunks > 0) {
    const dim3 grid((unsigned)((c + kColBlock - 1) / kColBlock), (unsigned)chunks);
    const uint16_t* ap = static_cast<const uint16_t*>(a);
    const uint16_t* bp = static_cast<const uint16_t*>(b);
    const float2* st = reinterpret_cast<const float2*>(stats);
    if (mode == 0)
      colsum_kernel<0><<<grid, dim3(256), 0, s>>>(ap, lda, bp, ldb, st, mod, n, c, kColsumRows,
                                                  partial);
    else if (mode == 1)
      colsum_kernel<1><<<grid, dim3(256), 0, s>>>(ap, lda, bp, ldb, st, mod, n, c, kColsumRows,
                                                  partial);
    else
      colsum_kernel<2><<<grid, dim3(256), 0, s>>>(ap, lda, bp, ldb, st, mod, n, c, kColsumRows,
                                                  partial);
  }
  const int64_t outs = (int64_t)groups * c;
  colsum_finalize_kernel<<<dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, s>>>(
      partial, (int)chunks, groups, c, out, out_gstride);
  return hipGetLastError();
}

}  // namespace dit
