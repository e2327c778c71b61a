// One step of the joint audio-video denoising loop over the packed latent
// state, in one streaming pass.
//
// [vLLM-Omni] section "4. Joint Audio-Video Denoising Execution Flow": after
// the DiT forward the packed output is split by modality into video and audio
// velocities (stage 4), converted to a clean estimate X0 with the Rectified
// Flow parameterisation (stage 5), advanced by a deterministic Euler step,
// eta = 0, with each modality's own sigma (stage 6), and anchor rows are
// re-pinned to their original values (stage 7).  [VeRL-Omni] section 5.1: H3's
// velocity is the negative of the standard one (velocity_sign = -1).
//
// Per element, with v_std = sign * v and (s, s') the row's modality sigmas:
//   x0 = z - s v_std,   z' = z + (s' - s) v_std        (video / audio rows)
//   x0 = z' = anchor value                            (anchor rows)
//   untouched                                         (text rows)
// Both updates are single fmas in float32; when s' = 0 the host passes
// s' - s = -s exactly, so the last step's z' equals x0 bit for bit.
//
// HBM-bound: a thread owns 4 consecutive channels of one row (16-byte z, x0
// and anchor accesses, an 8- or 16-byte velocity load).  Threads walk the
// flattened (row, 4-channel group) index, so with contiguous rows a wave
// touches one contiguous span of each array.  z, v and x0 are streamed
// (non-temporal); the one-byte ids are shared by the row's threads.
#include "common.h"

namespace dit {
namespace {

constexpr int kThreads = 256;

struct StepCoef {
  float sigma[2];   // video, audio: current noise level
  float dsigma[2];  // next - current
  float sign;       // +1 standard velocity, -1 H3's own
};

template <bool kBf16>
__device__ __forceinline__ f32x4 load_v4(const void* v, int64_t off) {
  if constexpr (kBf16) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = __builtin_nontemporal_load(
        reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(v) + off));
    return f32x4{bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y)};
  } else {
    const uint4 w = ld_stream(static_cast<const float*>(v) + off);
    return f32x4{__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                 __uint_as_float(w.w)};
  }
}

__device__ __forceinline__ uint4 as_u4(const f32x4& a) {
  return make_uint4(__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                    __float_as_uint(a[3]));
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void denoise_kernel(
    float* __restrict__ z, int64_t ld_z, const void* __restrict__ v, int64_t ld_v,
    float* __restrict__ x0, int64_t ld_x0, const uint8_t* __restrict__ mod,
    const uint8_t* __restrict__ anchor, const float* __restrict__ av, int64_t ld_a,
    uint32_t total, uint32_t groups_per_row, StepCoef k) {
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t idx = blockIdx.x * kThreads + threadIdx.x; idx < total; idx += stride) {
    const uint32_t row = idx / groups_per_row;
    const uint32_t c = (idx - row * groups_per_row) * 4u;
    const int m = mod[row];
    if (m > 1) continue;   // text rows are conditioning, not latent state
    float* zp = z + (int64_t)row * ld_z + c;
    float* xp = x0 ? x0 + (int64_t)row * ld_x0 + c : nullptr;
    if (anchor && anchor[row]) {
      const uint4 a = *reinterpret_cast<const uint4*>(av + (int64_t)row * ld_a + c);
      st_stream(zp, a);
      if (xp) st_stream(xp, a);
      continue;
    }
    const uint4 zw = ld_stream(zp);
    const f32x4 zz = {__uint_as_float(zw.x), __uint_as_float(zw.y), __uint_as_float(zw.z),
                      __uint_as_float(zw.w)};
    const f32x4 vv = load_v4<kBf16>(v, (int64_t)row * ld_v + c);
    const float ns = -(m ? k.sigma[1] : k.sigma[0]), ds = m ? k.dsigma[1] : k.dsigma[0];
    f32x4 zn, xe;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float vs = k.sign * vv[e];
      xe[e] = fmaf(ns, vs, zz[e]);
      zn[e] = fmaf(ds, vs, zz[e]);
    }
    st_stream(zp, as_u4(zn));
    if (xp) st_stream(xp, as_u4(xe));
  }
}

}  // namespace

hipError_t launch_denoise(int bf16, float* z, int64_t ld_z, const void* v, int64_t ld_v,
                          float* x0, int64_t ld_x0, const uint8_t* mod, const uint8_t* anchor,
                          const float* anchor_vals, int64_t ld_a, int64_t n_rows, int channels,
                          const float sigmas[4], float sign, hipStream_t s) {
  const int64_t groups = channels / 4;
  const int64_t total = n_rows * groups;
  if (channels % 4 != 0 || total > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  StepCoef k;
  k.sigma[0] = sigmas[0];
  k.sigma[1] = sigmas[2];
  k.dsigma[0] = sigmas[1] - sigmas[0];
  k.dsigma[1] = sigmas[3] - sigmas[2];
  k.sign = sign;
  const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 1 << 20);
  if (bf16)
    denoise_kernel<true><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
        z, ld_z, v, ld_v, x0, ld_x0, mod, anchor, anchor_vals, ld_a, (uint32_t)total,
        (uint32_t)groups, k);
  else
    denoise_kernel<false><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
        z, ld_z, v, ld_v, x0, ld_x0, mod, anchor, anchor_vals, ld_a, (uint32_t)total,
        (uint32_t)groups, k);
  return hipGetLastError();
}

}  // namespace dit
