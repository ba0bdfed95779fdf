// Gated RMSNorm of the scan output: g = y * silu(z) (g = y without a gate), normalised by its
// root mean square over each token's channels in groups of norm_heads heads and scaled per
// channel, out = g / sqrt(mean(g^2) + eps) * weight ("Agent 228: MAMBA-2 Reference
// Implementations Comparison", section 7.3: item 9, the output gate; item 11, the RMSNorm in
// front of the final projection).
//
// The norm couples all the channels of a group of heads of one token, while the scan's
// workgroups own slices of heads (and write a head's y before the next head is computed), so it
// runs as its own pass: one wavefront per (token, group) reads the group's y and z once (kept in
// registers for groups up to 5120 channels; larger groups sweep them a second time from cache)
// and writes out once -- an HBM-bound pass of 3 tensors (2 without a gate).  16-byte vectors of 8 channels per
// lane; the sum of squares in fp32 in a fixed order (deterministic).
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kNThreads = 512;                   // eight wavefronts, one (token, group) each

template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  static __device__ __forceinline__ void load(const __bf16* p, float (&v)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __builtin_bit_cast(float, w[k] << 16);
      v[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(__bf16* p, const float (&v)[8]) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{v[2 * k], v[2 * k + 1]}), b2));
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// g = y * silu(z) of 8 consecutive channels
template <typename T>
__device__ __forceinline__ void gated(const T* y, const T* z, size_t o, float (&g)[8]) {
  Vec8<T>::load(y + o, g);
  if (z) {
    float zv[8];
    Vec8<T>::load(z + o, zv);
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] *= silu(zv[k]);
  }
}

}  // namespace

// Groups of up to kRegChunks * 512 channels keep g in registers between the sum of squares and
// the output (one read of y and z); a workgroup then takes one group of kTokens * 8 consecutive
// tokens (kTokens per wavefront) with the group's weights staged once in LDS, instead of every
// wavefront reading them for its token.  Larger groups take one (token, group) per wavefront and
// read y and z twice (the second time from cache).
constexpr int kRegChunks = 10;
constexpr int kTokens = 1;

// (64-bit arithmetic: tokens * gpt may come within a few units of 2^32)
__host__ __device__ inline uint32_t norm_workgroups(uint32_t tokens, int gl, int gpt) {
  constexpr uint64_t per = kTokens * (kNThreads / 64);
  return (uint32_t)(gl <= kRegChunks * 512 ? ((uint64_t)tokens + per - 1) / per * (uint64_t)gpt
                                           : ((uint64_t)tokens * gpt + kNThreads / 64 - 1) / (kNThreads / 64));
}

template <typename T>
__global__ __launch_bounds__(kNThreads) void gated_rmsnorm_kernel(const T* __restrict__ y, const T* __restrict__ z,
                                                                 const float* __restrict__ weight, T* out,
                                                                 uint32_t tokens, int gl, int gpt, float eps) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (gl <= kRegChunks * 512) {
    __shared__ __attribute__((aligned(16))) float s_w[kRegChunks * 512];
    const uint32_t grp = blockIdx.x % gpt, tb = blockIdx.x / gpt;
    const float* wg = weight + (size_t)grp * gl;
    for (int i = 4 * threadIdx.x; i < gl; i += 4 * kNThreads)
      *reinterpret_cast<float4*>(&s_w[i]) = *reinterpret_cast<const float4*>(wg + i);
    __syncthreads();
    const uint32_t t0 = (tb * (kNThreads / 64) + wave) * kTokens, t1 = min(t0 + kTokens, tokens);
    for (uint32_t tok = t0; tok < t1; ++tok) {
      const size_t base = ((size_t)tok * gpt + grp) * gl;
      float g[kRegChunks][8];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < kRegChunks; ++c) {
        const int i = c * 512 + 8 * lane;
        if (i < gl) {
          gated(y, z, base + i, g[c]);
#pragma unroll
          for (int k = 0; k < 8; ++k) ss += g[c][k] * g[c][k];
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
      const float scale = 1.0f / sqrtf(ss / (float)gl + eps);
#pragma unroll
      for (int c = 0; c < kRegChunks; ++c) {
        const int i = c * 512 + 8 * lane;
        if (i < gl) {
          const float4 w0 = *reinterpret_cast<const float4*>(&s_w[i]), w1 = *reinterpret_cast<const float4*>(&s_w[i + 4]);
          const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
          for (int k = 0; k < 8; ++k) g[c][k] = g[c][k] * scale * wv[k];
          Vec8<T>::store(out + base + i, g[c]);
        }
      }
    }
    return;
  }
  const uint32_t unit = blockIdx.x * (kNThreads / 64) + wave;                 // (token, group)
  if (unit >= tokens * (uint32_t)gpt) return;                                // (whole wavefronts)
  const uint32_t tok = unit / gpt, grp = unit % gpt;
  const size_t base = ((size_t)tok * gpt + grp) * gl;
  const float* wg = weight + (size_t)grp * gl;
  float ss = 0.f;
  for (int i = 8 * lane; i < gl; i += 8 * 64) {
    float g[8];
    gated(y, z, base + i, g);
#pragma unroll
    for (int k = 0; k < 8; ++k) ss += g[k] * g[k];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float scale = 1.0f / sqrtf(ss / (float)gl + eps);
  for (int i = 8 * lane; i < gl; i += 8 * 64) {
    float g[8];
    gated(y, z, base + i, g);                     // (out may be y itself: each lane reads before it writes)
    const float4 w0 = *reinterpret_cast<const float4*>(wg + i), w1 = *reinterpret_cast<const float4*>(wg + i + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] = g[k] * scale * wv[k];
    Vec8<T>::store(out + base + i, g);
  }
}

hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t s) {
  const int gl = a.norm_heads * a.P, gpt = a.H / a.norm_heads;
  const uint32_t nwg = norm_workgroups((uint32_t)a.tokens, gl, gpt);
  if (nwg == 0) return hipSuccess;
  const dim3 grid(nwg);
  if (a.dtype == DT_BF16)
    hipExtLaunchKernelGGL(gated_rmsnorm_kernel<__bf16>, grid, dim3(kNThreads), 0, s, a.ev0, a.ev1, 0,
                          static_cast<const __bf16*>(a.y), static_cast<const __bf16*>(a.z), a.weight,
                          static_cast<__bf16*>(a.out), (uint32_t)a.tokens, gl, gpt, a.eps);
  else
    hipExtLaunchKernelGGL(gated_rmsnorm_kernel<float>, grid, dim3(kNThreads), 0, s, a.ev0, a.ev1, 0,
                          static_cast<const float*>(a.y), static_cast<const float*>(a.z), a.weight,
                          static_cast<float*>(a.out), (uint32_t)a.tokens, gl, gpt, a.eps);
  return hipGetLastError();
}

}  // namespace ssd
