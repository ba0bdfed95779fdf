// peak_probe: measurement-only kernels (libssd_peak.so, not part of the SSD library) that give
// the chip's attainable matrix-core rates for the two MFMA shapes the SSD kernels use, so the
// published peaks the rooflines quote can be set beside measured ones.
//
// Each lane runs CH independent accumulator chains of the same MFMA with operands held in
// registers: no memory traffic inside the loop, enough independent chains per wavefront to
// keep the matrix pipe issuing back to back, and one 256-thread workgroup per SIMD quad.
#include <hip/hip_runtime.h>

#include "ssd_common.h"
#include "ssd_peak.h"

namespace {

constexpr int kChains = 4;

__global__ __launch_bounds__(256) void mfma_f32_loop(float* __restrict__ out, int iters) {
  f32x4 acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) acc[k] = ssd::zero4();
  const float a = 1e-3f * (float)(threadIdx.x & 63), b = 1e-3f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) acc[k] = ssd::mfma_16x16x4_f32(a, b, acc[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_bf16_loop(float* __restrict__ out, int iters) {
  f32x4 acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) acc[k] = ssd::zero4();
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1e-3f * (float)(threadIdx.x & 63));
    b[e] = static_cast<__bf16>(1e-3f);
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) acc[k] = ssd::mfma_16x16x32_bf16(a, b, acc[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int ssd_peak_mfma_launch(int kind, int blocks, int iters, float* out, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || !out) return 1;
  if (kind == 0)
    mfma_f32_loop<<<blocks, 256, 0, stream>>>(out, iters);
  else if (kind == 1)
    mfma_bf16_loop<<<blocks, 256, 0, stream>>>(out, iters);
  else
    return 1;
  return (int)hipGetLastError();
}

double ssd_peak_mfma_flops(int kind, int blocks, int iters) {
  const double per = kind == 0 ? 2048.0 : 16384.0;
  return per * kChains * (double)iters * 4.0 * (double)blocks;
}

}  // extern "C"
