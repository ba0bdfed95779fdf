// chunk_cumsum: dt' = softplus(dt + dt_bias) and the inclusive in-chunk cumulative sum of
// dt' * A ("Agent 228: MAMBA-2 Reference Implementations Comparison", section 3.2: the
// discretised step and decay; the running sum of dt' A is the exponent of the decay between
// two positions of a chunk).  The sum is a wavefront prefix scan: each lane scans Q/64
// consecutive positions serially, then the 64 lane totals are combined with a log-step
// shuffle scan (the up-sweep idea of the parallel-scan section of "Agent 230:
// Comprehensive MAMBA-2 Implementation Comparison", on 64-wide wavefronts).
//
// One wavefront per (b, c, h); four heads per 256-thread workgroup, grid (ceil(H/4), nc, B).
// Every lane issues its Q/64 loads before any arithmetic, so one memory latency is exposed.
// dt' is optionally clamped to [lo, hi] (the dt limits of section 5.2 of the reference-
// comparison page).  Positions past the end of the sequence get dt' = 0, so the cumsum
// stays flat there.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename T>
__global__ __launch_bounds__(256) void chunk_cumsum_kernel(const T* __restrict__ dt,
                                                           const float* __restrict__ dt_bias,
                                                           const float* __restrict__ A,
                                                           float* __restrict__ dtp,
                                                           float* __restrict__ dAcs,
                                                           int L, int H, int nc, int Q, int clamp,
                                                           float lo, float hi) {
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int c = blockIdx.y, b = blockIdx.z;
  if (h >= H) return;
  const int t0 = c * Q;
  const int len = min(Q, L - t0);
  const int epl = Q >> 6;                      // positions per lane: 1, 2 or 4
  const int i0 = lane * epl;

  float raw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    raw[k] = 0.f;
    if (k < epl && i0 + k < len) raw[k] = to_f32(dt[((size_t)b * L + t0 + i0 + k) * H + h]);
  }
  const float bias = dt_bias[h];
  const float a = A[h];
  float d[4], cs[4];
  float run = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float v = softplus(raw[k] + bias);
    if (clamp) v = fminf(fmaxf(v, lo), hi);
    v = (k < epl && i0 + k < len) ? v : 0.f;
    d[k] = v;
    run += v * a;
    cs[k] = run;
  }
  // inclusive scan of the lane totals, then shift by one lane for the exclusive prefix
  float incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  float excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.f;
  const size_t base = (((size_t)b * H + h) * nc + c) * Q + i0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k < epl) {
      dtp[base + k] = d[k];
      dAcs[base + k] = cs[k] + excl;
    }
  }
}

hipError_t launch_chunk_cumsum(const FwdArgs& a, hipStream_t s) {
  dim3 grid((a.H + 3) / 4, a.nc, a.B);
  if (a.dtype == DT_F32) {
    chunk_cumsum_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(a.dt), a.dt_bias, a.A,
                                                    a.dtp, a.dAcs, a.L, a.H, a.nc, a.Q, a.clamp, a.dt_lo, a.dt_hi);
  } else {
    chunk_cumsum_kernel<__bf16><<<grid, 256, 0, s>>>(static_cast<const __bf16*>(a.dt), a.dt_bias, a.A,
                                                     a.dtp, a.dAcs, a.L, a.H, a.nc, a.Q, a.clamp, a.dt_lo, a.dt_hi);
  }
  return hipGetLastError();
}

}  // namespace ssd
