// chunk_cumsum: dt' = softplus(dt + dt_bias) and the inclusive in-chunk cumulative sum of
// dt' * A ("Agent 228: MAMBA-2 Reference Implementations Comparison", section 3.2: the
// discretised step and decay; the running sum of dt' A is the exponent of the decay between
// two positions of a chunk).  The sum is a wavefront prefix scan: each lane scans Q/64
// consecutive positions serially, then the 64 lane totals are combined with a log-step
// shuffle scan (the up-sweep idea of the parallel-scan section of "Agent 230:
// Comprehensive MAMBA-2 Implementation Comparison", on 64-wide wavefronts).
//
// Grid (ceil(H/16), nc, B), 256 threads.  One workgroup reads the Q x 16 (token, head)
// tile of dt with row-contiguous loads, then each wavefront scans four heads.
// Positions past the end of the sequence get dt' = 0, so the cumsum stays flat there.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kCumsumHeads = 16;

template <typename T>
__global__ __launch_bounds__(256) void chunk_cumsum_kernel(const T* __restrict__ dt,
                                                           const float* __restrict__ dt_bias,
                                                           const float* __restrict__ A,
                                                           float* __restrict__ dtp,
                                                           float* __restrict__ dAcs,
                                                           int L, int H, int nc, int Q) {
  __shared__ float s_dt[256][kCumsumHeads + 1];
  const int b = blockIdx.z, c = blockIdx.y, h0 = blockIdx.x * kCumsumHeads;
  const int nh = min(kCumsumHeads, H - h0);
  const int t0 = c * Q;
  const int len = min(Q, L - t0);
  const int tid = threadIdx.x;

  for (int idx = tid; idx < Q * kCumsumHeads; idx += 256) {
    const int i = idx / kCumsumHeads, hh = idx % kCumsumHeads;
    float v = 0.f;
    if (i < len && hh < nh) v = to_f32(dt[((size_t)b * L + t0 + i) * H + h0 + hh]);
    s_dt[i][hh] = v;
  }
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int epl = Q >> 6;  // positions per lane: 1, 2 or 4
  for (int hh = wave; hh < nh; hh += 4) {
    const int h = h0 + hh;
    const float bias = dt_bias[h];
    const float a = A[h];
    float d[4], cs[4];
    float run = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < epl) {
        const int i = lane * epl + k;
        const float v = (i < len) ? softplus(s_dt[i][hh] + bias) : 0.f;
        d[k] = v;
        run += v * a;
        cs[k] = run;
      }
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
    const size_t base = (((size_t)b * H + h) * nc + c) * Q + (size_t)lane * epl;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < epl) {
        dtp[base + k] = d[k];
        dAcs[base + k] = cs[k] + excl;
      }
    }
  }
}

hipError_t launch_chunk_cumsum(const FwdArgs& a, hipStream_t s) {
  dim3 grid((a.H + kCumsumHeads - 1) / kCumsumHeads, a.nc, a.B);
  if (a.dtype == DT_F32) {
    chunk_cumsum_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(a.dt), a.dt_bias, a.A,
                                                    a.dtp, a.dAcs, a.L, a.H, a.nc, a.Q);
  } else {
    chunk_cumsum_kernel<__bf16><<<grid, 256, 0, s>>>(static_cast<const __bf16*>(a.dt), a.dt_bias, a.A,
                                                     a.dtp, a.dAcs, a.L, a.H, a.nc, a.Q);
  }
  return hipGetLastError();
}

}  // namespace ssd
