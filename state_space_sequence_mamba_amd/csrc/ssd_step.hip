// ssd_step: one recurrent decode step for every (b, h),
//     dt' = softplus(dt + dt_bias),  a = exp(dt' A),
//     state[p,n] <- a * state[p,n] + dt' x[p] B[n],   y[p] = sum_n state[p,n] C[n] + D[p] x[p]
// (the carried hidden state of stateful inference: "MAMBA2 Inference Optimization Report",
// Step 4; the discretisation of section 3.2 of "Agent 228: MAMBA-2 Reference Implementations
// Comparison", optionally clamped as in its section 5.2; D skip from Gap 4 of "Agent 228:
// MAMBA-2 Implementation Gaps"; optional output gate y * silu(z) of its section 3.1).
//
// Bandwidth bound: the fp32 state is read and written once; everything else is small.
// The state is streamed with non-temporal loads and stores: it is touched once per step and
// a large decode batch does not fit the last-level cache, so caching it only evicts others.
// One 256-thread workgroup per (b, h), or per half or quarter of its rows for small batches.
// A row of N floats is covered by N/4 consecutive lanes (one float4 each), so the state tile
// streams with fully coalesced 16-byte accesses and the reduction over n is a butterfly of
// N/4 lanes inside a wavefront.  All state loads of a thread are issued before any use.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename T, int P, int N>
__global__ __launch_bounds__(256) void ssd_step_kernel(float* __restrict__ state,
                                                       const T* __restrict__ x,
                                                       const T* __restrict__ dt,
                                                       const float* __restrict__ dt_bias,
                                                       const float* __restrict__ A,
                                                       const T* __restrict__ Bm,
                                                       const T* __restrict__ Cm,
                                                       const float* __restrict__ Dw,
                                                       const T* __restrict__ Z,
                                                       T* __restrict__ y, int H, int G, int clamp,
                                                       float lo, float hi, int split) {
  constexpr int TPR = N / 4;           // lanes per state row
  constexpr int RPP = 256 / TPR;       // rows per pass
  constexpr int NPASS = (P + RPP - 1) / RPP;
  const int bh = blockIdx.x / split;
  const int prows = P / split, pbase = (blockIdx.x % split) * prows;   // this workgroup's rows
  const int h = bh % H, b = bh / H;
  const int g = h / (H / G);
  const int tid = threadIdx.x;
  const int col = (tid % TPR) * 4;
  const int row0 = tid / TPR;

  float d = softplus(to_f32(dt[bh]) + dt_bias[h]);
  if (clamp) d = fminf(fmaxf(d, lo), hi);
  const float a = expf(d * A[h]);
  float bv[4], cv[4];
  const T* Bp = Bm + ((size_t)b * G + g) * N + col;
  const T* Cp = Cm + ((size_t)b * G + g) * N + col;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bv[e] = to_f32(Bp[e]);
    cv[e] = to_f32(Cp[e]);
  }

  float* st = state + (size_t)bh * P * N;
  f32x4 s[NPASS];
  float xv[NPASS];
  // every load is issued (rows past the workgroup's share read its first row again) before
  // any use
#pragma unroll
  for (int u = 0; u < NPASS; ++u) {
    const int pl = row0 + u * RPP;
    const int p = pbase + (pl < prows ? pl : 0);
    s[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(st + (size_t)p * N + col));
    xv[u] = to_f32(x[(size_t)bh * P + p]);
  }
#pragma unroll
  for (int u = 0; u < NPASS; ++u) {
    const int pl = row0 + u * RPP;
    const int p = pbase + pl;
    if (pl < prows) {
      const float dx = d * xv[u];
      f32x4 v = s[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = a * v[e] + dx * bv[e];
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(st + (size_t)p * N + col));
      float part = v[0] * cv[0] + v[1] * cv[1] + v[2] * cv[2] + v[3] * cv[3];
#pragma unroll
      for (int off = TPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
      if ((tid % TPR) == 0) {
        const float dw = Dw ? Dw[(size_t)h * P + p] : 0.f;
        float out = part + dw * xv[u];
        if (Z) {
          const float zv = to_f32(Z[(size_t)bh * P + p]);
          out *= silu(zv);  // output gate
        }
        y[(size_t)bh * P + p] = from_f32<T>(out);
      }
    }
  }
}

template <typename T, int P, int N>
static hipError_t launch_step_impl(const StepArgs& a, hipStream_t s) {
  // small batches: the rows of a (b, h) state over up to 4 workgroups (whole passes of
  // 256 / (N / 4) rows each), so that the launch still spreads over the chip
  constexpr int RPP = 256 / (N / 4);
  int split = 1;
  while (split < 4 && (long)a.B * a.H * split < 1024 && P % (2 * split) == 0 && (P / (2 * split)) % RPP == 0)
    split *= 2;
  const unsigned nblocks = (unsigned)a.B * a.H * split;
  hipExtLaunchKernelGGL(ssd_step_kernel<T, P, N>, dim3(nblocks), dim3(256), 0, s, a.ev0, a.ev1, 0,
      a.state, static_cast<const T*>(a.x), static_cast<const T*>(a.dt), a.dt_bias, a.A,
      static_cast<const T*>(a.Bm), static_cast<const T*>(a.Cm), a.D, static_cast<const T*>(a.z),
      static_cast<T*>(a.y), a.H, a.G, a.clamp, a.dt_lo, a.dt_hi, split);
  return hipGetLastError();
}

hipError_t launch_ssd_step(const StepArgs& a, hipStream_t s) {
#define SSD_CASE(T, P_, N_) \
  if (a.dtype == SSD_DTYPE_CODE_##T && a.P == P_ && a.N == N_) return launch_step_impl<T, P_, N_>(a, s);
  SSD_FOR_EACH_SHAPE(SSD_CASE)
#undef SSD_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
