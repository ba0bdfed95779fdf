// state_passing: the inter-chunk recurrence on the chunk states,
//     H_0 = initial_state (or 0),   H_{c+1} = exp(dAcs[c, last]) * H_c + S_c,
// writing H_c (the state entering chunk c) over S_c in place and H_nc to final_state.  For
// bf16 inputs H_c goes instead (or, for the backward, also) to a bf16 copy, which is all the
// scan reads: it halves the largest stream of the bf16 forward (P N values per chunk and head).
// This is the carry step of the chunked scan ("Agent 228: MAMBA-2 Implementation Gaps",
// Gap 1: the last state of each chunk is carried into the next; the scan-of-block-carries
// phase of the block-parallel scan in "Agent 230: Comprehensive MAMBA-2 Implementation
// Comparison", section 2).
//
// The backward pass runs the same recurrence from the last chunk to the first (reverse != 0)
// on the per-chunk output gradients: G_c = exp(dAcs[c, last]) * G_{c+1} + dS_c, leaving in
// slot c the gradient of the state leaving chunk c and in final_state that of the initial
// state.
//
// Sequential over chunks, parallel over (b, h, p, n): each thread owns 4 consecutive state
// elements (one 16-byte load and store per chunk, fully coalesced: a (b, c, h) state block
// is P*N contiguous floats) and keeps its carry in registers.  Loads of up to 8 chunks are
// issued before the dependent multiply-adds, since they do not depend on the carry.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

__global__ __launch_bounds__(256) void state_passing_kernel(float* __restrict__ states,
                                                            const float* __restrict__ dAcs,
                                                            const float* init,
                                                            float* final_state,
                                                            __bf16* __restrict__ prev16, int keep_f32,
                                                            int H, int nc, int Q, int PN, int reverse) {
  constexpr int U = 8;
  const int h = blockIdx.y, b = blockIdx.z;
  const int e4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e4 >= PN) return;
  const size_t bh = (size_t)b * H + h;
  const float* dA = dAcs + bh * nc * Q + (Q - 1);
  float4 hs = make_float4(0.f, 0.f, 0.f, 0.f);
  if (init) hs = *reinterpret_cast<const float4*>(init + bh * PN + e4);
  const size_t cstride = (size_t)H * PN;
  float* s = states + ((size_t)b * nc * H + h) * PN + e4;

  for (int c0 = 0; c0 < nc; c0 += U) {
    float4 buf[U];
    float dec[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u < nc) {
        const int cc = reverse ? nc - 1 - (c0 + u) : c0 + u;
        buf[u] = *reinterpret_cast<const float4*>(s + (size_t)cc * cstride);
        dec[u] = expf(dA[(size_t)cc * Q]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u < nc) {
        const int cc = reverse ? nc - 1 - (c0 + u) : c0 + u;
        if (prev16) {
          // the scan's bf16 copy: the same rounding it would apply when staging fp32 states
          bf16x4 q;
          q[0] = static_cast<__bf16>(hs.x);
          q[1] = static_cast<__bf16>(hs.y);
          q[2] = static_cast<__bf16>(hs.z);
          q[3] = static_cast<__bf16>(hs.w);
          *reinterpret_cast<bf16x4*>(prev16 + ((size_t)b * nc * H + h) * PN + e4 + (size_t)cc * cstride) = q;
        }
        if (!prev16 || keep_f32) *reinterpret_cast<float4*>(s + (size_t)cc * cstride) = hs;
        hs.x = dec[u] * hs.x + buf[u].x;
        hs.y = dec[u] * hs.y + buf[u].y;
        hs.z = dec[u] * hs.z + buf[u].z;
        hs.w = dec[u] * hs.w + buf[u].w;
      }
    }
  }
  if (final_state) *reinterpret_cast<float4*>(final_state + bh * PN + e4) = hs;
}

hipError_t launch_state_passing(const FwdArgs& a, hipStream_t s) {
  const int PN = a.P * a.N;
  dim3 grid((PN / 4 + 255) / 256, a.H, a.B);
  hipExtLaunchKernelGGL(state_passing_kernel, grid, dim3(256), 0, s, a.ev0, a.ev1, 0, a.states, a.dAcs, a.init,
                        a.final_state, static_cast<__bf16*>(a.prev16), a.keep_f32_states, a.H, a.nc, a.Q, PN,
                                            a.passing_reverse);
  return hipGetLastError();
}

}  // namespace ssd
