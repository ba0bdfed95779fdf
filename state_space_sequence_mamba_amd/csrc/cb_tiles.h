// Pieces shared by chunk_state and chunk_scan: the contraction over dstate of two
// n-contiguous rows on MFMA (NDot), and the C B^T sub-tile blocks computed once per group.
#pragma once

#include "ssd_common.h"

namespace ssd {

constexpr int kCbKT = 64;                     // tokens per row block
constexpr int kCbBlock = 16 * 256;            // floats per (row block, column block) of C B^T

// Contraction over dstate of two n-contiguous rows.
template <typename T, int N> struct NDot;
template <int N> struct NDot<float, N> {
  static constexpr int NF = N / 4;                // k values per lane: n = (N/4) qd + kk
  typedef float frag[NF];
  __device__ static __forceinline__ void load(frag f, const float* row, int qd, bool ok = true) {
    const float* p = row + (N / 4) * qd;
#pragma unroll
    for (int m = 0; m < NF / 4; ++m) {
      const float4 v = *reinterpret_cast<const float4*>(p + 4 * m);
      f[4 * m + 0] = ok ? v.x : 0.f;
      f[4 * m + 1] = ok ? v.y : 0.f;
      f[4 * m + 2] = ok ? v.z : 0.f;
      f[4 * m + 3] = ok ? v.w : 0.f;
    }
  }
  __device__ static __forceinline__ f32x4 dot(const frag a, const frag b, f32x4 c) {
#pragma unroll
    for (int k = 0; k < NF; ++k) c = mfma_16x16x4_f32(a[k], b[k], c);
    return c;
  }
};
template <int N> struct NDot<__bf16, N> {
  static constexpr int NF = N / 32;               // 16x16x32 instructions: n = 32 k + 8 qd + e
  typedef bf16x8 frag[NF];
  __device__ static __forceinline__ void load(frag f, const __bf16* row, int qd, bool ok = true) {
#pragma unroll
    for (int k = 0; k < NF; ++k) {
      uint4 v = *reinterpret_cast<const uint4*>(row + 32 * k + 8 * qd);
      v.x = ok ? v.x : 0u;
      v.y = ok ? v.y : 0u;
      v.z = ok ? v.z : 0u;
      v.w = ok ? v.w : 0u;
      f[k] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __device__ static __forceinline__ f32x4 dot(const frag a, const frag b, f32x4 c) {
#pragma unroll
    for (int k = 0; k < NF; ++k) c = mfma_16x16x32_bf16(a[k], b[k], c);
    return c;
  }
};

// One block of C B^T sub-tiles (fp32 values, from fp32 or bf16 B and C): for (batch, chunk, group) and the row block / column
// block pair (rb, J <= rb) numbered blk = rb (rb + 1) / 2 + J, the 16 causal 16 x 16
// sub-tiles (strip 4 rb + w, column tile 4 J + js) that the scan's rows decomposition
// consumes, computed once per group instead of once per head.  Stored as 16 KB in the lane
// order of the scan's A operand (each scan wavefront loads its four sub-tiles with one
// 16-byte load per lane each): sub-tile (w, js), lane l, element e at ((4 w + js) 64 + l) 4 + e,
// i.e. lane (r, qd) holds CB[i = 16 (4 rb + w) + r][j = 16 (4 J + js) + 4 qd + e].  The MFMA
// sequence is the scan's own, so results are bit-identical to computing in place.  Sub-tiles
// past the diagonal and rows past the sequence are zeros.  Four wavefronts (tid in [0, 256)),
// one per strip.
// TRANS: the layout the backward's anti-causal kernel (bwd_dxdb) consumes: lane (r, qd) of
// sub-tile (w, js) holds CB[i = 16 (4 rb + w) + 4 qd + e][j = 16 (4 J + js) + r] (the MFMA with
// C as its A operand, as bwd_dxdb forms it), stored at ((4 js + w) 64 + l) 4 + e so that the
// wavefront owning column tile js reads its four row tiles contiguously.
template <typename T, int N, bool TRANS = false>
__device__ __forceinline__ void cb_block(const T* __restrict__ Bm, const T* __restrict__ Cm,
                                         float* __restrict__ cb, int L, int G, int nc, int Q, uint32_t id,
                                         int tid) {
  typedef NDot<T, N> ND;
  const int nrb = Q / kCbKT, nblk = nrb * (nrb + 1) / 2;
  const int blk = id % nblk;
  id /= nblk;
  const int g = id % G;
  id /= G;
  const int c = id % nc, b = id / nc;
  int rb = 0;
  while ((rb + 1) * (rb + 2) / 2 <= blk) ++rb;
  const int J = blk - rb * (rb + 1) / 2;
  const int t0 = c * Q, len = min(Q, L - t0);
  const int lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;
  const int strip = 4 * rb + w;
  const size_t bc_tok = (size_t)G * N;
  const T* Cb = Cm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  const T* Bb = Bm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  float* out = cb + ((((size_t)b * nc + c) * G + g) * nblk + blk) * (size_t)kCbBlock;
  // the fragment loads of JB column tiles are issued before their MFMAs (all four at once
  // where the registers allow it, two by two for bf16, whose caller keeps fewer)
  constexpr int JB = sizeof(T) == 4 ? 4 : 2;
  typename ND::frag cf, bfr[JB];
  const int i = 16 * strip + r;
  ND::load(cf, Cb + (size_t)(i < len ? i : 0) * bc_tok, qd, i < len);
#pragma unroll
  for (int j0 = 0; j0 < 4; j0 += JB) {
#pragma unroll
    for (int u = 0; u < JB; ++u) {
      const int j = 16 * (4 * J + j0 + u) + r;
      ND::load(bfr[u], Bb + (size_t)(j < len ? j : 0) * bc_tok, qd, j < len);
    }
#pragma unroll
    for (int u = 0; u < JB; ++u) {
      const int js = j0 + u;
      if constexpr (TRANS) {
        const f32x4 cbt = (4 * J + js <= strip) ? ND::dot(cf, bfr[u], zero4()) : zero4();
        *reinterpret_cast<f32x4*>(out + ((js * 4 + w) * 64 + lane) * 4) = cbt;
      } else {
        const f32x4 cbt = (4 * J + js <= strip) ? ND::dot(bfr[u], cf, zero4()) : zero4();
        *reinterpret_cast<f32x4*>(out + ((w * 4 + js) * 64 + lane) * 4) = cbt;
      }
    }
  }
}

}  // namespace ssd
