// chunk_state: the state each chunk contributes on its own, decayed to the chunk's end,
//     S[b,c,h,p,n] = sum_i x[b,cQ+i,h,p] * w_i * B[b,cQ+i,g,n],
//     w_i = exp(dAcs[last] - dAcs[i]) * dt'_i
// (the "diagonal block" local state of each chunk: Gap 1 of "Agent 228: MAMBA-2
// Implementation Gaps" and section 3.2 of "Agent 228: MAMBA-2 Reference Implementations
// Comparison"; the decay of the carried state from position i to the chunk end is the
// product of the per-step decays exp(dt' A), i.e. exp of the cumsum difference).
//
// One workgroup (4 wavefronts) per (b, c, h).  A (P x Q) . (Q x N) product on MFMA with
// fp32 accumulation: the contraction runs over tokens, which are the slow axis of x and B
// in HBM, so 64-token tiles are staged transposed in LDS (token-contiguous rows) where both
// operands can be read with one LDS load per fragment.  The per-token weight w_i is folded
// into x while staging.  Tokens past the end of the sequence are zero-filled.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename T, int P, int N>
__global__ __launch_bounds__(256) void chunk_state_kernel(const T* __restrict__ x,
                                                          const T* __restrict__ Bm,
                                                          const float* __restrict__ dtp,
                                                          const float* __restrict__ dAcs,
                                                          float* __restrict__ states,
                                                          int L, int H, int G, int nc, int Q,
                                                          uint32_t nblocks) {
  typedef KMma<T> M;
  constexpr int KT = 64;                           // tokens per LDS tile
  constexpr int PITCH = KT + (sizeof(T) == 4 ? 2 : 8);
  constexpr int VEC = Vec16<T>::n;
  constexpr int TP = P / 16, TN = N / 16;
  // wavefront layout over the (TP x TN) grid of 16x16 output tiles
  constexpr int WAVES_N = TN < 4 ? TN : 4;
  constexpr int WAVES_P = 4 / WAVES_N;
  constexpr int WN = TN / WAVES_N;
  constexpr int WP = (TP + WAVES_P - 1) / WAVES_P;

  __shared__ __attribute__((aligned(16))) T s_x[P][PITCH];   // (x * w)^T
  __shared__ __attribute__((aligned(16))) T s_b[N][PITCH];   // B^T
  __shared__ float s_w[256];

  uint32_t id = xcd_swizzle(blockIdx.x, nblocks);
  const int h = id % H;
  id /= H;
  const int c = id % nc;
  const int b = id / nc;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int len = min(Q, L - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;

  const float* dtp_c = dtp + (((size_t)b * H + h) * nc + c) * Q;
  const float* dA_c = dAcs + (((size_t)b * H + h) * nc + c) * Q;
  const float last = dA_c[Q - 1];
  for (int i = tid; i < Q; i += 256) s_w[i] = expf(last - dA_c[i]) * dtp_c[i];

  const int wn = wave % WAVES_N, wp = wave / WAVES_N;
  f32x4 acc[WP][WN];
#pragma unroll
  for (int i = 0; i < WP; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = zero4();

  const size_t x_tok_stride = (size_t)H * P;
  const size_t b_tok_stride = (size_t)G * N;
  const T* xb = x + ((size_t)b * L + t0) * x_tok_stride + (size_t)h * P;
  const T* bb = Bm + ((size_t)b * L + t0) * b_tok_stride + (size_t)g * N;

  for (int k0 = 0; k0 < len; k0 += KT) {
    __syncthreads();  // previous tile consumed (and s_w written, first time)
    for (int v = tid; v < KT * (P / VEC); v += 256) {
      const int i = v / (P / VEC), pv = (v % (P / VEC)) * VEC;
      const int tok = k0 + i;
      Vec16<T> d = (tok < len) ? load16(xb + (size_t)tok * x_tok_stride + pv) : zero16<T>();
      const float w = s_w[tok];
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_x[pv + e][i] = from_f32<T>(to_f32(d.v[e]) * w);
    }
    for (int v = tid; v < KT * (N / VEC); v += 256) {
      const int i = v / (N / VEC), nv = (v % (N / VEC)) * VEC;
      const int tok = k0 + i;
      Vec16<T> d = (tok < len) ? load16(bb + (size_t)tok * b_tok_stride + nv) : zero16<T>();
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_b[nv + e][i] = d.v[e];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KT; ks += M::K) {
      typename M::frag af[WP], bf[WN];
#pragma unroll
      for (int i = 0; i < WP; ++i) {
        const int tp = wp * WP + i;
        af[i] = (tp < TP) ? M::load(&s_x[tp * 16 + r][ks + qd * M::KPL]) : M::zero();
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) bf[j] = M::load(&s_b[(wn * WN + j) * 16 + r][ks + qd * M::KPL]);
#pragma unroll
      for (int i = 0; i < WP; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = M::mma(af[i], bf[j], acc[i][j]);
    }
  }

  float* out = states + (((size_t)b * nc + c) * H + h) * (size_t)(P * N);
#pragma unroll
  for (int i = 0; i < WP; ++i) {
    const int tp = wp * WP + i;
    if (tp >= TP) continue;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = (wn * WN + j) * 16 + r;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[(size_t)(tp * 16 + qd * 4 + e) * N + n] = acc[i][j][e];
    }
  }
}

template <typename T, int P, int N>
static hipError_t launch_state_impl(const FwdArgs& a, hipStream_t s) {
  const uint32_t nblocks = (uint32_t)a.B * a.nc * a.H;
  chunk_state_kernel<T, P, N><<<nblocks, 256, 0, s>>>(
      static_cast<const T*>(a.x), static_cast<const T*>(a.Bm), a.dtp, a.dAcs, a.states, a.L, a.H, a.G,
      a.nc, a.Q, nblocks);
  return hipGetLastError();
}

hipError_t launch_chunk_state(const FwdArgs& a, hipStream_t s) {
#define SSD_CASE(T, P_, N_) \
  if (a.dtype == SSD_DTYPE_CODE_##T && a.P == P_ && a.N == N_) return launch_state_impl<T, P_, N_>(a, s);
  SSD_FOR_EACH_SHAPE(SSD_CASE)
#undef SSD_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
