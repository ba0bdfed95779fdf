// conv1d_silu: the causal depthwise convolution + SiLU in front of the scan,
//     u[t, c] = bias[c] + sum_k w[c, k] v[t - (K-1) + k, c],   out[t, c] = u / (1 + e^-u),
// over the channels of xBC = [x | B | C], with the output split back into x, B and C
// ("Agent 228: MAMBA-2 Implementation Gaps", Gap 2: kernel width d_conv, one filter per
// channel, causal padding d_conv - 1; SiLU after it as in section 3.1 of "Agent 228: MAMBA-2
// Reference Implementations Comparison").  Inputs before t = 0 come from the carried conv
// state (the last K - 1 inputs of the previous call, oldest first), zeros when none is given.
//
// Bandwidth bound: every input is read once from HBM and every output written once.
// One thread owns one 16-byte channel vector (4 fp32 / 8 bf16 channels) over a segment of
// consecutive tokens; consecutive lanes take consecutive vectors of a group of up to 64, so
// each token row is read and written as contiguous segments.  Segments are sized so that a
// 64-token segment per thread on large inputs (shorter ones when that leaves too few
// threads).  Each thread streams its segment 4 rows at a time with two register buffers, the
// loads of the next rows in flight while the current ones are convolved and stored, and the
// window sliding in registers; the K - 1 rows before a segment (its halo) are the only
// re-read (K-1 in 64).  Vectors never straddle the x / B / C boundaries (H*P and G*N are multiples of 16
// channels), so the split is a per-thread pointer choice.
//
// The conv state is written by the threads of the first run of each sequence, which are
// the only ones that read the incoming state, after they have read it: the state may be
// updated in place (state_out == state_in).
#include <algorithm>

#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

namespace {
constexpr int kRun = 4;            // rows per load batch of one thread (two batches in flight)
constexpr int kSegment = 64;       // tokens per thread on large inputs (measured best)
constexpr int64_t kMinThreads = 65536;   // below this, segments shrink to keep the chip busy

template <typename T>
__device__ __forceinline__ void to_floats(const Vec16<T>& v, float* f) {
#pragma unroll
  for (int e = 0; e < Vec16<T>::n; ++e) f[e] = to_f32(v.v[e]);
}

template <typename T>
__device__ __forceinline__ void store_vec(T* p, const float* f) {
  Vec16<T> o;
#pragma unroll
  for (int e = 0; e < Vec16<T>::n; ++e) o.v[e] = from_f32<T>(f[e]);
  *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(&o);
}

// Taps and bias of channels c0 .. c0+V-1 (weight rows are K contiguous floats).
template <int K, int V>
__device__ __forceinline__ void load_taps(const float* w, const float* bias, int c0, float (&wk)[K][V],
                                          float (&bv)[V]) {
#pragma unroll
  for (int e = 0; e < V; ++e) {
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k][e] = w[(size_t)(c0 + e) * K + k];
    bv[e] = bias ? bias[c0 + e] : 0.f;
  }
}

// Destination of channel vector c0 in the split outputs: base pointer and row stride.
template <typename T>
__device__ __forceinline__ T* split_dst(T* xo, T* bo, T* co, int c0, int dx, int dbc, size_t row, int& ld) {
  if (c0 < dx) {
    ld = dx;
    return xo + row * dx + c0;
  }
  ld = dbc;
  if (c0 < dx + dbc) return bo + row * dbc + (c0 - dx);
  return co + row * dbc + (c0 - dx - dbc);
}
}  // namespace

// Rows r .. r+TT-1 of one channel vector, rows past `last` clamped to it (cache hits, never stored).
template <typename T, int TT>
__device__ __forceinline__ void load_rows(Vec16<T> (&raw)[TT], const T* src, int r, int last, int Dc) {
#pragma unroll
  for (int i = 0; i < TT; ++i) raw[i] = load16(src + (size_t)min(r + i, last) * Dc);
}

// Convolve, activate and store rows r .. min(r+TT, end)-1; the window slides through them.
template <typename T, int K, int TT>
__device__ __forceinline__ void conv_rows(const Vec16<T> (&raw)[TT], float (&win)[K > 1 ? K - 1 : 1][Vec16<T>::n],
                                          const float (&wk)[K][Vec16<T>::n], const float (&bv)[Vec16<T>::n],
                                          T* dst, int ld, int r, int end) {
  constexpr int V = Vec16<T>::n;
  constexpr int KH = K - 1;
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    float cur[V], out[V];
    to_floats(raw[i], cur);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float u = bv[e] + wk[KH][e] * cur[e];
#pragma unroll
      for (int j = 0; j < KH; ++j) u += wk[j][e] * win[j][e];
      out[e] = silu(u);
    }
#pragma unroll
    for (int j = 0; j + 1 < KH; ++j)
#pragma unroll
      for (int e = 0; e < V; ++e) win[j][e] = win[j + 1][e];
    if constexpr (KH > 0) {
#pragma unroll
      for (int e = 0; e < V; ++e) win[KH - 1][e] = cur[e];
    }
    if (r + i < end) store_vec(dst + (size_t)(r + i) * ld, out);
  }
}

template <typename T, int K>
__global__ __launch_bounds__(256) void conv1d_silu_kernel(const T* __restrict__ xbc, const float* __restrict__ w,
                                                          const float* __restrict__ bias, const T* st_in,
                                                          T* st_out, T* __restrict__ xo, T* __restrict__ bo,
                                                          T* __restrict__ co, int L, int Dc, int dx, int dbc,
                                                          int NV, int VG, int seg, int nseg, uint32_t total,
                                                          uint32_t nblocks) {
  constexpr int V = Vec16<T>::n;
  constexpr int KH = K - 1;                         // halo / state rows
  constexpr int TT = kRun;
  // thread -> (batch, vector group, segment, vector in group)
  const uint32_t gid = xcd_swizzle(blockIdx.x, nblocks) * 256u + threadIdx.x;
  if (gid >= total) return;
  const int vin = (int)(gid % (uint32_t)VG);
  uint32_t rest = gid / (uint32_t)VG;
  const int sg = (int)(rest % (uint32_t)nseg);
  rest /= (uint32_t)nseg;
  const int ngrp = NV / VG;
  const int vec = (int)(rest % (uint32_t)ngrp) * VG + vin;
  const int b = (int)(rest / (uint32_t)ngrp);
  const int c0 = vec * V;
  const int t0 = sg * seg;
  const int t1 = min(L, t0 + seg);
  const T* src = xbc + (size_t)b * L * Dc + c0;

  if (t0 < t1) {
    // halo: the KH inputs before t0 (from the sequence, else the carried state, else zero),
    // loaded branch-free (a dummy in-bounds address where the value is zero) so that they
    // overlap the first rows' loads
    Vec16<T> hraw[KH > 0 ? KH : 1];
#pragma unroll
    for (int j = 0; j < KH; ++j) {
      const int s = t0 - KH + j;
      const bool in_seq = s >= 0, in_state = !in_seq && st_in != nullptr;
      const T* p = in_seq ? src + (size_t)s * Dc
                          : (in_state ? st_in + ((size_t)b * KH + KH + s) * Dc + c0 : src);
      hraw[j] = load16_if(p, in_seq || in_state);
    }
    // ping-pong: the next TT rows are in flight while the current ones are convolved and stored
    Vec16<T> ra[TT], rb[TT];
    const int last = t1 - 1;
    int r = t0;
    load_rows<T, TT>(ra, src, r, last, Dc);
    float wk[K][V], bv[V];
    load_taps<K, V>(w, bias, c0, wk, bv);
    int ld;
    T* dst = split_dst(xo, bo, co, c0, dx, dbc, (size_t)b * L, ld);
    float win[KH > 0 ? KH : 1][V];
#pragma unroll
    for (int j = 0; j < KH; ++j) to_floats(hraw[j], win[j]);
    while (true) {
      load_rows<T, TT>(rb, src, r + TT, last, Dc);
      conv_rows<T, K, TT>(ra, win, wk, bv, dst, ld, r, t1);
      r += TT;
      if (r >= t1) break;
      load_rows<T, TT>(ra, src, r + TT, last, Dc);
      conv_rows<T, K, TT>(rb, win, wk, bv, dst, ld, r, t1);
      r += TT;
      if (r >= t1) break;
    }
  }

  // New conv state: the inputs at times L-KH .. L-1, older ones (L < KH) from the incoming
  // state, whose row L + j feeds row j.  Written by the first segment of each sequence, the
  // only reader of the incoming state, after all its reads (every source row is loaded before
  // the first store): in-place updates are safe.
  if (st_out && sg == 0) {
    Vec16<T> nraw[KH > 0 ? KH : 1];
#pragma unroll
    for (int j = 0; j < KH; ++j) {
      const int s = L - KH + j;
      const bool in_seq = s >= 0, in_state = !in_seq && st_in != nullptr;
      if (in_seq)
        nraw[j] = load16(src + (size_t)s * Dc);
      else if (in_state)
        nraw[j] = load16(st_in + ((size_t)b * KH + KH + s) * Dc + c0);
      else
        nraw[j] = zero16<T>();
    }
#pragma unroll
    for (int j = 0; j < KH; ++j)
      *reinterpret_cast<uint4*>(st_out + ((size_t)b * KH + j) * Dc + c0) = *reinterpret_cast<const uint4*>(&nraw[j]);
  }
}

// One decode token per sequence: out = silu(bias + sum_k w_k v_k) over the carried state and
// the new input, then the state shifts by one row (in place; each thread owns its column).
template <typename T, int K>
__global__ __launch_bounds__(256) void conv1d_silu_step_kernel(const T* __restrict__ xbc,
                                                               const float* __restrict__ w,
                                                               const float* __restrict__ bias, T* state,
                                                               T* __restrict__ xo, T* __restrict__ bo,
                                                               T* __restrict__ co, int Dc, int dx, int dbc, int NV,
                                                               uint32_t total) {
  constexpr int V = Vec16<T>::n;
  constexpr int KH = K - 1;
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  if (gid >= total) return;
  const int vec = (int)(gid % (uint32_t)NV);
  const int b = (int)(gid / (uint32_t)NV);
  const int c0 = vec * V;

  float wk[K][V], bv[V];
  load_taps<K, V>(w, bias, c0, wk, bv);
  float win[KH > 0 ? KH : 1][V], cur[V], out[V];
#pragma unroll
  for (int j = 0; j < KH; ++j) to_floats(load16(state + ((size_t)b * KH + j) * Dc + c0), win[j]);
  to_floats(load16(xbc + (size_t)b * Dc + c0), cur);
#pragma unroll
  for (int e = 0; e < V; ++e) {
    float u = bv[e] + wk[KH][e] * cur[e];
#pragma unroll
    for (int j = 0; j < KH; ++j) u += wk[j][e] * win[j][e];
    out[e] = silu(u);
  }
  int ld;
  T* dst = split_dst(xo, bo, co, c0, dx, dbc, (size_t)b, ld);
  store_vec(dst, out);
#pragma unroll
  for (int j = 0; j + 1 < KH; ++j) store_vec(state + ((size_t)b * KH + j) * Dc + c0, win[j + 1]);
  if constexpr (KH > 0) store_vec(state + ((size_t)b * KH + KH - 1) * Dc + c0, cur);
}

template <typename T, int K>
static hipError_t launch_conv_impl(const ConvArgs& a, hipStream_t s) {
  const int NV = a.Dc / Vec16<T>::n;
  int VG = 64;                                       // vectors per group: the largest power of
  while (NV % VG) VG >>= 1;                          // two up to 64 that divides NV
  // segment length (a multiple of the run): kSegment tokens, fewer when that would leave
  // fewer than kMinThreads threads; or as set explicitly
  int seg = a.segment;
  if (seg <= 0) {
    const int64_t cols = (int64_t)a.B * NV;
    const int64_t rows = ((int64_t)a.L * cols + kMinThreads - 1) / kMinThreads;
    seg = (int)std::min<int64_t>(std::max<int64_t>(rows, kRun), kSegment);
  }
  seg = (seg + kRun - 1) / kRun * kRun;
  const int nseg = a.L > 0 ? (a.L + seg - 1) / seg : 1;
  const uint64_t total = (uint64_t)a.B * nseg * NV;
  if (total == 0) return hipSuccess;
  if (total > 0xffffff00ull) return hipErrorInvalidValue;
  const uint32_t nblocks = (uint32_t)((total + 255) / 256);
  conv1d_silu_kernel<T, K><<<nblocks, 256, 0, s>>>(
      static_cast<const T*>(a.xbc), a.w, a.bias, static_cast<const T*>(a.state_in), static_cast<T*>(a.state_out),
      static_cast<T*>(a.x), static_cast<T*>(a.Bo), static_cast<T*>(a.Co), a.L, a.Dc, a.dx, a.dbc, NV, VG, seg, nseg,
      (uint32_t)total, nblocks);
  return hipGetLastError();
}

template <typename T, int K>
static hipError_t launch_conv_step_impl(const ConvArgs& a, hipStream_t s) {
  const int NV = a.Dc / Vec16<T>::n;
  const uint32_t total = (uint32_t)a.B * NV;
  if (total == 0) return hipSuccess;
  conv1d_silu_step_kernel<T, K><<<(total + 255) / 256, 256, 0, s>>>(
      static_cast<const T*>(a.xbc), a.w, a.bias, static_cast<T*>(a.state_out), static_cast<T*>(a.x),
      static_cast<T*>(a.Bo), static_cast<T*>(a.Co), a.Dc, a.dx, a.dbc, NV, total);
  return hipGetLastError();
}

#define SSD_CONV_DISPATCH(FN)                                      \
  switch (a.K) {                                                   \
    case 1: return a.dtype == DT_F32 ? FN<float, 1>(a, s) : FN<__bf16, 1>(a, s); \
    case 2: return a.dtype == DT_F32 ? FN<float, 2>(a, s) : FN<__bf16, 2>(a, s); \
    case 3: return a.dtype == DT_F32 ? FN<float, 3>(a, s) : FN<__bf16, 3>(a, s); \
    case 4: return a.dtype == DT_F32 ? FN<float, 4>(a, s) : FN<__bf16, 4>(a, s); \
  }                                                                \
  return hipErrorInvalidValue;

hipError_t launch_conv1d_silu(const ConvArgs& a, hipStream_t s) { SSD_CONV_DISPATCH(launch_conv_impl) }
hipError_t launch_conv1d_silu_step(const ConvArgs& a, hipStream_t s) { SSD_CONV_DISPATCH(launch_conv_step_impl) }

#undef SSD_CONV_DISPATCH

}  // namespace ssd
