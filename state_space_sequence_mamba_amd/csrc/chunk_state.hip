// chunk_state: the state each chunk contributes on its own, decayed to the chunk's end,
//     S[b,c,h,p,n] = sum_i x[b,cQ+i,h,p] * w_i * B[b,cQ+i,g,n],
//     w_i = exp(dAcs[last] - dAcs[i]) * dt'_i
// (the "diagonal block" local state of each chunk: Gap 1 of "Agent 228: MAMBA-2
// Implementation Gaps" and section 3.2 of "Agent 228: MAMBA-2 Reference Implementations
// Comparison"; the decay of the carried state from position i to the chunk end is the
// product of the per-step decays exp(dt' A), i.e. exp of the cumsum difference).
// The backward pass reuses it with (dy, C) in place of (x, B) and w_i = exp(dAcs[i]): the
// gradient that chunk c's outputs send into the state entering the chunk.
//
// One workgroup (8 wavefronts, two 16x16 output tiles each at P = N = 64) per (b, c, h);
// its wavefront 0 first computes the chunk's dt' and their cumsum (chunk_cumsum_wave
// below), which the other kernels read from the workspace.  A (P x Q) . (Q x N) product on
// MFMA with fp32 accumulation.  The contraction runs over tokens, the slow axis of x and B in HBM, so
// 64-token tiles are staged transposed in LDS (token-contiguous rows): each thread loads
// the same 16-byte column slice of two consecutive tokens and writes them as one packed
// pair, which keeps the transposed LDS writes free of bank conflicts.  The next tile's
// global loads are issued into registers before the current tile's MFMAs.  The per-token
// weight w_i is folded into x while staging.  Tokens past the end of the sequence are zero.
// fp32 fragments use the token permutation k = (KT/4) qd + kk so that each lane reads 128 bits.
#include "cb_tiles.h"
#include "ssd_common.h"
#include "ssd_launch.h"

// (dtype, P, N, PS) of the one-pass chunk-state kernel
#define SSD_FOR_EACH_SEQ_SHAPE(X) \
  X(float, 64, 64, 32) X(float, 64, 64, 64) X(__bf16, 64, 128, 64)

namespace ssd {

// dt' = softplus(dt + dt_bias) (optionally clamped to [lo, hi], the dt limits of section 5.2
// of the reference-comparison page) and the inclusive in-chunk cumulative sum of dt' A, for
// one (b, c, h), by one wavefront: each lane scans Q/64 consecutive positions serially, then
// the 64 lane totals are combined by a log-step shuffle scan (the up-sweep idea of the
// parallel-scan section of "Agent 230: Comprehensive MAMBA-2 Implementation Comparison", on
// 64-wide wavefronts).  Positions past the end of the sequence get dt' = 0, so the cumsum
// stays flat there.  Results go to the workspace (for state_passing and chunk_scan) and to LDS.
template <typename T>
__device__ __forceinline__ void chunk_cumsum_wave(const T* __restrict__ dt, float bias, float a, size_t tok0,
                                                  int H, int h, int len, int Q, int clamp, float lo, float hi,
                                                  float* __restrict__ dtp_c, float* __restrict__ dA_c,
                                                  float* s_d, float* s_cs, int lane) {
  const int epl = Q >> 6;                      // positions per lane: 1, 2 or 4
  const int i0 = lane * epl;
  float raw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    raw[k] = 0.f;
    if (k < epl && i0 + k < len) raw[k] = to_f32(dt[(tok0 + i0 + k) * H + h]);
  }
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
  // inclusive scan of the lane totals (DPP lane moves), then shifted by one lane for the
  // exclusive prefix
  const float excl = wave_shr1(wave_incl_scan(run));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k < epl) {
      dtp_c[i0 + k] = d[k];
      dA_c[i0 + k] = cs[k] + excl;
      s_d[i0 + k] = d[k];
      s_cs[i0 + k] = cs[k] + excl;
    }
  }
}

// Forward: workgroups [ncb_wg, ncb_wg + nblocks) compute the chunk states (each first the dt'
// cumsum of its own (b, c, h)); when the scan reads C B^T formed once per group (fp32, and bf16
// with many heads per group), the first ncb_wg workgroups compute those blocks (cb_block):
// dispatched ahead of the state workgroups, they overlap them instead of forming a tail behind
// the last ones.  Backward (from_start): dt' and the cumsum are read from the workspace.
template <typename T, int P, int N, int NTHR>
__global__ __launch_bounds__(NTHR, sizeof(T) == 2 ? 6 : 1) void chunk_state_kernel(const T* __restrict__ x,
                                                          const T* __restrict__ Bm,
                                                          const T* __restrict__ Cm,
                                                          const T* __restrict__ dt,
                                                          const float* __restrict__ dt_bias,
                                                          const float* __restrict__ A,
                                                          float* __restrict__ dtp,
                                                          float* __restrict__ dAcs,
                                                          float* __restrict__ states,
                                                          float* __restrict__ cb, float* __restrict__ cbT,
                                                          int L, int H, int G, int nc, int Q,
                                                          uint32_t nblocks, uint32_t ncb, uint32_t ncb_wg,
                                                          int from_start, int clamp, float lo, float hi) {
  if (blockIdx.x < ncb_wg) {
    // the C B^T blocks first (dispatched with the first state workgroups rather than as a
    // tail behind the last ones); NTHR / 256 blocks per workgroup, four wavefronts each
    const uint32_t id = blockIdx.x * (NTHR / 256) + threadIdx.x / 256;
    if (id < ncb)
      cb_block<T, N>(Bm, Cm, cb, L, G, nc, Q, id, threadIdx.x & 255);
    else if (cbT && id < 2 * ncb)       // the backward's transposed copy
      cb_block<T, N, true>(Bm, Cm, cbT, L, G, nc, Q, id - ncb, threadIdx.x & 255);
    return;
  }
  constexpr bool F32 = sizeof(T) == 4;
  constexpr int KT = 64;                                 // tokens per LDS tile
  constexpr int PITCH = KT + (F32 ? 4 : 8);              // 16-byte aligned rows
  constexpr int VEC = Vec16<T>::n;
  constexpr int PV = P / VEC, NV = N / VEC;
  constexpr int XU = (KT / 2) * PV, BU = (KT / 2) * NV;  // token-pair units per tile
  constexpr int XPT = (XU + NTHR - 1) / NTHR, BPT = (BU + NTHR - 1) / NTHR;
  constexpr int TP = P / 16, TN = N / 16;
  // wavefront layout over the (TP x TN) grid of 16x16 output tiles
  constexpr int NW = NTHR / 64;
  constexpr int WAVES_N = TN < NW ? TN : NW;
  constexpr int WAVES_P = NW / WAVES_N;
  constexpr int WN = TN / WAVES_N;
  constexpr int WP = (TP + WAVES_P - 1) / WAVES_P;

  __shared__ __attribute__((aligned(16))) T s_x[P * PITCH];   // (x * w)^T
  __shared__ __attribute__((aligned(16))) T s_b[N * PITCH];   // B^T
  __shared__ float s_w[256];
  __shared__ float s_d[256], s_cs[256];

  uint32_t id = xcd_swizzle(blockIdx.x - ncb_wg, nblocks);   // ncb_wg % 8 == 0: XCDs unchanged
  const int h = id % H;
  id /= H;
  const int c = id % nc;
  const int b = id / nc;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int len = min(Q, L - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;

  const size_t xs = (size_t)H * P, bs = (size_t)G * N;    // token strides
  const T* xb = x + ((size_t)b * L + t0) * xs + (size_t)h * P;
  const T* bb = Bm + ((size_t)b * L + t0) * bs + (size_t)g * N;

  // Tile registers: loads read clamped in-bounds addresses and only record which tokens are
  // real; the zeroing selects happen when the tile is written to LDS, so the next tile's
  // loads stay in flight during the current tile's MFMAs.
  Vec16<T> xr[XPT][2], br[BPT][2];
  uint32_t okm = 0;
  const uint32_t xs32 = (uint32_t)xs, bs32 = (uint32_t)bs;
  auto load_tile = [&](int k0) {
    okm = 0;
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int v = min(tid + NTHR * u, XU - 1);
      const int m = v % (KT / 2), pv = (v / (KT / 2)) * VEC;
      const int tok = k0 + 2 * m;
      const bool ok0 = tok < len, ok1 = tok + 1 < len;
      xr[u][0] = load16(xb + (uint32_t)(ok0 ? tok : 0) * xs32 + pv);
      xr[u][1] = load16(xb + (uint32_t)(ok1 ? tok + 1 : 0) * xs32 + pv);
      okm |= ((uint32_t)ok0 << (2 * u)) | ((uint32_t)ok1 << (2 * u + 1));
    }
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const int v = min(tid + NTHR * u, BU - 1);
      const int m = v % (KT / 2), nv = (v / (KT / 2)) * VEC;
      const int tok = k0 + 2 * m;
      const bool ok0 = tok < len, ok1 = tok + 1 < len;
      br[u][0] = load16(bb + (uint32_t)(ok0 ? tok : 0) * bs32 + nv);
      br[u][1] = load16(bb + (uint32_t)(ok1 ? tok + 1 : 0) * bs32 + nv);
      okm |= ((uint32_t)ok0 << (2 * XPT + 2 * u)) | ((uint32_t)ok1 << (2 * XPT + 2 * u + 1));
    }
  };
  auto store_tile = [&](int k0) {
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int v = tid + NTHR * u;
      if (XU % NTHR == 0 || v < XU) {
        const int m = v % (KT / 2), pv = (v / (KT / 2)) * VEC;
        const float w0 = s_w[k0 + 2 * m], w1 = s_w[k0 + 2 * m + 1];
        const Vec16<T> x0 = keep_if(xr[u][0], (okm >> (2 * u)) & 1u);
        const Vec16<T> x1 = keep_if(xr[u][1], (okm >> (2 * u + 1)) & 1u);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          T pair[2] = {from_f32<T>(to_f32(x0.v[e]) * w0), from_f32<T>(to_f32(x1.v[e]) * w1)};
          __builtin_memcpy(&s_x[(pv + e) * PITCH + 2 * m], pair, sizeof(pair));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const int v = tid + NTHR * u;
      if (BU % NTHR == 0 || v < BU) {
        const int m = v % (KT / 2), nv = (v / (KT / 2)) * VEC;
        const Vec16<T> b0 = keep_if(br[u][0], (okm >> (2 * XPT + 2 * u)) & 1u);
        const Vec16<T> b1 = keep_if(br[u][1], (okm >> (2 * XPT + 2 * u + 1)) & 1u);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          T pair[2] = {b0.v[e], b1.v[e]};
          __builtin_memcpy(&s_b[(nv + e) * PITCH + 2 * m], pair, sizeof(pair));
        }
      }
    }
  };

  const int wn = wave % WAVES_N, wp = wave / WAVES_N;
  f32x4 acc[WP][WN];
#pragma unroll
  for (int i = 0; i < WP; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = zero4();

  load_tile(0);                            // in flight while the weights are computed
  float* dtp_c = dtp + (((size_t)b * H + h) * nc + c) * Q;
  float* dA_c = dAcs + (((size_t)b * H + h) * nc + c) * Q;
  if (from_start) {
    // backward: decay from the chunk's start, exp(dAcs_i), which weighs each output's
    // gradient into the state entering the chunk
    for (int i = tid; i < Q; i += NTHR) s_w[i] = expf(dA_c[i]);
  } else {
    // forward: decay to the chunk's end times the step
    if (wave == 0)
      chunk_cumsum_wave<T>(dt, dt_bias[h], A[h], (size_t)b * L + t0, H, h, len, Q, clamp, lo, hi, dtp_c, dA_c,
                           s_d, s_cs, lane);
    __syncthreads();
    const float last = s_cs[Q - 1];
    for (int i = tid; i < Q; i += NTHR) s_w[i] = expf(last - s_cs[i]) * s_d[i];
  }

  for (int k0 = 0; k0 < len; k0 += KT) {
    __syncthreads();                       // previous tile consumed; s_w written
    store_tile(k0);
    if (k0 + KT < len) load_tile(k0 + KT);  // next tile's loads overlap this tile's MFMAs
    __syncthreads();
    if (F32) {
#pragma unroll
      for (int m = 0; m < KT / 16; ++m) {
        float4 af[WP], bf[WN];
#pragma unroll
        for (int i = 0; i < WP; ++i) {
          const int tp = wp * WP + i;
          const int tpc = tp < TP ? tp : TP - 1;  // clamped read, zeroed by select
          const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(s_x) +
                                                            (tpc * 16 + r) * PITCH + (KT / 4) * qd + 4 * m);
          af[i] = (tp < TP) ? v : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < WN; ++j)
          bf[j] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(s_b) +
                                                   ((wn * WN + j) * 16 + r) * PITCH + (KT / 4) * qd + 4 * m);
#pragma unroll
        for (int i = 0; i < WP; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            acc[i][j] = mfma_16x16x4_f32(af[i].x, bf[j].x, acc[i][j]);
            acc[i][j] = mfma_16x16x4_f32(af[i].y, bf[j].y, acc[i][j]);
            acc[i][j] = mfma_16x16x4_f32(af[i].z, bf[j].z, acc[i][j]);
            acc[i][j] = mfma_16x16x4_f32(af[i].w, bf[j].w, acc[i][j]);
          }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KT / 32; ++kk) {
        bf16x8 af[WP], bf[WN];
#pragma unroll
        for (int i = 0; i < WP; ++i) {
          const int tp = wp * WP + i;
          const int tpc = tp < TP ? tp : TP - 1;
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(s_x) +
                                                            (tpc * 16 + r) * PITCH + 32 * kk + 8 * qd);
          af[i] = (tp < TP) ? v : KMma<__bf16>::zero();
        }
#pragma unroll
        for (int j = 0; j < WN; ++j)
          bf[j] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(s_b) +
                                                   ((wn * WN + j) * 16 + r) * PITCH + 32 * kk + 8 * qd);
#pragma unroll
        for (int i = 0; i < WP; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j) acc[i][j] = mfma_16x16x32_bf16(af[i], bf[j], acc[i][j]);
      }
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

// Forward, chunk states and their recurrence in one pass: one workgroup per (b, h, slice of PS
// headdim rows) walks the chunks in order, keeping the running state H in its MFMA
// accumulators.  At the start of chunk c it writes H_c (the state entering the chunk: fp32 for
// fp32 inputs, rounded to bf16 for bf16 inputs, the copy the scan reads), scales H by the
// chunk's total decay exp(dAcs[last]) and then accumulates that chunk's x^T diag(w) B tiles
// into it, which is H_{c+1} = exp(dAcs_c[last]) H_c + S_c with S_c summed straight into the
// carried state; after the last chunk H is the final state.  Each chunk's own state never goes
// to memory, and no separate state_passing launch is needed.
// The loop is chunk-major with the TPC tiles of a chunk unrolled; tile loads run one chunk
// (TPC tiles) ahead through a ring of register sets, and the dt of the next chunk is loaded at
// the start of the current one.  Every global load is unconditional (addresses clamped in
// bounds, tokens past the end zeroed by flags), so the compiler's wait counts stay exact and
// no wait drains the ring.  When the scan reads C B^T formed once per group, the first ncb_wg
// workgroups form those blocks.
template <typename T, int P, int N, int PS, int NTHR, int TPC>
__global__ __launch_bounds__(NTHR) void chunk_state_seq_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm, const T* __restrict__ dt,
    const float* __restrict__ dt_bias, const float* __restrict__ A, float* __restrict__ dtp,
    float* __restrict__ dAcs, float* __restrict__ states, __bf16* __restrict__ prev16,
    const float* __restrict__ init, float* __restrict__ final_state, float* __restrict__ cb, int L, int H,
    int G, int nc, uint32_t nseq, uint32_t ncb, uint32_t ncb_wg, int clamp, float lo, float hi) {
  constexpr int KT = 64;                                 // tokens per LDS tile
  constexpr int Q = TPC * KT;
  if (blockIdx.x < ncb_wg) {
    const uint32_t id = blockIdx.x * (NTHR / 256) + threadIdx.x / 256;
    if (id < ncb) cb_block<T, N>(Bm, Cm, cb, L, G, nc, Q, id, threadIdx.x & 255);
    return;
  }
  constexpr bool F32 = sizeof(T) == 4;
  constexpr int PITCH = KT + (F32 ? 4 : 8);
  constexpr int VEC = Vec16<T>::n;
  constexpr int PV = PS / VEC, NV = N / VEC;
  constexpr int XU = (KT / 2) * PV, BU = (KT / 2) * NV;  // token-pair units per tile
  constexpr int XPT = (XU + NTHR - 1) / NTHR, BPT = (BU + NTHR - 1) / NTHR;
  constexpr int TP = PS / 16, TN = N / 16;
  constexpr int NW = NTHR / 64;
  constexpr int WAVES_N = TN < NW ? TN : NW;
  constexpr int WAVES_P = NW / WAVES_N;
  constexpr int WN = TN / WAVES_N;
  constexpr int WP = (TP + WAVES_P - 1) / WAVES_P;
  constexpr int NS = P / PS;
  constexpr int EPL = Q / 64;                            // cumsum positions per lane

  __shared__ __attribute__((aligned(16))) T s_x[PS * PITCH];   // (x * w)^T, this slice's rows
  __shared__ __attribute__((aligned(16))) T s_b[N * PITCH];    // B^T
  __shared__ float s_d[Q], s_w[Q];
  __shared__ float s_last;

  uint32_t id = xcd_swizzle(blockIdx.x - ncb_wg, nseq);   // consecutive ids share b (and B)
  const int sl = id % NS;
  id /= NS;
  const int h = id % H;
  const int b = id / H;
  const int g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;
  const int wn = wave % WAVES_N, wp = wave / WAVES_N;

  const size_t xs = (size_t)H * P, bs = (size_t)G * N;    // token strides
  const uint32_t xs32 = (uint32_t)xs, bs32 = (uint32_t)bs;
  const T* xb = x + (size_t)b * L * xs + (size_t)h * P + sl * PS;
  const T* bb = Bm + (size_t)b * L * bs + (size_t)g * N;
  const size_t PN = (size_t)P * N;
  const size_t bh = (size_t)b * H + h;

  // ---- tile ring
  Vec16<T> xr[TPC][XPT][2], br[TPC][BPT][2];
  uint32_t okm[TPC];
  auto load_tile = [&](Vec16<T> (&xq)[XPT][2], Vec16<T> (&bq)[BPT][2], uint32_t& ok, int tb) {
    const int rem = L - tb;                                // real tokens from tb on (may be <= 0)
    const size_t base = rem > 0 ? (size_t)tb : 0;          // past the end: read token 0, zeroed
    const T* xt = xb + base * xs;
    const T* bt = bb + base * bs;
    ok = 0;
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int v = min(tid + NTHR * u, XU - 1);
      const int m = v % (KT / 2), pv = (v / (KT / 2)) * VEC;
      const int tok = 2 * m;
      const bool ok0 = tok < rem, ok1 = tok + 1 < rem;
      xq[u][0] = load16(xt + (uint32_t)(ok0 ? tok : 0) * xs32 + pv);
      xq[u][1] = load16(xt + (uint32_t)(ok1 ? tok + 1 : 0) * xs32 + pv);
      ok |= ((uint32_t)ok0 << (2 * u)) | ((uint32_t)ok1 << (2 * u + 1));
    }
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const int v = min(tid + NTHR * u, BU - 1);
      const int m = v % (KT / 2), nv = (v / (KT / 2)) * VEC;
      const int tok = 2 * m;
      const bool ok0 = tok < rem, ok1 = tok + 1 < rem;
      bq[u][0] = load16(bt + (uint32_t)(ok0 ? tok : 0) * bs32 + nv);
      bq[u][1] = load16(bt + (uint32_t)(ok1 ? tok + 1 : 0) * bs32 + nv);
      ok |= ((uint32_t)ok0 << (2 * XPT + 2 * u)) | ((uint32_t)ok1 << (2 * XPT + 2 * u + 1));
    }
  };
  // a loaded register made opaque where it is stored, so that no work on it (the bf16 pair
  // packing) is hoisted up to its load, which would wait for the load there
  auto opaque = [](const Vec16<T>& q) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 t;
    __builtin_memcpy(&t, &q, 16);
    asm volatile("" : "+v"(t));
    Vec16<T> o;
    __builtin_memcpy(&o, &t, 16);
    return o;
  };
  auto store_tile = [&](const Vec16<T> (&xq)[XPT][2], const Vec16<T> (&bq)[BPT][2], uint32_t ok, int k0) {
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int v = tid + NTHR * u;
      if (XU % NTHR == 0 || v < XU) {
        const int m = v % (KT / 2), pv = (v / (KT / 2)) * VEC;
        const float w0 = s_w[k0 + 2 * m], w1 = s_w[k0 + 2 * m + 1];
        const Vec16<T> x0 = keep_if(opaque(xq[u][0]), (ok >> (2 * u)) & 1u);
        const Vec16<T> x1 = keep_if(opaque(xq[u][1]), (ok >> (2 * u + 1)) & 1u);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          T pair[2] = {from_f32<T>(to_f32(x0.v[e]) * w0), from_f32<T>(to_f32(x1.v[e]) * w1)};
          __builtin_memcpy(&s_x[(pv + e) * PITCH + 2 * m], pair, sizeof(pair));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const int v = tid + NTHR * u;
      if (BU % NTHR == 0 || v < BU) {
        const int m = v % (KT / 2), nv = (v / (KT / 2)) * VEC;
        const Vec16<T> b0 = keep_if(opaque(bq[u][0]), (ok >> (2 * XPT + 2 * u)) & 1u);
        const Vec16<T> b1 = keep_if(opaque(bq[u][1]), (ok >> (2 * XPT + 2 * u + 1)) & 1u);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          T pair[2] = {b0.v[e], b1.v[e]};
          __builtin_memcpy(&s_b[(nv + e) * PITCH + 2 * m], pair, sizeof(pair));
        }
      }
    }
  };

  // ---- dt: one position of the next chunk per thread (clamped in-bounds read)
  const int dpos = tid % Q;
  auto load_dt = [&](int c) {
    return dt[((size_t)b * L + min(c * Q + dpos, L - 1)) * H + h];
  };
  const float bias = dt_bias[h], av = A[h];

  // ---- the carried state (initial state read and waited for before the ring's loads)
  f32x4 acc[WP][WN];
#pragma unroll
  for (int i = 0; i < WP; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = zero4();
  if (init) {
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int tp = wp * WP + i;
      if (tp >= TP) continue;
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int n = (wn * WN + j) * 16 + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = init[bh * PN + (size_t)(sl * PS + tp * 16 + qd * 4 + e) * N + n];
        asm volatile("" : "+v"(acc[i][j]));              // wait here, not inside the loop
      }
    }
  }
  auto write_state = [&](float* f32dst, __bf16* bf16dst) {
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int tp = wp * WP + i;
      if (tp >= TP) continue;
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int n = (wn * WN + j) * 16 + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const size_t o = (size_t)(sl * PS + tp * 16 + qd * 4 + e) * N + n;
          if (f32dst) f32dst[o] = acc[i][j][e];
          else bf16dst[o] = static_cast<__bf16>(acc[i][j][e]);
        }
      }
    }
  };

  T dtv = load_dt(0);
  // issued in the order the loop reissues them (slot 0 first), so that the waits the compiler
  // derives for the loop hold for the first chunk too and do not drain the ring
#pragma unroll
  for (int k = 0; k < TPC; ++k) {
    load_tile(xr[k], br[k], okm[k], k * KT);
    __builtin_amdgcn_sched_barrier(0);
  }

  for (int c = 0; c < nc; ++c) {
    // chunk prologue: dt' of this chunk into LDS, the next chunk's dt on its way
    {
      const int len = min(Q, L - c * Q);
      float d = softplus(to_f32(dtv) + bias);
      if (clamp) d = fminf(fmaxf(d, lo), hi);
      if (tid < Q) s_d[dpos] = dpos < len ? d : 0.f;
    }
    dtv = load_dt(c + 1 < nc ? c + 1 : c);
    __syncthreads();                     // s_d complete; the previous tile's MFMAs are done
    if (wave == 0) {
      // inclusive cumsum of dt' A (as chunk_cumsum_wave), weights and the total decay exponent
      float d[EPL], cs[EPL];
      float run = 0.f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        d[k] = s_d[lane * EPL + k];
        run += d[k] * av;
        cs[k] = run;
      }
      const float excl = wave_shr1(wave_incl_scan(run));
#pragma unroll
      for (int k = 0; k < EPL; ++k) cs[k] += excl;
      // the stored dAcs[Q - 1]
      const float last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cs[EPL - 1]), 63));
#pragma unroll
      for (int k = 0; k < EPL; ++k) s_w[lane * EPL + k] = expf(last - cs[k]) * d[k];
      if (lane == 0) s_last = last;
      if (sl == 0) {
        float* dtp_c = dtp + (bh * nc + c) * Q + lane * EPL;
        float* dA_c = dAcs + (bh * nc + c) * Q + lane * EPL;
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
          dtp_c[k] = d[k];
          dA_c[k] = cs[k];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < TPC; ++k) {
      __syncthreads();                   // previous tile consumed; s_w and s_last written
      if (k == 0) {
        // H_c leaves for the scan, then the decay over chunk c
        const size_t o = (((size_t)b * nc + c) * H + h) * PN;
        if (F32) write_state(states + o, nullptr);
        else write_state(nullptr, prev16 + o);
        const float dec = expf(s_last);
#pragma unroll
        for (int i = 0; i < WP; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] *= dec;
      }
      store_tile(xr[k], br[k], okm[k], k * KT);
      load_tile(xr[k], br[k], okm[k], (c + 1) * Q + k * KT);   // the same tile of the next chunk
      __syncthreads();
      if (F32) {
#pragma unroll
        for (int m = 0; m < KT / 16; ++m) {
          float4 af[WP], bf[WN];
#pragma unroll
          for (int i = 0; i < WP; ++i) {
            const int tp = wp * WP + i;
            const int tpc = tp < TP ? tp : TP - 1;
            const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(s_x) +
                                                              (tpc * 16 + r) * PITCH + (KT / 4) * qd + 4 * m);
            af[i] = (tp < TP) ? v : make_float4(0.f, 0.f, 0.f, 0.f);
          }
#pragma unroll
          for (int j = 0; j < WN; ++j)
            bf[j] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(s_b) +
                                                     ((wn * WN + j) * 16 + r) * PITCH + (KT / 4) * qd + 4 * m);
#pragma unroll
          for (int i = 0; i < WP; ++i)
#pragma unroll
            for (int j = 0; j < WN; ++j) {
              acc[i][j] = mfma_16x16x4_f32(af[i].x, bf[j].x, acc[i][j]);
              acc[i][j] = mfma_16x16x4_f32(af[i].y, bf[j].y, acc[i][j]);
              acc[i][j] = mfma_16x16x4_f32(af[i].z, bf[j].z, acc[i][j]);
              acc[i][j] = mfma_16x16x4_f32(af[i].w, bf[j].w, acc[i][j]);
            }
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < KT / 32; ++kk) {
          bf16x8 af[WP], bf[WN];
#pragma unroll
          for (int i = 0; i < WP; ++i) {
            const int tp = wp * WP + i;
            const int tpc = tp < TP ? tp : TP - 1;
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(s_x) +
                                                              (tpc * 16 + r) * PITCH + 32 * kk + 8 * qd);
            af[i] = (tp < TP) ? v : KMma<__bf16>::zero();
          }
#pragma unroll
          for (int j = 0; j < WN; ++j)
            bf[j] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(s_b) +
                                                     ((wn * WN + j) * 16 + r) * PITCH + 32 * kk + 8 * qd);
#pragma unroll
          for (int i = 0; i < WP; ++i)
#pragma unroll
            for (int j = 0; j < WN; ++j) acc[i][j] = mfma_16x16x32_bf16(af[i], bf[j], acc[i][j]);
        }
      }
    }
  }
  if (final_state) write_state(final_state + bh * PN, nullptr);
}

template <typename T, int P, int N, int PS>
static hipError_t launch_state_seq_impl(const FwdArgs& a, hipStream_t s) {
  constexpr int NTHR = (PS / 16) * (N / 16) >= 32 ? 512 : 256;
  const uint32_t nseq = (uint32_t)a.B * a.H * (P / PS);
  const int nrb = a.Q / kCbKT;
  const uint32_t ncb = a.cb ? (uint32_t)a.B * a.nc * a.G * (nrb * (nrb + 1) / 2) : 0u;
  const uint32_t ncb_wg = ((ncb + NTHR / 256 - 1) / (NTHR / 256) + 7) / 8 * 8;
  if (nseq == 0 || a.nc == 0) return hipErrorInvalidValue;
#define SSD_SEQ_LAUNCH(TPC_)                                                                                    \
  hipExtLaunchKernelGGL(chunk_state_seq_kernel<T, P, N, PS, NTHR, TPC_>, dim3(nseq + ncb_wg), dim3(NTHR), 0, s,  \
                        a.ev0, a.ev1, 0, static_cast<const T*>(a.x), static_cast<const T*>(a.Bm),               \
                        static_cast<const T*>(a.Cm), static_cast<const T*>(a.dt), a.dt_bias, a.A, a.dtp, a.dAcs,  \
                        a.states, static_cast<__bf16*>(a.prev16), a.init, a.final_state, a.cb, a.L, a.H, a.G,   \
                        a.nc, nseq, ncb, ncb_wg, a.clamp, a.dt_lo, a.dt_hi)
  if (a.Q == 256)
    SSD_SEQ_LAUNCH(4);
  else if (a.Q == 128)
    SSD_SEQ_LAUNCH(2);
  else
    return hipErrorInvalidValue;
#undef SSD_SEQ_LAUNCH
  return hipGetLastError();
}

template <typename T, int P, int N>
static hipError_t launch_state_impl(const FwdArgs& a, hipStream_t s) {
  const uint32_t nblocks = (uint32_t)a.B * a.nc * a.H;
  const int nrb = a.Q / kCbKT;
  const uint32_t ncb = (a.cb && !a.state_from_start)
                           ? (uint32_t)a.B * a.nc * a.G * (nrb * (nrb + 1) / 2) : 0u;
  if (nblocks + ncb == 0) return hipSuccess;
  constexpr int NTHR = 512;
  const uint32_t ncb_all = a.cbT && ncb ? 2 * ncb : ncb;
  const uint32_t ncb_wg = ((ncb_all + NTHR / 256 - 1) / (NTHR / 256) + 7) / 8 * 8;
  hipExtLaunchKernelGGL(chunk_state_kernel<T, P, N, NTHR>, dim3(nblocks + ncb_wg), dim3(NTHR), 0, s, a.ev0, a.ev1,
      0, static_cast<const T*>(a.x), static_cast<const T*>(a.Bm), static_cast<const T*>(a.Cm),
      static_cast<const T*>(a.dt), a.dt_bias, a.A, a.dtp, a.dAcs, a.states, a.cb, a.cbT, a.L, a.H, a.G, a.nc, a.Q,
      nblocks, ncb, ncb_wg, a.state_from_start, a.clamp, a.dt_lo, a.dt_hi);
  return hipGetLastError();
}

hipError_t launch_chunk_state(const FwdArgs& a, hipStream_t s) {
#define SSD_CASE(T, P_, N_) \
  if (a.dtype == SSD_DTYPE_CODE_##T && a.P == P_ && a.N == N_) return launch_state_impl<T, P_, N_>(a, s);
  SSD_FOR_EACH_SHAPE(SSD_CASE)
#undef SSD_CASE
  return hipErrorInvalidValue;
}

bool chunk_state_seq_supported(const FwdArgs& a, int ps) {
  if (a.Q != 256 && a.Q != 128) return false;
#define SSD_SEQ_CASE(T, P_, N_, PS_) \
  if (a.dtype == SSD_DTYPE_CODE_##T && a.P == P_ && a.N == N_ && ps == PS_) return true;
  SSD_FOR_EACH_SEQ_SHAPE(SSD_SEQ_CASE)
#undef SSD_SEQ_CASE
  return false;
}

hipError_t launch_chunk_state_seq(const FwdArgs& a, int ps, hipStream_t s) {
#define SSD_SEQ_CASE(T, P_, N_, PS_) \
  if (a.dtype == SSD_DTYPE_CODE_##T && a.P == P_ && a.N == N_ && ps == PS_) \
    return launch_state_seq_impl<T, P_, N_, PS_>(a, s);
  SSD_FOR_EACH_SEQ_SHAPE(SSD_SEQ_CASE)
#undef SSD_SEQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
