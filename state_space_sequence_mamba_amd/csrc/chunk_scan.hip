// chunk_scan: the output of every position of a chunk,
//   y[i,p] = sum_{j<=i} CB[i,j] exp(dAcs[i] - dAcs[j]) dt'_j x[j,p]        (diagonal block)
//          + exp(dAcs[i]) sum_n C[i,n] Hprev[p,n]                            (carried state)
//          + D[p] x[i,p]                                                     (skip term)
// with CB[i,j] = sum_n C[i,n] B[j,n] and Hprev the state entering the chunk.
// Sources: "Agent 228: MAMBA-2 Reference Implementations Comparison", section 2.2 (the SSD
// output as a 1-semiseparable causal mask applied to attention-like C B^T scores) and
// section 3.2 (chunked evaluation: diagonal blocks plus the inter-chunk carry); "Agent 228:
// MAMBA-2 Implementation Gaps", Gap 1 (off-diagonal block from the previous state) and
// Gap 4 (D skip).
//
// Work decomposition.  A workgroup owns one 64-row block of a chunk (4 wavefronts, one
// 16-row strip each) for HB heads of one group.  Row blocks lower in the chunk have more
// causal column tiles; they are dispatched first (longest work first) and every XCD gets an
// equal share of each row-block class, with consecutive (batch, chunk) pairs on one XCD so
// that they share its L2 for B and C.
//
// Per strip, per 16-column causal sub-tile: CB^T (16x16) is contracted on MFMA once and
// consumed at once by all HB heads: each head applies its decay exp(dAcs_i - dAcs_j) dt'_j
// and the causal mask in registers (CB^T, not CB, so that the MFMA result layout -- four
// consecutive columns of one row per lane -- is directly the A operand of the (L o CB) X
// product), then accumulates into its own (16 x P) output tile.
// Contractions over dstate use the k-permutation n = 16*qd + kk (fp32) so that every lane
// reads its operand with 128-bit LDS loads; only consistency between the A and B operands
// matters for a sum over k.
//
// MFMA use: fp32 inputs -> v_mfma_f32_16x16x4_f32 for all three products;
// bf16 inputs -> 16x16x32 bf16 for C B^T and C Hprev^T, 16x16x16 bf16 for (L o CB) X.
// Decay factors use the hardware base-2 exponential on log2(e)-scaled cumsums; factors
// below 2^-126 become 0.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kKT = 64;                       // tokens per staged tile == rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;

template <int P> struct TPof { static constexpr int v = P / 16; };

template <typename T, int P, int N, int HB>
struct ScanLds {
  static constexpr bool F32 = sizeof(T) == 4;
  static constexpr int BP = N + (F32 ? 4 : 8);   // B tile / Hprev rows (n-contiguous), 16-byte rows
  static constexpr int XP = kKT + 4;              // x^T rows (token-contiguous)
  static constexpr int B_ELEMS = kKT * BP;
  static constexpr int X_ELEMS = HB * P * XP;
  static constexpr int PREV_ELEMS = P * BP;
  static constexpr int XU_ELEMS = X_ELEMS > PREV_ELEMS ? X_ELEMS : PREV_ELEMS;  // x tiles alias Hprev
};

// Contraction over dstate of two n-contiguous rows: fp32 takes 16 k values per lane in 4 float4
// loads (n = 16*qd + kk), bf16 takes 8 per 16x16x32 instruction (n = 32*kk + 8*qd + e).
template <typename T, int N> struct NDot;
template <int N> struct NDot<float, N> {
  static constexpr int NF = N / 4;                // k values per lane
  typedef float frag[NF];
  __device__ static __forceinline__ void load(frag f, const float* row, int qd) {
    const float* p = row + (N / 4) * qd;
#pragma unroll
    for (int m = 0; m < NF / 4; ++m) {
      const float4 v = *reinterpret_cast<const float4*>(p + 4 * m);
      f[4 * m + 0] = v.x; f[4 * m + 1] = v.y; f[4 * m + 2] = v.z; f[4 * m + 3] = v.w;
    }
  }
  __device__ static __forceinline__ void zero(frag f) {
#pragma unroll
    for (int k = 0; k < NF; ++k) f[k] = 0.f;
  }
  __device__ static __forceinline__ f32x4 dot(const frag a, const frag b, f32x4 c) {
#pragma unroll
    for (int k = 0; k < NF; ++k) c = mfma_16x16x4_f32(a[k], b[k], c);
    return c;
  }
};
template <int N> struct NDot<__bf16, N> {
  static constexpr int NF = N / 32;               // 16x16x32 instructions
  typedef bf16x8 frag[NF];
  __device__ static __forceinline__ void load(frag f, const __bf16* row, int qd) {
#pragma unroll
    for (int k = 0; k < NF; ++k) f[k] = *reinterpret_cast<const bf16x8*>(row + 32 * k + 8 * qd);
  }
  __device__ static __forceinline__ void zero(frag f) {
#pragma unroll
    for (int k = 0; k < NF; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) f[k][e] = static_cast<__bf16>(0.f);
  }
  __device__ static __forceinline__ f32x4 dot(const frag a, const frag b, f32x4 c) {
#pragma unroll
    for (int k = 0; k < NF; ++k) c = mfma_16x16x32_bf16(a[k], b[k], c);
    return c;
  }
};

// ---------------------------------------------------------------- shared pieces
// Stage the (P x N) fp32 state entering the chunk into LDS as T, n-contiguous rows.
template <typename T, int P, int N, int HB>
__device__ __forceinline__ void stage_prev(T* s_prev, const float* hp, int tid, int nthr) {
  typedef ScanLds<T, P, N, HB> SL;
  for (int v = tid; v < P * N / 4; v += nthr) {
    const int p = (v * 4) / N, n = (v * 4) % N;
    const float4 f = *reinterpret_cast<const float4*>(hp + (size_t)p * N + n);
    T* dst = &s_prev[p * SL::BP + n];
    if (SL::F32) {
      *reinterpret_cast<float4*>(dst) = f;
    } else {
      dst[0] = from_f32<T>(f.x);
      dst[1] = from_f32<T>(f.y);
      dst[2] = from_f32<T>(f.z);
      dst[3] = from_f32<T>(f.w);
    }
  }
}

// Stage token tile J: B rows (n-contiguous) and x^T for every head of the block
// (token-contiguous; each thread writes one packed pair of consecutive tokens).
template <typename T, int P, int N, int HB>
__device__ __forceinline__ void stage_tile(T* s_b, T* s_x, const T* Bb, const T* xb, size_t bc_tok, size_t x_tok,
                                           int J, int len, int tid, int nthr) {
  typedef ScanLds<T, P, N, HB> SL;
  constexpr int VEC = Vec16<T>::n;
  for (int v = tid; v < kKT * (N / VEC); v += nthr) {
    const int i = v / (N / VEC), nv = (v % (N / VEC)) * VEC;
    const int tok = J * kKT + i;
    const Vec16<T> d = (tok < len) ? load16(Bb + (size_t)tok * bc_tok + nv) : zero16<T>();
    *reinterpret_cast<Vec16<T>*>(&s_b[i * SL::BP + nv]) = d;
  }
  constexpr int PV = P / VEC;
  for (int v = tid; v < HB * (kKT / 2) * PV; v += nthr) {
    const int m = v % (kKT / 2);
    const int rest = v / (kKT / 2);
    const int pv = (rest % PV) * VEC, hh = rest / PV;
    const int tok = J * kKT + 2 * m;
    const T* src = xb + (size_t)tok * x_tok + (size_t)hh * P + pv;
    const Vec16<T> d0 = (tok < len) ? load16(src) : zero16<T>();
    const Vec16<T> d1 = (tok + 1 < len) ? load16(src + x_tok) : zero16<T>();
    T* dst = &s_x[(hh * P + pv) * SL::XP + 2 * m];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      T pair[2] = {d0.v[e], d1.v[e]};
      __builtin_memcpy(dst + e * SL::XP, pair, sizeof(pair));
    }
  }
}

// acc_h += exp(dAcs_i) * C_strip . Hprev^T  (Hprev of head hh staged in s_prev)
template <typename T, int P, int N, int HB>
__device__ __forceinline__ void carried_term(f32x4 (&acc)[TPof<P>::v], const typename NDot<T, N>::frag& cf,
                                             const T* s_prev, const float* s_da_h, int strip, int r, int qd) {
  typedef ScanLds<T, P, N, HB> SL;
  typedef NDot<T, N> ND;
  constexpr int TP = P / 16;
  f32x4 t[TP];
#pragma unroll
  for (int pt = 0; pt < TP; ++pt) {
    typename ND::frag pf;
    ND::load(pf, &s_prev[(pt * 16 + r) * SL::BP], qd);
    t[pt] = ND::dot(cf, pf, zero4());
  }
  float sc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sc[e] = __builtin_amdgcn_exp2f(s_da_h[16 * strip + 4 * qd + e]);
#pragma unroll
  for (int pt = 0; pt < TP; ++pt)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[pt][e] += t[pt][e] * sc[e];
}

// Diagonal-block contributions of staged tile J to one strip, for every head of the block.
template <typename T, int P, int N, int HB>
__device__ __forceinline__ void diag_tile(f32x4 (&acc)[HB][TPof<P>::v], const typename NDot<T, N>::frag& cf,
                                          const T* s_b, const T* s_x, const float (*s_da)[256],
                                          const float (*s_dt)[256], int strip, int J, int r, int qd) {
  typedef ScanLds<T, P, N, HB> SL;
  typedef NDot<T, N> ND;
  constexpr int TP = P / 16;
  const int i_row = 16 * strip + r;
#pragma unroll
  for (int js = 0; js < 4; ++js) {
    const int jt = 4 * J + js;
    if (jt > strip) break;                               // causal: sub-tiles past the diagonal
    // CB^T sub-tile: lane holds CB[i = 16 strip + r][j = 16 jt + 4 qd + e]
    typename ND::frag bfr;
    ND::load(bfr, &s_b[(js * 16 + r) * SL::BP], qd);
    const f32x4 cbt = ND::dot(bfr, cf, zero4());
    const int j0 = 16 * jt + 4 * qd;
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      const float da_i = s_da[hh][i_row];
      const float4 daj = *reinterpret_cast<const float4*>(&s_da[hh][j0]);
      const float4 dtj = *reinterpret_cast<const float4*>(&s_dt[hh][j0]);
      const float w0 = cbt[0] * __builtin_amdgcn_exp2f(da_i - daj.x) * dtj.x;
      const float w1 = cbt[1] * __builtin_amdgcn_exp2f(da_i - daj.y) * dtj.y;
      const float w2 = cbt[2] * __builtin_amdgcn_exp2f(da_i - daj.z) * dtj.z;
      const float w3 = cbt[3] * __builtin_amdgcn_exp2f(da_i - daj.w) * dtj.w;
      float lw[4];
      lw[0] = (j0 + 0 <= i_row) ? w0 : 0.f;
      lw[1] = (j0 + 1 <= i_row) ? w1 : 0.f;
      lw[2] = (j0 + 2 <= i_row) ? w2 : 0.f;
      lw[3] = (j0 + 3 <= i_row) ? w3 : 0.f;
      const T* xt = &s_x[(hh * P + r) * SL::XP + js * 16 + 4 * qd];
      if (SL::F32) {
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          const float4 xv =
              *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(xt) + pt * 16 * SL::XP);
          acc[hh][pt] = mfma_16x16x4_f32(lw[0], xv.x, acc[hh][pt]);
          acc[hh][pt] = mfma_16x16x4_f32(lw[1], xv.y, acc[hh][pt]);
          acc[hh][pt] = mfma_16x16x4_f32(lw[2], xv.z, acc[hh][pt]);
          acc[hh][pt] = mfma_16x16x4_f32(lw[3], xv.w, acc[hh][pt]);
        }
      } else {
        bf16x4 a;
        a[0] = static_cast<__bf16>(lw[0]);
        a[1] = static_cast<__bf16>(lw[1]);
        a[2] = static_cast<__bf16>(lw[2]);
        a[3] = static_cast<__bf16>(lw[3]);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          const bf16x4 xv =
              *reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(xt) + pt * 16 * SL::XP);
          acc[hh][pt] = mfma_16x16x16_bf16(a, xv, acc[hh][pt]);
        }
      }
    }
  }
}

// Skip term and store of one strip: lane holds rows 16 strip + 4 qd + e, column 16 pt + r.
template <typename T, int P, int HB>
__device__ __forceinline__ void store_strip(const f32x4 (&acc)[HB][TPof<P>::v], const T* x, const float* Dw, T* y,
                                            size_t row0, size_t x_tok, int h0, int strip, int len, int r, int qd) {
  constexpr int TP = P / 16;
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const int h = h0 + hh;
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) {
      const int p = pt * 16 + r;
      const float dw = Dw ? Dw[(size_t)h * P + p] : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * strip + 4 * qd + e;
        if (i < len) {
          const size_t o = (row0 + i) * x_tok + (size_t)h * P + p;
          y[o] = from_f32<T>(acc[hh][pt][e] + dw * to_f32(x[o]));
        }
      }
    }
  }
}

// ---------------------------------------------------------------- row-block decomposition
// One workgroup per (64-row block, HB heads): many small workgroups, for compute-bound
// (fp32) problems.  Rows of one chunk are spread over Q/64 workgroups, so x tiles and the
// carried state are read once per row block.
template <typename T, int P, int N, int HB>
__global__ __launch_bounds__(256, 2) void chunk_scan_rows_kernel(const T* __restrict__ x,
                                                                 const T* __restrict__ Bm,
                                                                 const T* __restrict__ Cm,
                                                                 const float* __restrict__ dtp,
                                                                 const float* __restrict__ dAcs,
                                                                 const float* __restrict__ states,
                                                                 const float* __restrict__ Dw,
                                                                 T* __restrict__ y,
                                                                 int L, int H, int G, int nc, int Q, int B) {
  typedef ScanLds<T, P, N, HB> SL;
  typedef NDot<T, N> ND;
  constexpr int TP = P / 16;

  __shared__ __attribute__((aligned(16))) T s_b[SL::B_ELEMS];
  __shared__ __attribute__((aligned(16))) T s_xu[SL::XU_ELEMS];   // Hprev, then x^T tiles
  __shared__ __attribute__((aligned(16))) float s_da[HB][256];     // dAcs * log2(e)
  __shared__ __attribute__((aligned(16))) float s_dt[HB][256];

  // work unit: row-block class (heaviest first), then XCD-local (b, c, head block)
  const int nrb = Q / kKT;
  const int nhb = H / HB;
  const uint32_t U = (uint32_t)B * nc * nhb;          // units per row-block class
  const uint32_t hw = blockIdx.x;
  uint32_t cls, unit;
  if ((U & 7u) == 0) {
    const uint32_t per = U >> 3, seq = hw >> 3;
    cls = seq / per;
    unit = (hw & 7u) * per + seq % per;
  } else {
    cls = hw / U;
    unit = hw % U;
  }
  const int rb = nrb - 1 - (int)cls;
  const int hblk = unit % nhb;
  const int bc = unit / nhb;
  const int c = bc % nc, b = bc / nc;
  const int h0 = hblk * HB;
  const int g = h0 / (H / G);
  const int t0 = c * Q;
  const int len = min(Q, L - t0);
  if (rb * kKT >= len) return;                         // whole row block is padding

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;
  const int s = rb * 4 + wave;                          // this wavefront's strip
  const bool strip_ok = 16 * s < len;

  for (int idx = tid; idx < HB * Q; idx += 256) {
    const int hh = idx / Q, i = idx % Q;
    const size_t off = (((size_t)b * H + h0 + hh) * nc + c) * Q + i;
    s_dt[hh][i] = dtp[off];
    s_da[hh][i] = dAcs[off] * kLog2e;
  }
  const size_t bc_tok = (size_t)G * N, x_tok = (size_t)H * P;
  const T* Cb = Cm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  const T* Bb = Bm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  typename ND::frag cf;
  if (16 * s + r < len) ND::load(cf, Cb + (size_t)(16 * s + r) * bc_tok, qd);
  else ND::zero(cf);

  f32x4 acc[HB][TP];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) acc[hh][pt] = zero4();

#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    __syncthreads();
    stage_prev<T, P, N, HB>(s_xu, states + (((size_t)b * nc + c) * H + h0 + hh) * (size_t)(P * N), tid, 256);
    __syncthreads();
    if (strip_ok) carried_term<T, P, N, HB>(acc[hh], cf, s_xu, s_da[hh], s, r, qd);
  }
  const T* xb = x + ((size_t)b * L + t0) * x_tok + (size_t)h0 * P;
  for (int J = 0; J <= rb; ++J) {
    __syncthreads();
    stage_tile<T, P, N, HB>(s_b, s_xu, Bb, xb, bc_tok, x_tok, J, len, tid, 256);
    __syncthreads();
    if (strip_ok) diag_tile<T, P, N, HB>(acc, cf, s_b, s_xu, s_da, s_dt, s, J, r, qd);
  }
  if (strip_ok) store_strip<T, P, HB>(acc, x, Dw, y, (size_t)b * L + t0, x_tok, h0, s, len, r, qd);
}

// ---------------------------------------------------------------- whole-chunk decomposition
// One workgroup per (chunk, HB heads) with Q/32 wavefronts; wavefront w owns the strip pair
// (w, S-1-w), so every wavefront has S+1 causal sub-tiles.  x, the carried state and y move
// exactly once, for memory-bound (bf16) problems.
template <typename T, int P, int N, int HB>
__global__ __launch_bounds__(512) void chunk_scan_chunk_kernel(const T* __restrict__ x,
                                                               const T* __restrict__ Bm,
                                                               const T* __restrict__ Cm,
                                                               const float* __restrict__ dtp,
                                                               const float* __restrict__ dAcs,
                                                               const float* __restrict__ states,
                                                               const float* __restrict__ Dw,
                                                               T* __restrict__ y,
                                                               int L, int H, int G, int nc, int Q, uint32_t nblocks) {
  typedef ScanLds<T, P, N, HB> SL;
  typedef NDot<T, N> ND;
  constexpr int TP = P / 16;

  __shared__ __attribute__((aligned(16))) T s_b[SL::B_ELEMS];
  __shared__ __attribute__((aligned(16))) T s_xu[SL::XU_ELEMS];
  __shared__ __attribute__((aligned(16))) float s_da[HB][256];
  __shared__ __attribute__((aligned(16))) float s_dt[HB][256];

  uint32_t id = xcd_swizzle(blockIdx.x, nblocks);
  const int nhb = H / HB;
  const int hblk = id % nhb;
  id /= nhb;
  const int c = id % nc, b = id / nc;
  const int h0 = hblk * HB;
  const int g = h0 / (H / G);
  const int t0 = c * Q;
  const int len = min(Q, L - t0);
  const int S = Q >> 4;
  const int nthr = blockDim.x;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;
  int strip[2];
  strip[0] = wave;                                      // short strip
  strip[1] = S - 1 - wave;                              // long strip

  for (int idx = tid; idx < HB * Q; idx += nthr) {
    const int hh = idx / Q, i = idx % Q;
    const size_t off = (((size_t)b * H + h0 + hh) * nc + c) * Q + i;
    s_dt[hh][i] = dtp[off];
    s_da[hh][i] = dAcs[off] * kLog2e;
  }
  const size_t bc_tok = (size_t)G * N, x_tok = (size_t)H * P;
  const T* Cb = Cm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  const T* Bb = Bm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  typename ND::frag cf[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    if (16 * strip[st] + r < len) ND::load(cf[st], Cb + (size_t)(16 * strip[st] + r) * bc_tok, qd);
    else ND::zero(cf[st]);
  }

  f32x4 acc[2][HB][TP];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int hh = 0; hh < HB; ++hh)
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) acc[st][hh][pt] = zero4();

#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    __syncthreads();
    stage_prev<T, P, N, HB>(s_xu, states + (((size_t)b * nc + c) * H + h0 + hh) * (size_t)(P * N), tid, nthr);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 2; ++st)
      if (16 * strip[st] < len) carried_term<T, P, N, HB>(acc[st][hh], cf[st], s_xu, s_da[hh], strip[st], r, qd);
  }
  const T* xb = x + ((size_t)b * L + t0) * x_tok + (size_t)h0 * P;
  const int ntiles = (len + kKT - 1) / kKT;
  for (int J = 0; J < ntiles; ++J) {
    __syncthreads();
    stage_tile<T, P, N, HB>(s_b, s_xu, Bb, xb, bc_tok, x_tok, J, len, tid, nthr);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 2; ++st)
      if (16 * strip[st] < len && 4 * J <= strip[st])
        diag_tile<T, P, N, HB>(acc[st], cf[st], s_b, s_xu, s_da, s_dt, strip[st], J, r, qd);
  }
#pragma unroll
  for (int st = 0; st < 2; ++st)
    if (16 * strip[st] < len)
      store_strip<T, P, HB>(acc[st], x, Dw, y, (size_t)b * L + t0, x_tok, h0, strip[st], len, r, qd);
}

template <typename T, int P, int N, int HB>
static hipError_t launch_scan_hb(const FwdArgs& a, hipStream_t s) {
  if (a.scan_variant == 2) {
    const uint32_t nblocks = (uint32_t)a.B * a.nc * (a.H / HB);
    chunk_scan_chunk_kernel<T, P, N, HB><<<nblocks, 64 * (a.Q / 32), 0, s>>>(
        static_cast<const T*>(a.x), static_cast<const T*>(a.Bm), static_cast<const T*>(a.Cm), a.dtp, a.dAcs,
        a.states, a.D, static_cast<T*>(a.y), a.L, a.H, a.G, a.nc, a.Q, nblocks);
  } else {
    const uint32_t nblocks = (uint32_t)a.B * a.nc * (a.H / HB) * (a.Q / kKT);
    chunk_scan_rows_kernel<T, P, N, HB><<<nblocks, 256, 0, s>>>(
        static_cast<const T*>(a.x), static_cast<const T*>(a.Bm), static_cast<const T*>(a.Cm), a.dtp, a.dAcs,
        a.states, a.D, static_cast<T*>(a.y), a.L, a.H, a.G, a.nc, a.Q, a.B);
  }
  return hipGetLastError();
}

template <typename T, int P, int N>
static hipError_t launch_scan_impl(const FwdArgs& a, hipStream_t s) {
  switch (a.heads_per_block) {
    case 4: return launch_scan_hb<T, P, N, 4>(a, s);
    case 3: return launch_scan_hb<T, P, N, 3>(a, s);
    case 2: return launch_scan_hb<T, P, N, 2>(a, s);
    default: return launch_scan_hb<T, P, N, 1>(a, s);
  }
}

hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t s) {
#define SSD_CASE(T, P_, N_) \
  if (a.dtype == SSD_DTYPE_CODE_##T && a.P == P_ && a.N == N_) return launch_scan_impl<T, P_, N_>(a, s);
  SSD_FOR_EACH_SHAPE(SSD_CASE)
#undef SSD_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
