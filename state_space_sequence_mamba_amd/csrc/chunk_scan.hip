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
// Work decomposition.  A chunk's Q rows form S = Q/16 strips of 16 rows.  Strip s needs
// s+1 causal 16x16 column sub-tiles, so strips are paired (k, S-1-k): every pair costs S+1
// sub-tiles and each wavefront owns one pair.  A workgroup holds 4 wavefronts (4 pairs,
// i.e. half of a 256-token chunk) and `hb` heads of one group.  CB does not depend on the
// head, so each wavefront evaluates its CB sub-tiles once on MFMA, keeps them in registers
// (fp32) and reuses them for all hb heads; only the head-dependent decay and dt' mask is
// applied per head, in registers, before the result feeds the second MFMA as its A operand.
// CB^T (not CB) is computed so that the MFMA result lane layout (4 consecutive columns of
// one row per lane) is directly the A-operand layout of the (L o CB) X product: no data
// movement between the two products.
//
// MFMA use: fp32 inputs -> v_mfma_f32_16x16x4_f32 for all three products;
// bf16 inputs -> 16x16x32 bf16 for C B^T and C Hprev^T, 16x16x16 bf16 for (L o CB) X.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kScanKT = 64;    // tokens per staged LDS tile
constexpr int kMaxSlots = 17;  // S + 1 sub-tiles per strip pair, S <= 16 (Q <= 256)

template <typename T, int P, int N>
struct ScanSmem {
  static constexpr bool F32 = sizeof(T) == 4;
  static constexpr int BPITCH = N + (F32 ? 2 : 8);        // B tile rows / Hprev rows, n-contiguous
  static constexpr int XPITCH_F32 = P + 4;                // fp32 x tile [token][p]
  static constexpr int XPITCH_BF16 = kScanKT + 4;         // bf16 x tile transposed [p][token]
  static constexpr int B_ELEMS = kScanKT * BPITCH;
  static constexpr int X_ELEMS = F32 ? kScanKT * XPITCH_F32 : P * XPITCH_BF16;
  static constexpr int U_ELEMS = B_ELEMS > X_ELEMS ? B_ELEMS : X_ELEMS;
  static constexpr int PREV_ELEMS = P * BPITCH;
};

template <typename T, int P, int N>
__global__ __launch_bounds__(256) void chunk_scan_kernel(const T* __restrict__ x,
                                                         const T* __restrict__ Bm,
                                                         const T* __restrict__ Cm,
                                                         const float* __restrict__ dtp,
                                                         const float* __restrict__ dAcs,
                                                         const float* __restrict__ states,
                                                         const float* __restrict__ Dw,
                                                         T* __restrict__ y,
                                                         int L, int H, int G, int nc, int Q, int hb,
                                                         int npg, uint32_t nblocks) {
  typedef KMma<T> M;
  typedef ScanSmem<T, P, N> SM;
  constexpr bool F32 = SM::F32;
  constexpr int NK = N / M::K;
  constexpr int TP = P / 16;
  constexpr int VEC = Vec16<T>::n;
  const int W = blockDim.x >> 6;                         // wavefronts per workgroup

  __shared__ __attribute__((aligned(16))) T s_u[SM::U_ELEMS];       // B tile, later x tile
  __shared__ __attribute__((aligned(16))) T s_prev[SM::PREV_ELEMS]; // Hprev (P x N) as T
  __shared__ __attribute__((aligned(16))) float s_dt[256];
  __shared__ __attribute__((aligned(16))) float s_da[256];

  // ---- which (b, c, head block, pair group)
  uint32_t id = xcd_swizzle(blockIdx.x, nblocks);
  const int pg = id % npg;
  id /= npg;
  const int nhb = (H / G) * G / hb;                      // head blocks = H / hb
  const int hblk = id % nhb;
  id /= nhb;
  const int c = id % nc;
  const int b = id / nc;
  const int h0 = hblk * hb;
  const int g = h0 / (H / G);
  const int t0 = c * Q;
  const int len = min(Q, L - t0);
  const int S = Q >> 4;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;
  const int k = pg * W + wave;                           // strip pair
  const int s_lo = k, s_hi = S - 1 - k;
  const bool lo_ok = 16 * s_lo < len, hi_ok = 16 * s_hi < len;
  // highest column tile any wavefront of this workgroup needs
  const int max_strip = S - 1 - pg * W;
  const int ntiles = min((16 * (max_strip + 1) + kScanKT - 1) / kScanKT, (len + kScanKT - 1) / kScanKT);

  const size_t bc_tok = (size_t)G * N;
  const T* Bb = Bm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  const T* Cb = Cm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;

  // ---- C fragments of both strips (A operand of C Hprev^T, B operand of B C^T)
  typename M::frag c_lo[NK], c_hi[NK];
  {
    const int i_lo = 16 * s_lo + r, i_hi = 16 * s_hi + r;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int n = kk * M::K + qd * M::KPL;
      c_lo[kk] = (i_lo < len) ? M::load(Cb + (size_t)i_lo * bc_tok + n) : M::zero();
      c_hi[kk] = (i_hi < len) ? M::load(Cb + (size_t)i_hi * bc_tok + n) : M::zero();
    }
  }

  // ---- phase A: CB^T sub-tiles of both strips, kept in registers
  // slot t <= k: strip s_lo, column tile t;  slot t > k: strip s_hi, column tile t-k-1
  f32x4 cb[kMaxSlots];
#pragma unroll
  for (int t = 0; t < kMaxSlots; ++t) cb[t] = zero4();

  T* s_b = s_u;
  for (int J = 0; J < ntiles; ++J) {
    __syncthreads();
    for (int v = tid; v < kScanKT * (N / VEC); v += blockDim.x) {
      const int i = v / (N / VEC), nv = (v % (N / VEC)) * VEC;
      const int tok = J * kScanKT + i;
      Vec16<T> d = (tok < len) ? load16(Bb + (size_t)tok * bc_tok + nv) : zero16<T>();
      if (F32) {  // fp32 rows are padded by 2 floats (conflict-free fragment reads): not 16-byte aligned
#pragma unroll
        for (int e = 0; e < VEC; ++e) s_b[i * SM::BPITCH + nv + e] = d.v[e];
      } else {
        *reinterpret_cast<Vec16<T>*>(&s_b[i * SM::BPITCH + nv]) = d;
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kMaxSlots; ++t) {
      if (t > S) continue;
      const bool lo = t <= k;
      const int jt = lo ? t : t - k - 1;
      if (!(lo ? lo_ok : hi_ok) || (jt >> 2) != J) continue;
      const T* brow = &s_b[((jt & 3) * 16 + r) * SM::BPITCH + qd * M::KPL];
      if (lo) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) cb[t] = M::mma(M::load(brow + kk * M::K), c_lo[kk], cb[t]);
      } else {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) cb[t] = M::mma(M::load(brow + kk * M::K), c_hi[kk], cb[t]);
      }
    }
  }

  // ---- phase B: per head
  for (int hh = 0; hh < hb; ++hh) {
    const int h = h0 + hh;
    __syncthreads();  // previous users of s_u / s_prev / s_dt / s_da are done
    {
      const size_t off = (((size_t)b * H + h) * nc + c) * Q;
      for (int i = tid; i < Q; i += blockDim.x) {
        s_dt[i] = dtp[off + i];
        s_da[i] = dAcs[off + i];
      }
      const float* hp = states + (((size_t)b * nc + c) * H + h) * (size_t)(P * N);
      for (int v = tid; v < P * N / 4; v += blockDim.x) {
        const int p = (v * 4) / N, n = (v * 4) % N;
        const float4 f = *reinterpret_cast<const float4*>(hp + (size_t)p * N + n);
        T* dst = &s_prev[p * SM::BPITCH + n];
        dst[0] = from_f32<T>(f.x);
        dst[1] = from_f32<T>(f.y);
        dst[2] = from_f32<T>(f.z);
        dst[3] = from_f32<T>(f.w);
      }
    }
    __syncthreads();

    // carried state: exp(dAcs[i]) * C_i . Hprev^T
    f32x4 acc_lo[TP], acc_hi[TP];
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) {
      acc_lo[pt] = zero4();
      acc_hi[pt] = zero4();
      const T* prow = &s_prev[(pt * 16 + r) * SM::BPITCH + qd * M::KPL];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const typename M::frag pf = M::load(prow + kk * M::K);
        acc_lo[pt] = M::mma(c_lo[kk], pf, acc_lo[pt]);
        acc_hi[pt] = M::mma(c_hi[kk], pf, acc_hi[pt]);
      }
    }
    {
      float sc_lo[4], sc_hi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc_lo[e] = expf(s_da[16 * s_lo + 4 * qd + e]);
        sc_hi[e] = expf(s_da[16 * s_hi + 4 * qd + e]);
      }
#pragma unroll
      for (int pt = 0; pt < TP; ++pt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc_lo[pt][e] *= sc_lo[e];
          acc_hi[pt][e] *= sc_hi[e];
        }
    }

    // diagonal blocks: (L o CB) X, x staged per 64-token tile
    const T* xh = x + ((size_t)b * L + t0) * (size_t)H * P + (size_t)h * P;
    const float da_lo = s_da[16 * s_lo + r], da_hi = s_da[16 * s_hi + r];
    for (int J = 0; J < ntiles; ++J) {
      __syncthreads();
      for (int v = tid; v < kScanKT * (P / VEC); v += blockDim.x) {
        const int i = v / (P / VEC), pv = (v % (P / VEC)) * VEC;
        const int tok = J * kScanKT + i;
        Vec16<T> d = (tok < len) ? load16(xh + (size_t)tok * H * P + pv) : zero16<T>();
        if (F32) {
          *reinterpret_cast<Vec16<T>*>(&s_u[i * SM::XPITCH_F32 + pv]) = d;
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) s_u[(pv + e) * SM::XPITCH_BF16 + i] = d.v[e];
        }
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < kMaxSlots; ++t) {
        if (t > S) continue;
        const bool lo = t <= k;
        const int jt = lo ? t : t - k - 1;
        if (!(lo ? lo_ok : hi_ok) || (jt >> 2) != J) continue;
        const int strip = lo ? s_lo : s_hi;
        const int i_row = 16 * strip + r;
        const float da_i = lo ? da_lo : da_hi;
        const int j0 = 16 * jt + 4 * qd;
        const float4 daj = *reinterpret_cast<const float4*>(&s_da[j0]);
        const float4 dtj = *reinterpret_cast<const float4*>(&s_dt[j0]);
        float lw[4];
        lw[0] = (j0 + 0 <= i_row) ? cb[t][0] * expf(da_i - daj.x) * dtj.x : 0.f;
        lw[1] = (j0 + 1 <= i_row) ? cb[t][1] * expf(da_i - daj.y) * dtj.y : 0.f;
        lw[2] = (j0 + 2 <= i_row) ? cb[t][2] * expf(da_i - daj.z) * dtj.z : 0.f;
        lw[3] = (j0 + 3 <= i_row) ? cb[t][3] * expf(da_i - daj.w) * dtj.w : 0.f;
        const int jl = (jt & 3) * 16 + 4 * qd;   // token row inside the staged tile
        if (F32) {
          const float* xs = reinterpret_cast<const float*>(s_u);
          if (lo) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int pt = 0; pt < TP; ++pt)
                acc_lo[pt] = mfma_16x16x4_f32(lw[e], xs[(jl + e) * SM::XPITCH_F32 + pt * 16 + r], acc_lo[pt]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int pt = 0; pt < TP; ++pt)
                acc_hi[pt] = mfma_16x16x4_f32(lw[e], xs[(jl + e) * SM::XPITCH_F32 + pt * 16 + r], acc_hi[pt]);
          }
        } else {
          const __bf16* xs = reinterpret_cast<const __bf16*>(s_u);
          bf16x4 a;
          a[0] = static_cast<__bf16>(lw[0]);
          a[1] = static_cast<__bf16>(lw[1]);
          a[2] = static_cast<__bf16>(lw[2]);
          a[3] = static_cast<__bf16>(lw[3]);
          if (lo) {
#pragma unroll
            for (int pt = 0; pt < TP; ++pt)
              acc_lo[pt] = mfma_16x16x16_bf16(
                  a, *reinterpret_cast<const bf16x4*>(&xs[(pt * 16 + r) * SM::XPITCH_BF16 + jl]), acc_lo[pt]);
          } else {
#pragma unroll
            for (int pt = 0; pt < TP; ++pt)
              acc_hi[pt] = mfma_16x16x16_bf16(
                  a, *reinterpret_cast<const bf16x4*>(&xs[(pt * 16 + r) * SM::XPITCH_BF16 + jl]), acc_hi[pt]);
          }
        }
      }
    }

    // skip term and store
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int strip = half ? s_hi : s_lo;
      if (16 * strip >= len) continue;
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        const int p = pt * 16 + r;
        const float dw = Dw ? Dw[(size_t)h * P + p] : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * strip + 4 * qd + e;
          if (i < len) {
            const size_t o = ((size_t)b * L + t0 + i) * (size_t)H * P + (size_t)h * P + p;
            const float v = (half ? acc_hi[pt][e] : acc_lo[pt][e]) + dw * to_f32(x[o]);
            y[o] = from_f32<T>(v);
          }
        }
      }
    }
  }
}

template <typename T, int P, int N>
static hipError_t launch_scan_impl(const FwdArgs& a, hipStream_t s) {
  const int S = a.Q / 16;
  const int pairs = S / 2;
  const int W = pairs < 4 ? pairs : 4;
  const int npg = pairs / W;
  const int hb = a.heads_per_block;
  const uint32_t nblocks = (uint32_t)a.B * a.nc * (a.H / hb) * npg;
  chunk_scan_kernel<T, P, N><<<nblocks, 64 * W, 0, s>>>(
      static_cast<const T*>(a.x), static_cast<const T*>(a.Bm), static_cast<const T*>(a.Cm), a.dtp, a.dAcs,
      a.states, a.D, static_cast<T*>(a.y), a.L, a.H, a.G, a.nc, a.Q, hb, npg, nblocks);
  return hipGetLastError();
}

hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t s) {
#define SSD_CASE(T, P_, N_) \
  if (a.dtype == SSD_DTYPE_CODE_##T && a.P == P_ && a.N == N_) return launch_scan_impl<T, P_, N_>(a, s);
  SSD_FOR_EACH_SHAPE(SSD_CASE)
#undef SSD_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
