// chunk_state_seg: the chunk states and their recurrence over one segment of consecutive chunks,
// for a group's slice of heads (bf16 inputs, chunk 256, headdim 64, dstate 128).
//
// The state recurrence H_{c+1} = exp(dAcs_c[last]) H_c + S_c, with the chunk's own state
//     S_c[p, n] = sum_i x[cQ+i, p] w_i B[cQ+i, n],   w_i = exp(dAcs[last] - dAcs[i]) dt'_i
// ("Agent 228: MAMBA-2 Implementation Gaps", Gap 1; section 3.2 of "Agent 228: MAMBA-2 Reference
// Implementations Comparison"), is linear, so a chain of chunks splits into segments: each
// segment runs the recurrence from a zero state, and the state entering chunk c of segment s is
//     H_c = L_c + exp(D_c) H^in_s,
// with L_c the state this segment alone has carried into chunk c, D_c = sum of dAcs_{c'}[last]
// over the segment's chunks before c, and H^in_s the state entering the segment.  The segments'
// end states E_s and total exponents then combine with the same recurrence over segments
// (H^in_{s+1} = exp(sum of the segment's exponents) H^in_s + E_s, H^in_0 = initial state; the
// scan of block carries of the block-parallel scan, section 2 of "Agent 230: Comprehensive
// MAMBA-2 Implementation Comparison"), which state_passing runs; chunk_scan adds exp(D_c) H^in_s
// to L_c when it stages the entering state.
//
// One workgroup (8 wavefronts) per (batch, segment, group, slice of HS heads of the group).  Per
// chunk: dt' and the in-chunk cumsum of dt' A for every head of the slice (wavefront hh, as in
// chunk_state: a log-step shuffle scan over 64 lanes), written to the workspace for chunk_scan;
// B^T staged once in LDS (token-contiguous rows) for all the slice's heads, and each wavefront's
// sixteen dstate columns of it held in registers for the chunk.  Per head: the weighted x^T
// staged in LDS, L_c written (rounded to bf16) unless c opens the segment, the state scaled by the
// chunk's decay and the chunk's x^T diag(w) B added on 16x16x32 bf16 MFMA, the state of each head
// held in the accumulators of the whole segment.  The next chunk's B and dt and the next head's x
// are loaded into registers while the current ones are in use.  At the segment's end E_s goes out
// in fp32 with the segment's total exponent; D_c goes out for every chunk.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kSQ = 256;                       // chunk length
constexpr int kSThreads = 512;
constexpr int kSXP = kSQ + 8;                  // token-contiguous LDS rows (bf16)

// One token-pair unit of a (token x 16-byte vector) tile: the same 16-byte slice of two
// consecutive tokens; consecutive lanes take consecutive token pairs, so the transposed LDS
// stores (one packed pair of bf16 per row) of a wavefront hit consecutive banks.
template <int VECS>                               // 16-byte vectors per token row
struct PairTile {
  static constexpr int U = (kSQ / 2) * VECS;      // units
  static constexpr int UPT = U / kSThreads;
  static_assert(U % kSThreads == 0, "shape");
  uint4 v[UPT][2];
  uint32_t okm;

  // rows of `stride` elements from `base` (wavefront-uniform), tokens past `len` read row 0
  __device__ __forceinline__ void load(const __bf16* base, uint32_t stride, int len, int tid) {
    okm = 0;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int w = tid + kSThreads * u;
      const int m = w % (kSQ / 2), vec = (w / (kSQ / 2)) * 8;
      const int t = 2 * m;
      const bool ok0 = t < len, ok1 = t + 1 < len;
      uint32_t o0 = (uint32_t)(ok0 ? t : 0) * stride + vec, o1 = (uint32_t)(ok1 ? t + 1 : 0) * stride + vec;
      asm volatile("" : "+v"(o0), "+v"(o1));
      v[u][0] = *reinterpret_cast<const uint4*>(base + o0);
      v[u][1] = *reinterpret_cast<const uint4*>(base + o1);
      okm |= ((uint32_t)ok0 << (2 * u)) | ((uint32_t)ok1 << (2 * u + 1));
    }
  }
  // transposed into `dst` rows (element row vec + e, token column 2m), each value times the
  // token's weight when `wt` is given (weights of tokens past the end are 0, and so are they)
  __device__ __forceinline__ void store(__bf16* dst, const float* wt, int tid) const {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int w = tid + kSThreads * u;
      const int m = w % (kSQ / 2), vec = (w / (kSQ / 2)) * 8;
      uint4 a = v[u][0], b = v[u][1];
      if (!((okm >> (2 * u)) & 1u)) a = make_uint4(0, 0, 0, 0);
      if (!((okm >> (2 * u + 1)) & 1u)) b = make_uint4(0, 0, 0, 0);
      const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
      if (wt) {
        const float w0 = wt[2 * m], w1 = wt[2 * m + 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a0 = __builtin_bit_cast(float, av[q] << 16), a1 = __builtin_bit_cast(float, av[q] & 0xffff0000u);
          const float b0 = __builtin_bit_cast(float, bv[q] << 16), b1 = __builtin_bit_cast(float, bv[q] & 0xffff0000u);
          const __bf16 pa[2] = {static_cast<__bf16>(a0 * w0), static_cast<__bf16>(b0 * w1)};
          const __bf16 pb[2] = {static_cast<__bf16>(a1 * w0), static_cast<__bf16>(b1 * w1)};
          __builtin_memcpy(&dst[(vec + 2 * q) * kSXP + 2 * m], pa, 4);
          __builtin_memcpy(&dst[(vec + 2 * q + 1) * kSXP + 2 * m], pb, 4);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = (av[q] & 0xffffu) | (bv[q] << 16);
          const uint32_t hi = (av[q] >> 16) | (bv[q] & 0xffff0000u);
          *reinterpret_cast<uint32_t*>(&dst[(vec + 2 * q) * kSXP + 2 * m]) = lo;
          *reinterpret_cast<uint32_t*>(&dst[(vec + 2 * q + 1) * kSXP + 2 * m]) = hi;
        }
      }
    }
  }
};

}  // namespace

template <int HS>
__global__ __launch_bounds__(kSThreads, 1) void chunk_state_seg_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ Bm, const __bf16* __restrict__ dt,
    const float* __restrict__ dt_bias, const float* __restrict__ A, float* __restrict__ dtp,
    float* __restrict__ dAcs, __bf16* __restrict__ prev16, float* __restrict__ E, float* __restrict__ segdec,
    float* __restrict__ cdec, int L, int H, int G, int nc, int SL, int nseg, int clamp, float lo, float hi,
    uint32_t nblocks) {
  constexpr int P = 64, N = 128, Q = kSQ, TP = P / 16, KS = Q / 32;
  constexpr int EPL = Q / 64;                      // cumsum positions per lane

  __shared__ __attribute__((aligned(16))) __bf16 s_bt[N * kSXP];   // B^T of the chunk
  __shared__ __attribute__((aligned(16))) __bf16 s_xt[P * kSXP];   // (x w)^T of one head
  __shared__ __attribute__((aligned(16))) float s_w[HS][Q];         // token weights per head
  __shared__ float s_last[HS];

  uint32_t id = xcd_swizzle(blockIdx.x, nblocks);  // the slices of one (b, s, g) on one XCD share B
  const int hpg = H / G, nsl = hpg / HS;
  const int sl = id % nsl;
  id /= nsl;
  const int g = id % G;
  id /= G;
  const int seg = id % nseg, b = id / nseg;
  const int h0 = g * hpg + sl * HS;
  const int c0 = seg * SL, c1 = min(nc, c0 + SL);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wavefront's 16 dstate columns
  const int r = lane & 15, qd = lane >> 4;
  const uint32_t x_tok = (uint32_t)H * P, b_tok = (uint32_t)G * N;
  const size_t PN = (size_t)P * N;

  auto x_base = [&](int c, int hh) { return x + ((size_t)b * L + (size_t)c * Q) * x_tok + (size_t)(h0 + hh) * P; };
  auto b_base = [&](int c) { return Bm + ((size_t)b * L + (size_t)c * Q) * b_tok + (size_t)g * N; };
  // dt of the positions this lane scans (wavefront hh < HS: head h0 + hh), clamped in bounds
  auto load_dt = [&](int c, float (&dv)[EPL]) {
    const int hh = w < HS ? w : 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int t = min(c * Q + lane * EPL + k, L - 1);
      dv[k] = static_cast<float>(dt[((size_t)b * L + t) * H + h0 + hh]);
    }
  };

  f32x4 st[HS][TP];                                // the states, n column 16 w + r, rows 16 pt + 4 qd + e
#pragma unroll
  for (int hh = 0; hh < HS; ++hh)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) st[hh][pt] = zero4();
  float run = 0.f;                                 // wavefront hh: exponent sum since the segment start

  PairTile<N / 8> breg;
  PairTile<P / 8> xreg;
  float dtv[EPL];
  breg.load(b_base(c0), b_tok, min(Q, L - c0 * Q), tid);
  xreg.load(x_base(c0, 0), x_tok, min(Q, L - c0 * Q), tid);
  load_dt(c0, dtv);

  for (int c = c0; c < c1; ++c) {
    const int len = min(Q, L - c * Q);
    __syncthreads();                               // the previous chunk's weights and B^T consumed
    breg.store(s_bt, nullptr, tid);
    if (w < HS) {
      // dt' and the inclusive in-chunk cumsum of dt' A of head h0 + w; weights to the chunk end
      const int h = h0 + w;
      const float bias = dt_bias[h], av = A[h];
      float d[EPL], cs[EPL], run_l = 0.f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        float v = softplus(dtv[k] + bias);
        if (clamp) v = fminf(fmaxf(v, lo), hi);
        d[k] = lane * EPL + k < len ? v : 0.f;
        run_l += d[k] * av;
        cs[k] = run_l;
      }
      float incl = run_l;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(incl, off, 64);
        if (lane >= off) incl += t;
      }
      float excl = __shfl_up(incl, 1, 64);
      if (lane == 0) excl = 0.f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) cs[k] += excl;
      const float last = __shfl(cs[EPL - 1], 63, 64);
      const size_t o = (((size_t)b * H + h) * nc + c) * Q + lane * EPL;
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        dtp[o + k] = d[k];
        dAcs[o + k] = cs[k];
        s_w[w][lane * EPL + k] = expf(last - cs[k]) * d[k];
      }
      if (lane == 0) {
        s_last[w] = last;
        cdec[((size_t)b * H + h) * nc + c] = run;
      }
      run += last;
    }
    if (c + 1 < c1) {
      breg.load(b_base(c + 1), b_tok, min(Q, L - (c + 1) * Q), tid);
      load_dt(c + 1, dtv);
    }
    __syncthreads();                               // B^T, weights and exponents of chunk c in LDS
    bf16x8 bfr[KS];                                // this wavefront's B^T rows for the whole chunk
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      bfr[kk] = *reinterpret_cast<const bf16x8*>(&s_bt[(16 * w + r) * kSXP + 32 * kk + 8 * qd]);

#pragma unroll
    for (int hh = 0; hh < HS; ++hh) {
      if (hh > 0) __syncthreads();                 // the previous head's x^T consumed
      xreg.store(s_xt, s_w[hh], tid);
      // the next x tile: the next head of this chunk, or the first head of the next chunk
      if (hh + 1 < HS)
        xreg.load(x_base(c, hh + 1), x_tok, len, tid);
      else if (c + 1 < c1)
        xreg.load(x_base(c + 1, 0), x_tok, min(Q, L - (c + 1) * Q), tid);
      __syncthreads();
      const int h = h0 + hh;
      if (c > c0) {
        // L_c: the state this segment carried into chunk c, rounded to bf16 for the scan
        __bf16* dst = prev16 + (((size_t)b * nc + c) * H + h) * PN + 16 * w + r;
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[(size_t)(16 * pt + 4 * qd + e) * N] = static_cast<__bf16>(st[hh][pt][e]);
      }
      const float dec = expf(s_last[hh]);
#pragma unroll
      for (int pt = 0; pt < TP; ++pt)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[hh][pt][e] *= dec;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(&s_xt[(16 * pt + r) * kSXP + 32 * kk + 8 * qd]);
          st[hh][pt] = mfma_16x16x32_bf16(af, bfr[kk], st[hh][pt]);
        }
    }
  }
  // the segment's end states and total exponents
#pragma unroll
  for (int hh = 0; hh < HS; ++hh) {
    float* dst = E + (((size_t)b * nseg + seg) * H + h0 + hh) * PN + 16 * w + r;
#pragma unroll
    for (int pt = 0; pt < TP; ++pt)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(size_t)(16 * pt + 4 * qd + e) * N] = st[hh][pt][e];
  }
  if (w < HS && lane == 0) segdec[((size_t)b * H + h0 + w) * nseg + seg] = run;
}

bool chunk_state_seg_supported(int dtype, int P, int N, int Q, int hs) {
  return dtype == DT_BF16 && P == 64 && N == 128 && Q == kSQ && (hs == 1 || hs == 2 || hs == 4 || hs == 5);
}

hipError_t launch_chunk_state_seg(const FwdArgs& a, const SegArgs& sg, hipStream_t s) {
  if (!chunk_state_seg_supported(a.dtype, a.P, a.N, a.Q, sg.hs) || (a.H / a.G) % sg.hs != 0 || sg.SL < 1)
    return hipErrorInvalidValue;
  const uint32_t nblocks = (uint32_t)a.B * sg.nseg * a.G * ((a.H / a.G) / sg.hs);
  if (nblocks == 0) return hipSuccess;
#define SSD_SEG_LAUNCH(HS_)                                                                                   \
  hipExtLaunchKernelGGL(chunk_state_seg_kernel<HS_>, dim3(nblocks), dim3(kSThreads), 0, s, a.ev0, a.ev1, 0,   \
                        static_cast<const __bf16*>(a.x), static_cast<const __bf16*>(a.Bm),                     \
                        static_cast<const __bf16*>(a.dt), a.dt_bias, a.A, a.dtp, a.dAcs,                       \
                        static_cast<__bf16*>(a.prev16), sg.E, sg.segdec, sg.cdec, a.L, a.H, a.G, a.nc, sg.SL,   \
                        sg.nseg, a.clamp, a.dt_lo, a.dt_hi, nblocks)
  switch (sg.hs) {
    case 1: SSD_SEG_LAUNCH(1); break;
    case 2: SSD_SEG_LAUNCH(2); break;
    case 4: SSD_SEG_LAUNCH(4); break;
    default: SSD_SEG_LAUNCH(5); break;
  }
#undef SSD_SEG_LAUNCH
  return hipGetLastError();
}

}  // namespace ssd
