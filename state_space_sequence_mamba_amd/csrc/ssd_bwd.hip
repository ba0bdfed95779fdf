// Backward pass of the chunked SSD scan: the exact gradient of the forward recurrence
// (section 3.2 of "Agent 228: MAMBA-2 Reference Implementations Comparison", D skip of
// Gap 4 of "Agent 228: MAMBA-2 Implementation Gaps", optional gate and dt clamp), taken
// through the chunked form of Gap 1.
//
// Per batch row b, head h and chunk c (positions i, j inside the chunk, S = the in-chunk
// cumsum of dt' A, d = dt', CB_ij = C_i . B_j, DX_ij = dy_i . x_j, Hprev the state entering
// the chunk, Gnext the gradient of the state leaving it):
//   xi_j  = sum_{i>=j} e^(S_i-S_j) CB_ij dy_i  +  e^(S_last-S_j) Gnext B_j          (P)
//   dx_j  = D dy_j + d_j xi_j                       d(dt')_j direct part = x_j . xi_j
//   dB_j  = d_j [ sum_{i>=j} e^(S_i-S_j) DX_ij C_i  +  e^(S_last-S_j) x_j Gnext ]   (N, per head)
//   dC_i  = sum_{j<=i} e^(S_i-S_j) d_j DX_ij B_j  +  e^(S_i) dy_i Hprev             (N, per head)
//   dS_k  = sum_{j<=k} T_kj - sum_{i>=k} T_ik + R_k - U_k (+ sum_j U_j + V at the last position)
//           T_ij = e^(S_i-S_j) CB_ij d_j DX_ij,  R_k = e^(S_k) dy_k . (Hprev C_k),
//           U_j = e^(S_last-S_j) d_j x_j . (Gnext B_j),  V = e^(S_last) <Gnext, Hprev>
//   d(dt')_k = x_k . xi_k + A sum_{i>=k} dS_i,   dA += sum_k d_k sum_{i>=k} dS_i
// The state gradients G come from the forward's chunk_state (weights e^(S_i), on dy and C)
// and state_passing run in reverse; the forward states Hprev are recomputed by the forward
// kernels.
//
// Kernels here, each one workgroup of 256 threads:
//   bwd_dxdb   per (b, c, 64-row block R, slice of hs heads of a group): the anti-causal sums
//              over row blocks I >= R, head after head, dB summed over the slice in registers
//              (fp32: C B^T read from transposed blocks the forward recompute formed)
//   bwd_dc     per (b, c, R, slice of heads): the causal sums over row blocks J <= R, dC summed
//              over the slice (fp32: C B^T read from the blocks the forward recompute formed once
//              per group)
//   bwd_finalize per (b, c, h): dS, its reverse cumsum, d(dt), and the dA / d dt_bias partials
//   bwd_reduce_*: per-slice dB, dC summed over the slices of each group; parameter partials
//                 summed in a fixed order (results are run-to-run deterministic)
//   gate_bwd:  dy = dout silu(z) and dz = dout y~ silu'(z)
// Token tiles are staged in LDS in the input dtype (bf16 -> fp32 is exact, so the fp32 MFMA
// arithmetic is the same either way and bf16 tiles take half the LDS), with row pitches that
// start consecutive rows on different banks; the fp32 state tiles (Hprev, Gnext) reuse the
// space of the token tiles once those are consumed.  For bf16 inputs every product runs on bf16
// MFMA: the weighted tiles are rounded to bf16 (as the forward rounds its weighted C B^T), Hprev
// is rounded to bf16 (as the forward's carried term reads it), and Gnext, a gradient the forward
// never rounds, is split into bf16 hi and lo parts contracted in two exact passes.
#include <type_traits>

#include "cb_tiles.h"
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

namespace {
constexpr int KT = 64;   // tokens per tile (row block)
constexpr float kLog2e = 1.4426950408889634f;

// LDS row pitch (elements) of a W-wide tile of S: 16-byte aligned rows whose start banks
// differ from row to row.
template <typename S, int W> struct Pitch { static constexpr int v = W + (sizeof(S) == 4 ? 4 : 8); };

// Four consecutive tile elements, or one, as fp32 (bf16 -> fp32 is exact).
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4(const __bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ float ld1(const float* p) { return *p; }
__device__ __forceinline__ float ld1(const __bf16* p) { return static_cast<float>(*p); }

// KT token rows of width W (row stride `stride` elements), held in registers between their
// global loads and their LDS stores (pitch Pitch<T, W>), so that the next tile's loads are in
// flight during the current tile's MFMAs.  Rows past `nvalid` read row 0 and are zeroed at
// store time (a select at load time would wait for the data there).
template <typename T, int W>
struct RowTile {
  static constexpr int VEC = Vec16<T>::n, WV = W / VEC, UNITS = KT * WV, NIT = (UNITS + 255) / 256;
  static_assert(NIT <= 32, "validity mask");
  Vec16<T> v[NIT];
  uint32_t okm;
  __device__ __forceinline__ void load(const T* src, size_t stride, int nvalid, int tid) {
    okm = 0;
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const int u = min(tid + 256 * k, UNITS - 1);
      const int tok = u / WV, cv = (u % WV) * VEC;
      const bool ok = tok < nvalid;
      v[k] = load16(src + (size_t)(ok ? tok : 0) * stride + cv);
      okm |= (uint32_t)ok << k;
    }
  }
  __device__ __forceinline__ void store(T* dst, int tid) const {
    constexpr int PW = Pitch<T, W>::v;
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const int u = tid + 256 * k;
      if (UNITS % 256 == 0 || u < UNITS) {
        const int tok = u / WV, cv = (u % WV) * VEC;
        *reinterpret_cast<Vec16<T>*>(dst + tok * PW + cv) = keep_if(v[k], (okm >> k) & 1u);
      }
    }
  }
};

// Stage a (P x N) fp32 state as rows of pitch Pitch<S, N>, in S (fp32, or bf16 rounded to
// nearest even for the bf16 path, as the forward's carried term reads the entering states).
template <typename S, int P, int N>
__device__ __forceinline__ void stage_state(S* dst, const float* src, int tid) {
  constexpr int UNITS = P * N / 4, NIT = (UNITS + 255) / 256, PN = Pitch<S, N>::v;
  float4 v[NIT];
#pragma unroll
  for (int k = 0; k < NIT; ++k) v[k] = reinterpret_cast<const float4*>(src)[min(tid + 256 * k, UNITS - 1)];
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int u = tid + 256 * k;
    if (u < UNITS) {
      S* d = dst + ((4 * u) / N) * PN + (4 * u) % N;
      if constexpr (sizeof(S) == 4) {
        *reinterpret_cast<float4*>(d) = v[k];
      } else {
        bf16x4 q;
        q[0] = static_cast<__bf16>(v[k].x);
        q[1] = static_cast<__bf16>(v[k].y);
        q[2] = static_cast<__bf16>(v[k].z);
        q[3] = static_cast<__bf16>(v[k].w);
        *reinterpret_cast<bf16x4*>(d) = q;
      }
    }
  }
}

// Stage a (P x N) fp32 state as two bf16 arrays of rows of pitch Pitch<bf16, N>: hi = v rounded
// to bf16 (nearest even) and lo = (v - hi) rounded to bf16, so that hi + lo carries v to about
// 2^-17 of its magnitude.  A contraction of a bf16 tile with the state then runs as two bf16 MFMA
// passes (hi, then lo, into one fp32 accumulator) whose products are exact in fp32.
template <int P, int N>
__device__ __forceinline__ void stage_state_split(__bf16* hi, __bf16* lo, const float* src, int tid) {
  constexpr int UNITS = P * N / 4, NIT = (UNITS + 255) / 256, PN = Pitch<__bf16, N>::v;
  float4 v[NIT];
#pragma unroll
  for (int k = 0; k < NIT; ++k) v[k] = reinterpret_cast<const float4*>(src)[min(tid + 256 * k, UNITS - 1)];
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int u = tid + 256 * k;
    if (u < UNITS) {
      const int o = ((4 * u) / N) * PN + (4 * u) % N;
      const float vv[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
      bf16x4 qh, ql;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qh[e] = static_cast<__bf16>(vv[e]);
        ql[e] = static_cast<__bf16>(vv[e] - static_cast<float>(qh[e]));
      }
      *reinterpret_cast<bf16x4*>(hi + o) = qh;
      *reinterpret_cast<bf16x4*>(lo + o) = ql;
    }
  }
}

// Stage a (P x N) bf16 state as rows of pitch Pitch<bf16, N> (16-byte vectors, copied as they are).
template <int P, int N>
__device__ __forceinline__ void stage_state16(__bf16* dst, const __bf16* src, int tid) {
  constexpr int UNITS = P * N / 8, NIT = (UNITS + 255) / 256, PN = Pitch<__bf16, N>::v;
  uint4 v[NIT];
#pragma unroll
  for (int k = 0; k < NIT; ++k) v[k] = reinterpret_cast<const uint4*>(src)[min(tid + 256 * k, UNITS - 1)];
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int u = tid + 256 * k;
    if (u < UNITS) *reinterpret_cast<uint4*>(dst + ((8 * u) / N) * PN + (8 * u) % N) = v[k];
  }
}

// One 16 x 16 tile of A Bt^T over a contraction of length K along both operands' rows:
//   out[i][j] += sum_k A[i][k] * Bt[j][k]     (A, Bt: 16 rows each, pitch PA / PB)
// Lane (r, qd) feeds A row r and Bt row r with k = (K/4) qd + 4 m + c, one LDS read each per
// four MFMAs; it receives out[4 qd + e][r].
// Both operands bf16 (input tiles, K a multiple of 32): 16x16x32 bf16 MFMAs with
// k = 32 m + 8 qd + e, the same products (exact in fp32) summed in fp32 in another order.
template <int K, int PA, int PB, typename SA, typename SB>
__device__ __forceinline__ f32x4 mm_rows(f32x4 acc, const SA* A, const SB* Bt, int r, int qd) {
  if constexpr (sizeof(SA) == 2 && sizeof(SB) == 2 && K % 32 == 0) {
#pragma unroll
    for (int m = 0; m < K / 32; ++m) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + r * PA + 32 * m + 8 * qd);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + r * PB + 32 * m + 8 * qd);
      acc = mfma_16x16x32_bf16(a, b, acc);
    }
  } else {
#pragma unroll
    for (int m = 0; m < K / 16; ++m) {
      const float4 a = ld4(A + r * PA + (K / 4) * qd + 4 * m);
      const float4 b = ld4(Bt + r * PB + (K / 4) * qd + 4 * m);
      acc = mfma_16x16x4_f32(a.x, b.x, acc);
      acc = mfma_16x16x4_f32(a.y, b.y, acc);
      acc = mfma_16x16x4_f32(a.z, b.z, acc);
      acc = mfma_16x16x4_f32(a.w, b.w, acc);
    }
  }
  return acc;
}

// out[i][c] += sum_k M[k][i] * V[k][c] over the 16 k of one tile, where lane (r, qd) holds
// M[k = 4 qd + e][i = r] in m[e] (the result layout of mm_rows, used directly as the A
// operand), and V rows k (pitch PV) are read from LDS at column c0 + r.
// bf16 tiles: one 16x16x16 bf16 MFMA with M rounded to bf16 (the A operand layout is the same:
// lane (r, qd) holds k = 4 qd + e), as the forward rounds its weighted C B^T for (L o CB) X.
typedef short bwd_i16x4 __attribute__((ext_vector_type(4)));
typedef float bwd_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bwd_bf16x2 __attribute__((ext_vector_type(2)));
// Four consecutive rows of one column of a bf16 LDS tile as an MFMA B operand, in one transpose
// read (ds_read_b64_tr_b16): in each group of 16 lanes, with M[j][q] the q-th 16-bit element at
// lane j's 8-byte address, lane i receives M[4 k + i / 4][i % 4], k = 0..3.  Lane j of group qd
// points at row row0 + j / 4, columns c0 + 4 (j % 4) .. + 3, so lane (r, qd) receives
// V[row0 + k][c0 + r]: row0 = the group's first row (pitch PV and c0 multiples of 4: 8-byte
// aligned addresses).
template <int PV>
__device__ __forceinline__ bf16x4 col4_tr(const __bf16* V, int row0, int c0, int r) {
  const __bf16* p = V + (row0 + r / 4) * PV + c0 + 4 * (r % 4);
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                        (__attribute__((address_space(3))) bwd_i16x4*)(p)));
}
// four fp32 values rounded to bf16 (nearest even) by two two-value conversions
__device__ __forceinline__ bf16x4 round4(const f32x4& m) {
  const bwd_bf16x2 lo = __builtin_convertvector((bwd_f32x2{m[0], m[1]}), bwd_bf16x2);
  const bwd_bf16x2 hi = __builtin_convertvector((bwd_f32x2{m[2], m[3]}), bwd_bf16x2);
  return bf16x4{lo[0], lo[1], hi[0], hi[1]};
}

template <int PV, typename SV>
__device__ __forceinline__ f32x4 mm_regs(f32x4 acc, const f32x4& m, const SV* V, int c0, int r, int qd) {
  if constexpr (sizeof(SV) == 2) {
    static_assert(PV % 4 == 0, "8-byte aligned transpose reads");
    acc = mfma_16x16x16_bf16(round4(m), col4_tr<PV>(V, 4 * qd, c0, r), acc);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_16x16x4_f32(m[e], ld1(V + (4 * qd + e) * PV + c0 + r), acc);
  }
  return acc;
}

// out[i][c] += sum_k A[i][k] * V[k][c] over K, A rows i (pitch PA) and V rows k (pitch PV) in
// LDS; lane (r, qd) reads A row r as runs of four and V column c0 + r.  Both bf16: one
// 16x16x16 bf16 MFMA per run of four k.
template <int K, int PA, int PV, typename SA, typename SV>
__device__ __forceinline__ f32x4 mm_cols(f32x4 acc, const SA* A, const SV* V, int c0, int r, int qd) {
#pragma unroll
  for (int m = 0; m < K / 16; ++m) {
    const int k0 = (K / 4) * qd + 4 * m;
    if constexpr (sizeof(SA) == 2 && sizeof(SV) == 2) {
      static_assert(PV % 4 == 0, "8-byte aligned transpose reads");
      const bf16x4 a = *reinterpret_cast<const bf16x4*>(A + r * PA + k0);
      acc = mfma_16x16x16_bf16(a, col4_tr<PV>(V, k0, c0, r), acc);
    } else {
      const float4 a = ld4(A + r * PA + k0);
      acc = mfma_16x16x4_f32(a.x, ld1(V + (k0 + 0) * PV + c0 + r), acc);
      acc = mfma_16x16x4_f32(a.y, ld1(V + (k0 + 1) * PV + c0 + r), acc);
      acc = mfma_16x16x4_f32(a.z, ld1(V + (k0 + 2) * PV + c0 + r), acc);
      acc = mfma_16x16x4_f32(a.w, ld1(V + (k0 + 3) * PV + c0 + r), acc);
    }
  }
  return acc;
}

// Sum over the 16 lanes r of one qd group.
__device__ __forceinline__ float sum_r(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over the 4 qd groups of one lane r.
__device__ __forceinline__ float sum_qd(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}
}  // namespace

// ------------------------------------------------------------------ anti-causal: dx, dB
// Wavefront w owns the 16 columns j = 16 w .. 16 w + 15 of the row block R: it computes the
// (i, j) tiles of C B^T and dy x^T for every i of the block I, weights them in registers,
// and feeds them straight into xi[j][:] and dB[j][:] as MFMA A operands.  The tiles of block
// I + 1 are loaded into registers while block I is computed.
template <typename T, int P, int N, bool PRECB, int HS>
__global__ __launch_bounds__(256, 2) void bwd_dxdb_kernel(const T* __restrict__ x, const T* __restrict__ Bm,
                                                       const T* __restrict__ Cm, const T* __restrict__ dy,
                                                       const float* __restrict__ dtp, const float* __restrict__ dAcs,
                                                       const float* __restrict__ gstates,
                                                       const float* __restrict__ cbT,
                                                       const float* __restrict__ Dw, T* __restrict__ dx,
                                                       float* __restrict__ dBh, float* __restrict__ ddir,
                                                       float* __restrict__ dSa, float* __restrict__ Ub,
                                                       float* __restrict__ pD, int L, int H, int G, int nc, int Q,
                                                       uint32_t nblocks) {
  constexpr int hs = HS;
  constexpr int PP = Pitch<T, P>::v, NP = Pitch<T, N>::v, NPF = N + 4, TPm = P / 16, TNm = N / 16;
  constexpr int C_BYTES = KT * NP * (int)sizeof(T), DY_BYTES = KT * PP * (int)sizeof(T);
  // Gnext staged in fp32, or for bf16 tiles as bf16 hi and lo parts (stage_state_split)
  constexpr int G_BYTES = sizeof(T) == 2 ? 2 * P * NP * 2 : P * NPF * 4;
  constexpr int U_BYTES = C_BYTES + DY_BYTES > G_BYTES ? C_BYTES + DY_BYTES : G_BYTES;
  __shared__ __attribute__((aligned(16))) T s_b[KT * NP];       // B of the own block R
  __shared__ __attribute__((aligned(16))) T s_x[KT * PP];       // x of R
  __shared__ __attribute__((aligned(16))) char s_un[U_BYTES];   // C and dy of block I; later Gnext
  __shared__ float s_SR[KT], s_dR[KT], s_SI[KT];
  __shared__ float s_red[4][P];
  T* s_c = reinterpret_cast<T*>(s_un);
  T* s_dy = reinterpret_cast<T*>(s_un + C_BYTES);
  float* s_g = reinterpret_cast<float*>(s_un);
  __bf16* s_ghi = reinterpret_cast<__bf16*>(s_un);
  __bf16* s_glo = s_ghi + P * NP;

  // a workgroup takes `hs` consecutive heads of one group (one after the other) and sums their
  // dB contributions in registers, in head order: dB leaves per slice of heads, not per head
  const int nrb = Q / KT, nsl = H / hs;
  uint32_t id = xcd_swizzle(blockIdx.x, nblocks);
  const int hsl = id % nsl;
  id /= nsl;
  const int R = id % nrb;
  id /= nrb;
  const int c = id % nc, b = id / nc;
  const int h0 = hsl * hs;
  const int g = h0 / (H / G);
  const int t0 = c * Q, len = min(Q, L - t0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;
  if (R * KT >= len) {                 // a row block past the end of the sequence: no rows,
    if (tid < P)                       // but its dD partials are still summed
      for (int hh = 0; hh < hs; ++hh)
        pD[(((size_t)b * nc + c) * nrb + R) * (size_t)(H * P) + (size_t)(h0 + hh) * P + tid] = 0.f;
    return;
  }
  const int lenR = min(KT, len - R * KT);
  const size_t xs = (size_t)H * P, bs = (size_t)G * N;
  const T* Cg = Cm + ((size_t)b * L + t0) * bs + (size_t)g * N;

  RowTile<T, N> tb, tc;
  RowTile<T, P> tx, tdy;
  if constexpr (HS > 1) {                          // the own block's B, once for the slice's heads
    tb.load(Bm + ((size_t)b * L + t0 + R * KT) * bs + (size_t)g * N, bs, lenR, tid);
    tb.store(s_b, tid);
  }
  f32x4 dbs[TNm];                                  // sum over the slice's heads of d_j dB_h[j][n]
#pragma unroll
  for (int m = 0; m < TNm; ++m) dbs[m] = zero4();
  float djs[4];

#pragma unroll 1
  for (int hh = 0; hh < hs; ++hh) {
  // lane-dependent values re-derived from an opaque copy of the thread index each head, so that
  // nothing per lane is hoisted out of the head loop and kept live across it
  int tid_l = threadIdx.x;
  if constexpr (HS > 1) asm volatile("" : "+v"(tid_l));
  const int tid = tid_l, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;
  const int tk = min(tid, KT - 1);
  const int h = h0 + hh;
  if (hh > 0) __syncthreads();                     // the previous head's tiles and partials consumed
  const size_t cq = (((size_t)b * H + h) * nc + c) * Q;
  const T* dyg = dy + ((size_t)b * L + t0) * xs + (size_t)h * P;

  // prologue: the own block's B (once for the slice's heads) and x, block I = R's C and dy, and
  // the cumsums, all in flight
  if constexpr (HS == 1) tb.load(Bm + ((size_t)b * L + t0 + R * KT) * bs + (size_t)g * N, bs, lenR, tid);
  tx.load(x + ((size_t)b * L + t0 + R * KT) * xs + (size_t)h * P, xs, lenR, tid);
  tc.load(Cg + (size_t)(R * KT) * bs, bs, lenR, tid);
  tdy.load(dyg + (size_t)(R * KT) * xs, xs, lenR, tid);
  const float sR = dAcs[cq + R * KT + tk], dR = dtp[cq + R * KT + tk];
  float sI = sR;
  const float Slast = dAcs[cq + Q - 1];
  if constexpr (HS == 1) tb.store(s_b, tid);
  tx.store(s_x, tid);
  if (tid < KT) {
    s_SR[tid] = sR;
    s_dR[tid] = dR;
  }

  f32x4 xi[TPm], db[TNm];
#pragma unroll
  for (int m = 0; m < TPm; ++m) xi[m] = zero4();
#pragma unroll
  for (int m = 0; m < TNm; ++m) db[m] = zero4();
  float cs = 0.f;                                  // column j = 16 w + r: sum_i M1 DX (partial over qd)
  const int jl = 16 * w + r;                       // this lane's column of R
  // bf16: the own block's dy at the lane's output positions (rows j = 16 w + 4 qd + e, columns
  // p = 16 m + r), taken from the staged tile of the first block (I = R) for the skip term and
  // the dD partial at the end, instead of global loads there
  bf16x4 dyR[TPm];

  const int nI = (len + KT - 1) / KT;
  // PRECB: the C B^T sub-tiles (row tiles of block I, own column tile w of R) come from the
  // transposed blocks the forward recompute formed once per group (cb_block TRANS: the same
  // MFMA sequence as mm_rows here, so the same values), one 16-byte load per lane and sub-tile
  const float* cb_grp = cbT + (((size_t)b * nc + c) * G + g) * (size_t)(nrb * (nrb + 1) / 2) * kCbBlock +
                        ((size_t)(w * 4) * 64 + lane) * 4;
  auto cb_at = [&](int I, int ti) {
    return *reinterpret_cast<const f32x4*>(cb_grp + (size_t)(I * (I + 1) / 2 + R) * kCbBlock + 256 * ti);
  };
  f32x4 cbr[4] = {};
  if constexpr (PRECB) {
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) cbr[ti] = cb_at(R, ti);
  }
  for (int I = R; I < nI; ++I) {
    const int lenI = min(KT, len - I * KT);
    __syncthreads();
    tc.store(s_c, tid);
    tdy.store(s_dy, tid);
    if (tid < KT) s_SI[tid] = sI;
    if (I + 1 < nI) {
      const int lenN = min(KT, len - (I + 1) * KT);
      tc.load(Cg + (size_t)((I + 1) * KT) * bs, bs, lenN, tid);
      tdy.load(dyg + (size_t)((I + 1) * KT) * xs, xs, lenN, tid);
      sI = dAcs[cq + (I + 1) * KT + tk];
    }
    __syncthreads();
    if constexpr (sizeof(T) == 2) {
      if (I == R) {
#pragma unroll
        for (int m = 0; m < TPm; ++m) dyR[m] = col4_tr<PP>(s_dy, 16 * w + 4 * qd, 16 * m, r);
      }
    }
    const float sj = s_SR[jl];
    // MASK: the diagonal block or a block that crosses the end of the sequence; other blocks
    // (every i after every j, all rows real) run as straight-line code without the mask
    auto block = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        f32x4 cb;
        if constexpr (PRECB) {
          cb = cbr[ti];
          if (I + 1 < nI) cbr[ti] = cb_at(I + 1, ti);  // block I + 1's, into the released register
        }
        if (MASK && I == R && ti < w) continue;    // tile entirely above the diagonal (i < j)
        if constexpr (!PRECB) cb = mm_rows<N, NP, NP>(zero4(), s_c + 16 * ti * NP, s_b + 16 * w * NP, r, qd);
        f32x4 dxv = mm_rows<P, PP, PP>(zero4(), s_dy + 16 * ti * PP, s_x + 16 * w * PP, r, qd);
        f32x4 m1, m2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int il = 16 * ti + 4 * qd + e;
          const bool ok = !MASK || ((I * KT + il >= R * KT + jl) && il < lenI && jl < lenR);
          const float ev = ok ? __builtin_amdgcn_exp2f((s_SI[il] - sj) * kLog2e) : 0.f;
          m1[e] = ev * cb[e];
          m2[e] = ev * dxv[e];
          cs += m1[e] * dxv[e];
        }
#pragma unroll
        for (int m = 0; m < TPm; ++m) xi[m] = mm_regs<PP>(xi[m], m1, s_dy + 16 * ti * PP, 16 * m, r, qd);
#pragma unroll
        for (int m = 0; m < TNm; ++m) db[m] = mm_regs<NP>(db[m], m2, s_c + 16 * ti * NP, 16 * m, r, qd);
      }
    };
    // (fp32 only: for bf16 tiles the second copy of the block was slower, 936 -> 1325 us)
    if (sizeof(T) == 4 && I > R && lenI == KT && lenR == KT)
      block(std::false_type());
    else
      block(std::true_type());
  }

  // carried terms through the gradient of the state leaving the chunk (for bf16 tiles on bf16
  // MFMA: two passes over Gnext's hi and lo parts, B and x being exact in bf16)
  __syncthreads();
  if constexpr (sizeof(T) == 2)
    stage_state_split<P, N>(s_ghi, s_glo, gstates + (((size_t)b * nc + c) * H + h) * (size_t)(P * N), tid);
  else
    stage_state<float, P, N>(s_g, gstates + (((size_t)b * nc + c) * H + h) * (size_t)(P * N), tid);
  __syncthreads();
  // lane rows j = 16 w + 4 qd + e from here on
  float f[4], dj[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 16 * w + 4 * qd + e;
    f[e] = __builtin_amdgcn_exp2f((Slast - s_SR[j]) * kLog2e);
    dj[e] = s_dR[j];
  }
  float u[4] = {0.f, 0.f, 0.f, 0.f};
  // x of the own block at the lane's positions (rows j = 16 w + 4 qd + e, columns p = 16 m + r):
  // for bf16 tiles by transpose reads, once for the carried terms, dd and the dD partial
  auto x_at = [&](int m, int e) -> float { return ld1(s_x + (16 * w + 4 * qd + e) * PP + 16 * m + r); };
  bf16x4 xR[TPm];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int m = 0; m < TPm; ++m) xR[m] = col4_tr<PP>(s_x, 16 * w + 4 * qd, 16 * m, r);
  }
  auto xv = [&](int m, int e) -> float {
    if constexpr (sizeof(T) == 2) return static_cast<float>(xR[m][e]);
    else return x_at(m, e);
  };
#pragma unroll
  for (int m = 0; m < TPm; ++m) {
    // tmp[j][p] = sum_n B[j][n] Gnext[p][n]
    f32x4 tmp;
    if constexpr (sizeof(T) == 2) {
      tmp = mm_rows<N, NP, NP>(zero4(), s_b + 16 * w * NP, s_ghi + 16 * m * NP, r, qd);
      tmp = mm_rows<N, NP, NP>(tmp, s_b + 16 * w * NP, s_glo + 16 * m * NP, r, qd);
    } else {
      tmp = mm_rows<N, NP, NPF>(zero4(), s_b + 16 * w * NP, s_g + 16 * m * NPF, r, qd);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[e] += xv(m, e) * tmp[e];
      xi[m][e] += f[e] * tmp[e];
    }
  }
#pragma unroll
  for (int m = 0; m < TNm; ++m) {
    // xg[j][n] = sum_p x[j][p] Gnext[p][n]
    f32x4 xg;
    if constexpr (sizeof(T) == 2) {
      xg = mm_cols<P, PP, NP>(zero4(), s_x + 16 * w * PP, s_ghi, 16 * m, r, qd);
      xg = mm_cols<P, PP, NP>(xg, s_x + 16 * w * PP, s_glo, 16 * m, r, qd);
    } else {
      xg = mm_cols<P, PP, NPF>(zero4(), s_x + 16 * w * PP, s_g, 16 * m, r, qd);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) db[m][e] += f[e] * xg[e];
  }
  float U[4], dd[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float q = 0.f;
#pragma unroll
    for (int m = 0; m < TPm; ++m) q += xv(m, e) * xi[m][e];
    U[e] = f[e] * dj[e] * sum_r(u[e]);
    dd[e] = sum_r(q);
  }
  const float colsum = s_dR[jl] * sum_qd(cs);

  // outputs of the own block R
  const size_t row0 = (size_t)b * L + t0 + R * KT;
  float dDp[TPm];
#pragma unroll
  for (int m = 0; m < TPm; ++m) dDp[m] = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 16 * w + 4 * qd + e;
    const bool ok = j < lenR;
    const size_t tok = row0 + (ok ? j : 0);
#pragma unroll
    for (int m = 0; m < TPm; ++m) {
      const int p = 16 * m + r;
      float dyv;
      if constexpr (sizeof(T) == 2)
        dyv = ok ? static_cast<float>(dyR[m][e]) : 0.f;
      else
        dyv = ok ? to_f32(dy[tok * xs + (size_t)h * P + p]) : 0.f;
      const float dw = Dw ? Dw[(size_t)h * P + p] : 0.f;
      if (ok) dx[tok * xs + (size_t)h * P + p] = from_f32<T>(dw * dyv + dj[e] * xi[m][e]);
      dDp[m] += dyv * xv(m, e);
    }
    if constexpr (HS == 1) {                       // one head: dB straight out
      if (ok) {
#pragma unroll
        for (int m = 0; m < TNm; ++m) dBh[(tok * H + h) * (size_t)N + 16 * m + r] = dj[e] * db[m][e];
      }
    } else {
#pragma unroll
      for (int m = 0; m < TNm; ++m) dbs[m][e] += dj[e] * db[m][e];
    }
    if (ok && r == 0) {
      ddir[cq + R * KT + j] = dd[e];
      Ub[cq + R * KT + j] = U[e];
    }
  }
  // the column sums belong to column j = 16 w + r; its U was computed by the lane holding row j
  __syncthreads();
  float* s_u = s_g;                                  // Gnext no longer needed
  if (r == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) s_u[16 * w + 4 * qd + e] = U[e];
  }
  // dD partial of this block: per channel p, summed over the block's rows
#pragma unroll
  for (int m = 0; m < TPm; ++m) {
    float v = dDp[m];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (qd == 0) s_red[w][16 * m + r] = v;
  }
  __syncthreads();
  if (qd == 0 && jl < lenR) dSa[cq + R * KT + jl] = -colsum - s_u[jl];
  if (tid < P)
    pD[(((size_t)b * nc + c) * nrb + R) * (size_t)(H * P) + (size_t)h * P + tid] =
        s_red[0][tid] + s_red[1][tid] + s_red[2][tid] + s_red[3][tid];
  }  // heads of the slice
  (void)djs;
  if constexpr (HS == 1) return;
  // dB of the slice: rows j = 16 w + 4 qd + e of R
  const size_t row0s = (size_t)b * L + t0 + R * KT;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 16 * w + 4 * qd + e;
    if (j < lenR) {
#pragma unroll
      for (int m = 0; m < TNm; ++m) dBh[((row0s + j) * nsl + hsl) * (size_t)N + 16 * m + r] = dbs[m][e];
    }
  }
}

// ------------------------------------------------------------------ causal: dC
// Wavefront w owns the 16 rows i = 16 w .. 16 w + 15 of the row block R.  It computes the
// transposed tiles (j, i) of B C^T and x dy^T for every j of block J, so that the weighted
// tile feeds dC[i][:] directly as an MFMA A operand.  The tiles of block J + 1 are loaded
// into registers while block J is computed.
template <typename T, int P, int N, bool PRECB, int HS>
__global__ __launch_bounds__(256, 2) void bwd_dc_kernel(const T* __restrict__ x, const T* __restrict__ Bm,
                                                     const T* __restrict__ Cm, const T* __restrict__ dy,
                                                     const float* __restrict__ dtp, const float* __restrict__ dAcs,
                                                     const float* __restrict__ states,
                                                     const __bf16* __restrict__ states16,
                                                     const float* __restrict__ cbp, float* __restrict__ dCh,
                                                     float* __restrict__ dSc, int L, int H, int G, int nc, int Q,
                                                     uint32_t nblocks) {
  constexpr int hs = HS;
  constexpr int PP = Pitch<T, P>::v, NP = Pitch<T, N>::v, TNm = N / 16;
  constexpr int B_BYTES = KT * NP * (int)sizeof(T), X_BYTES = KT * PP * (int)sizeof(T);
  constexpr int H_BYTES = P * NP * (int)sizeof(T);                // Hprev staged in T
  constexpr int U_BYTES = B_BYTES + X_BYTES > H_BYTES ? B_BYTES + X_BYTES : H_BYTES;
  __shared__ __attribute__((aligned(16))) T s_c[KT * NP];       // C of the own block R
  __shared__ __attribute__((aligned(16))) T s_dy[KT * PP];      // dy of R
  __shared__ __attribute__((aligned(16))) char s_un[U_BYTES];   // B and x of block J; later Hprev
  __shared__ float s_SR[KT], s_SJ[KT], s_dJ[KT], s_rr[KT];
  T* s_b = reinterpret_cast<T*>(s_un);
  T* s_x = reinterpret_cast<T*>(s_un + B_BYTES);
  T* s_h = reinterpret_cast<T*>(s_un);

  // a workgroup takes `hs` consecutive heads of one group (one after the other) and sums their
  // dC contributions in registers, in head order: dC leaves per slice of heads, not per head
  const int nrb = Q / KT, nsl = H / hs;
  uint32_t id = xcd_swizzle(blockIdx.x, nblocks);
  const int hsl = id % nsl;
  id /= nsl;
  const int R = id % nrb;
  id /= nrb;
  const int c = id % nc, b = id / nc;
  const int h0 = hsl * hs;
  const int g = h0 / (H / G);
  const int t0 = c * Q, len = min(Q, L - t0);
  if (R * KT >= len) return;
  const int lenR = min(KT, len - R * KT);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;
  const size_t xs = (size_t)H * P, bs = (size_t)G * N;
  const T* Bg = Bm + ((size_t)b * L + t0) * bs + (size_t)g * N;

  RowTile<T, N> tc, tb;
  RowTile<T, P> tdy, tx;
  // dC[i][n] of this lane, accumulated over the slice's heads in head order (the accumulators are
  // not reset between heads: one set of registers instead of a per-head set and a sum)
  f32x4 dc[TNm];
#pragma unroll
  for (int m = 0; m < TNm; ++m) dc[m] = zero4();

#pragma unroll 1
  for (int hh = 0; hh < hs; ++hh) {
  // lane-dependent values re-derived from an opaque copy of the thread index each head, so that
  // nothing per lane is hoisted out of the head loop and kept live across it
  int tid_l = threadIdx.x;
  if constexpr (HS > 1) asm volatile("" : "+v"(tid_l));
  const int tid = tid_l, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;
  const int tk = min(tid, KT - 1);
  const int h = h0 + hh;
  if (hh > 0) __syncthreads();                     // the previous head's tiles and partials consumed
  const size_t cq = (((size_t)b * H + h) * nc + c) * Q;
  const T* xg = x + ((size_t)b * L + t0) * xs + (size_t)h * P;

  // prologue: the own block's C (once for the slice's heads) and dy, block J = 0's B and x, and
  // the cumsums, all in flight
  if (HS == 1 || hh == 0) tc.load(Cm + ((size_t)b * L + t0 + R * KT) * bs + (size_t)g * N, bs, lenR, tid);
  tdy.load(dy + ((size_t)b * L + t0 + R * KT) * xs + (size_t)h * P, xs, lenR, tid);
  const int len0 = min(KT, len);
  tb.load(Bg, bs, len0, tid);
  tx.load(xg, xs, len0, tid);
  const float sR = dAcs[cq + R * KT + tk];
  float sJ = dAcs[cq + tk], dJ = dtp[cq + tk];
  // PRECB: the C B^T sub-tiles (own strip w, column tiles of block J) come from the blocks the
  // forward recompute formed once per group (cb_block: the same MFMA sequence as mm_rows here,
  // so the same values), one 16-byte load per lane and sub-tile
  const float* cb_lane = cbp + ((((size_t)b * nc + c) * G + g) * (size_t)(nrb * (nrb + 1) / 2) +
                                (size_t)(R * (R + 1) / 2)) * kCbBlock + ((size_t)(w * 4) * 64 + lane) * 4;
  f32x4 cbr[4] = {};
  if constexpr (PRECB) {
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) cbr[tj] = *reinterpret_cast<const f32x4*>(cb_lane + 256 * tj);
  }
  if (HS == 1 || hh == 0) tc.store(s_c, tid);
  tdy.store(s_dy, tid);
  if (tid < KT) s_SR[tid] = sR;

  float rs = 0.f;                                  // row i = 16 w + r: sum_j T_ij (partial over qd)
  const int il = 16 * w + r;
  for (int J = 0; J <= R; ++J) {
    const int lenJ = min(KT, len - J * KT);
    __syncthreads();
    tb.store(s_b, tid);
    tx.store(s_x, tid);
    if (tid < KT) {
      s_SJ[tid] = sJ;
      s_dJ[tid] = dJ;
    }
    if (J < R) {
      const int lenN = min(KT, len - (J + 1) * KT);
      tb.load(Bg + (size_t)((J + 1) * KT) * bs, bs, lenN, tid);
      tx.load(xg + (size_t)((J + 1) * KT) * xs, xs, lenN, tid);
      sJ = dAcs[cq + (J + 1) * KT + tk];
      dJ = dtp[cq + (J + 1) * KT + tk];
    }
    __syncthreads();
    const float si = s_SR[il];
    // MASK as in bwd_dxdb: blocks before the diagonal with all rows real run unmasked
    auto block = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        if (MASK && J == R && tj > w) continue;    // tile entirely after the diagonal (j > i)
        f32x4 cbt;
        if constexpr (PRECB) {
          cbt = cbr[tj];
          // block J + 1's sub-tile into the register this one releases
          if (J < R) cbr[tj] = *reinterpret_cast<const f32x4*>(cb_lane + (size_t)(J + 1) * kCbBlock + 256 * tj);
        } else {
          cbt = mm_rows<N, NP, NP>(zero4(), s_b + 16 * tj * NP, s_c + 16 * w * NP, r, qd);
        }
        const f32x4 dxt = mm_rows<P, PP, PP>(zero4(), s_x + 16 * tj * PP, s_dy + 16 * w * PP, r, qd);
        f32x4 wt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jl = 16 * tj + 4 * qd + e;
          const bool ok = !MASK || ((R * KT + il >= J * KT + jl) && il < lenR && jl < lenJ);
          wt[e] = ok ? __builtin_amdgcn_exp2f((si - s_SJ[jl]) * kLog2e) * s_dJ[jl] * dxt[e] : 0.f;
          rs += wt[e] * cbt[e];
        }
#pragma unroll
        for (int m = 0; m < TNm; ++m) dc[m] = mm_regs<NP>(dc[m], wt, s_b + 16 * tj * NP, 16 * m, r, qd);
      }
    };
    if (J < R && lenJ == KT && lenR == KT)
      block(std::false_type());
    else
      block(std::true_type());
  }
  __syncthreads();
  // Hprev in T; for bf16, the copy state_passing rounded to bf16 when it wrote the states (the
  // same rounding, half the bytes) when there is one
  if constexpr (sizeof(T) == 2) {
    if (states16)
      stage_state16<P, N>(s_h, states16 + (((size_t)b * nc + c) * H + h) * (size_t)(P * N), tid);
    else
      stage_state<T, P, N>(s_h, states + (((size_t)b * nc + c) * H + h) * (size_t)(P * N), tid);
  } else {
    stage_state<T, P, N>(s_h, states + (((size_t)b * nc + c) * H + h) * (size_t)(P * N), tid);
  }
  __syncthreads();
  // lane rows i = 16 w + 4 qd + e from here on
  const size_t row0 = (size_t)b * L + t0 + R * KT;
  float rr[4] = {0.f, 0.f, 0.f, 0.f}, ei[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ei[e] = __builtin_amdgcn_exp2f(s_SR[16 * w + 4 * qd + e] * kLog2e);
#pragma unroll
  for (int m = 0; m < TNm; ++m) {
    // cr[i][n] = sum_p dy[i][p] Hprev[p][n]
    const f32x4 cr = mm_cols<P, PP, NP>(zero4(), s_dy + 16 * w * PP, s_h, 16 * m, r, qd);
    // C[i][n] at the lane's positions (rows i = 16 w + 4 qd + e, column n = 16 m + r); for bf16
    // tiles one transpose read
    bf16x4 cT;
    if constexpr (sizeof(T) == 2) cT = col4_tr<NP>(s_c, 16 * w + 4 * qd, 16 * m, r);
    auto cv = [&](int e) -> float {
      if constexpr (sizeof(T) == 2) return static_cast<float>(cT[e]);
      else return ld1(s_c + (16 * w + 4 * qd + e) * NP + 16 * m + r);
    };
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rr[e] += cr[e] * cv(e);
      dc[m][e] += ei[e] * cr[e];
    }
  }
  const float rsum = sum_qd(rs);                   // row il
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 16 * w + 4 * qd + e;
    const float rv = ei[e] * sum_r(rr[e]);
    if (r == 0) s_rr[i] = rv;
    if constexpr (HS == 1) {                       // one head: dC straight out
      if (i < lenR) {
#pragma unroll
        for (int m = 0; m < TNm; ++m) dCh[((row0 + i) * H + h) * (size_t)N + 16 * m + r] = dc[m][e];
      }
    }
  }
  __syncthreads();
  if (qd == 0 && il < lenR) dSc[cq + R * KT + il] = rsum + s_rr[il];
  }  // heads of the slice
  if constexpr (HS == 1) return;
  // dC of the slice: rows i = 16 w + 4 qd + e of R
  const size_t row0s = (size_t)b * L + t0 + R * KT;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 16 * w + 4 * qd + e;
    if (i < lenR) {
#pragma unroll
      for (int m = 0; m < TNm; ++m) dCh[((row0s + i) * nsl + hsl) * (size_t)N + 16 * m + r] = dc[m][e];
    }
  }
}

// ------------------------------------------------------------------ per-chunk finalize
template <typename T, int P, int N>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(const T* __restrict__ dt, const float* __restrict__ dt_bias,
                                                           const float* __restrict__ A, const float* __restrict__ dtp,
                                                           const float* __restrict__ dAcs,
                                                           const float* __restrict__ states,
                                                           const float* __restrict__ gstates,
                                                           const float* __restrict__ ddir,
                                                           const float* __restrict__ dSa,
                                                           const float* __restrict__ dSc,
                                                           const float* __restrict__ Ub, T* __restrict__ ddt,
                                                           float* __restrict__ pA, float* __restrict__ pbias, int L,
                                                           int H, int nc, int Q, int clamp, float lo, float hi) {
  __shared__ float s_v[256];
  __shared__ float s_red[4][4];
  const int h = blockIdx.x % H;
  const int c = (blockIdx.x / H) % nc;
  const int b = blockIdx.x / (H * nc);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = c * Q, len = min(Q, L - t0);
  const size_t cq = (((size_t)b * H + h) * nc + c) * Q;
  const size_t st = (((size_t)b * nc + c) * H + h) * (size_t)(P * N);

  // block sums of up to four values, in a fixed order
  auto block_sum = [&](float (&v)[4], int cnt) {
    for (int k = 0; k < cnt; ++k) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v[k] += __shfl_xor(v[k], o, 64);
    }
    __syncthreads();
    if (lane == 0)
      for (int k = 0; k < cnt; ++k) s_red[wave][k] = v[k];
    __syncthreads();
    for (int k = 0; k < cnt; ++k) v[k] = s_red[0][k] + s_red[1][k] + s_red[2][k] + s_red[3][k];
  };

  // V = e^(S_last) <Gnext, Hprev>, and the sum of U over the chunk
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int e = tid; e < P * N / 4; e += 256) {
    const float4 gv = reinterpret_cast<const float4*>(gstates + st)[e];
    const float4 hv = reinterpret_cast<const float4*>(states + st)[e];
    acc[0] += gv.x * hv.x + gv.y * hv.y + gv.z * hv.z + gv.w * hv.w;
  }
  const bool ok = tid < len;
  acc[1] = ok ? Ub[cq + tid] : 0.f;
  block_sum(acc, 2);
  const float V = expf(dAcs[cq + Q - 1]) * acc[0];
  const float Usum = acc[1];

  // dS and its reverse inclusive cumsum over the chunk
  float dS = ok ? dSa[cq + tid] + dSc[cq + tid] : 0.f;
  if (tid == len - 1) dS += Usum + V;
  s_v[tid] = dS;
  for (int o = 1; o < 256; o <<= 1) {
    __syncthreads();
    const float add = tid + o < 256 ? s_v[tid + o] : 0.f;
    __syncthreads();
    s_v[tid] += add;
  }
  __syncthreads();
  const float rsum = s_v[tid];
  const float d = ok ? dtp[cq + tid] : 0.f;
  const float Ah = A[h];
  float g = 0.f;
  if (ok) {
    const float dd = ddir[cq + tid] + Ah * rsum;
    const size_t tok = (size_t)b * L + t0 + tid;
    const float raw = to_f32(dt[tok * H + h]) + dt_bias[h];
    const float sig = 1.f / (1.f + expf(-raw));
    float inside = 1.f;
    if (clamp) {
      const float sp = softplus(raw);
      inside = (sp >= lo && sp <= hi) ? 1.f : 0.f;
    }
    g = dd * sig * inside;
    ddt[tok * H + h] = from_f32<T>(g);
  }
  float part[4] = {d * rsum, g, 0.f, 0.f};
  block_sum(part, 2);
  if (tid == 0) {
    pA[((size_t)b * nc + c) * H + h] = part[0];
    pbias[((size_t)b * nc + c) * H + h] = part[1];
  }
}

// ------------------------------------------------------------------ reductions
// dB, dC of each group: the per-head partials summed over the heads of the group in head
// order.  Each thread owns four consecutive n (16-byte loads and stores) and keeps the loads
// of four heads in flight; the order of the additions is the sequential one.
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ dBh,
                                                            const float* __restrict__ dCh, T* __restrict__ dB,
                                                            T* __restrict__ dC, int H, int G, int N, size_t total4,
                                                            int nsl_b, int nsl_c) {
  const size_t e4 = (size_t)blockIdx.x * 256 + threadIdx.x;   // index into (B, L, G, N / 4)
  if (e4 >= total4) return;
  const int N4 = N / 4;
  const int n = (int)(e4 % N4) * 4;
  const size_t bg = e4 / N4;
  const int g = (int)(bg % G);
  const size_t bl = bg / G;
  (void)H;
  // dB and dC: per slice of heads, nsl_b / nsl_c slices per batch-token row, hb / hc per group
  const int hb = nsl_b / G, hc = nsl_c / G;
  const float* pb = dBh + (bl * nsl_b + (size_t)g * hb) * N + n;
  const float* pc = dCh + (bl * nsl_c + (size_t)g * hc) * N + n;
  auto add = [](float4& acc, const float4& v) {
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  };
  // the slices of one tensor in order, four loads in flight
  auto sum = [&](const float* p, int k_n) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int k = 0;
    for (; k + 4 <= k_n; k += 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4*>(p + (size_t)(k + u) * N);
#pragma unroll
      for (int u = 0; u < 4; ++u) add(acc, v[u]);
    }
    for (; k < k_n; ++k) add(acc, *reinterpret_cast<const float4*>(p + (size_t)k * N));
    return acc;
  };
  const float4 sb = sum(pb, hb), sc = sum(pc, hc);
  const size_t e = e4 * 4;
  dB[e + 0] = from_f32<T>(sb.x);
  dB[e + 1] = from_f32<T>(sb.y);
  dB[e + 2] = from_f32<T>(sb.z);
  dB[e + 3] = from_f32<T>(sb.w);
  dC[e + 0] = from_f32<T>(sc.x);
  dC[e + 1] = from_f32<T>(sc.y);
  dC[e + 2] = from_f32<T>(sc.z);
  dC[e + 3] = from_f32<T>(sc.w);
}

__global__ __launch_bounds__(256) void bwd_reduce_params_kernel(const float* __restrict__ pA,
                                                                const float* __restrict__ pbias,
                                                                const float* __restrict__ pD, float* __restrict__ dA,
                                                                float* __restrict__ dbias, float* __restrict__ dD,
                                                                int H, int P, int nbc, int nbr) {
  // one workgroup per head: nbc = B * nc partial rows of pA / pbias, nbr = B * nc * (Q/64) of pD
  __shared__ float s_a[256], s_b[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  float a = 0.f, bb = 0.f;
  for (int k = tid; k < nbc; k += 256) {
    a += pA[(size_t)k * H + h];
    bb += pbias[(size_t)k * H + h];
  }
  s_a[tid] = a;
  s_b[tid] = bb;
  for (int o = 128; o > 0; o >>= 1) {
    __syncthreads();
    if (tid < o) {
      s_a[tid] += s_a[tid + o];
      s_b[tid] += s_b[tid + o];
    }
  }
  if (tid == 0) {
    dA[h] = s_a[0];
    dbias[h] = s_b[0];
  }
  if (dD) {
    // thread (slice sl, channel p) sums the partial rows k = sl (mod S), four loads in flight;
    // the S slice sums are then added in slice order
    const int S = 256 / P, p = tid % P, sl = tid / P;
    float sD = 0.f;
    int k = sl;
    for (; k + 3 * S < nbr; k += 4 * S) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = pD[((size_t)(k + u * S) * H + h) * P + p];
#pragma unroll
      for (int u = 0; u < 4; ++u) sD += v[u];
    }
    for (; k < nbr; k += S) sD += pD[((size_t)k * H + h) * P + p];
    __syncthreads();
    s_a[tid] = sD;
    __syncthreads();
    if (tid < P) {
      float t = 0.f;
      for (int j = 0; j < S; ++j) t += s_a[j * P + tid];
      dD[(size_t)h * P + tid] = t;
    }
  }
}

// ------------------------------------------------------------------ gate
template <typename T>
__global__ __launch_bounds__(256) void gate_bwd_kernel(const T* __restrict__ dout, const T* __restrict__ z,
                                                       const T* __restrict__ ypre, T* __restrict__ dy,
                                                       T* __restrict__ dz, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const float go = to_f32(dout[e]), zv = to_f32(z[e]), yv = to_f32(ypre[e]);
  const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-zv * 1.4426950408889634f));
  dy[e] = from_f32<T>(go * zv * sg);
  dz[e] = from_f32<T>(go * yv * sg * (1.f + zv * (1.f - sg)));
}

// ------------------------------------------------------------------ launchers
template <typename T, int P, int N, int HS>
static hipError_t launch_dxdb_hs(const BwdArgs& a, hipStream_t s) {
  const FwdArgs& f = a.f;
  const uint32_t nblocks = (uint32_t)f.B * f.nc * (f.Q / KT) * (f.H / HS);
  auto kern = bwd_dxdb_kernel<T, P, N, false, HS>;
  if constexpr (sizeof(T) == 4)
    if (f.cbT) kern = bwd_dxdb_kernel<T, P, N, true, HS>;  // fp32: C B^T read from the transposed blocks
  hipExtLaunchKernelGGL(kern, dim3(nblocks), dim3(256), 0, s, f.ev0, f.ev1, 0,
      static_cast<const T*>(f.x), static_cast<const T*>(f.Bm), static_cast<const T*>(f.Cm),
      static_cast<const T*>(a.dy), f.dtp, f.dAcs, a.gstates, f.cbT, f.D, static_cast<T*>(a.dx), a.dBh, a.ddir,
      a.dSa, a.Ub, a.pD, f.L, f.H, f.G, f.nc, f.Q, nblocks);
  return hipGetLastError();
}

template <typename T, int P, int N, int HS>
static hipError_t launch_dc_hs(const BwdArgs& a, hipStream_t s) {
  const FwdArgs& f = a.f;
  const uint32_t nblocks = (uint32_t)f.B * f.nc * (f.Q / KT) * (f.H / HS);
  auto kern = bwd_dc_kernel<T, P, N, false, HS>;
  if constexpr (sizeof(T) == 4)
    if (f.cb) kern = bwd_dc_kernel<T, P, N, true, HS>;     // fp32: C B^T read from the shared blocks
  hipExtLaunchKernelGGL(kern, dim3(nblocks),
      dim3(256), 0, s, f.ev0, f.ev1, 0,
      static_cast<const T*>(f.x), static_cast<const T*>(f.Bm), static_cast<const T*>(f.Cm),
      static_cast<const T*>(a.dy), f.dtp, f.dAcs, f.states, static_cast<const __bf16*>(f.prev16), f.cb, a.dCh,
      a.dSc, f.L, f.H, f.G, f.nc, f.Q, nblocks);
  return hipGetLastError();
}

// slices of 4 heads exist for bf16 inputs (fp32 keeps one head per workgroup)
template <typename T, int P, int N>
static hipError_t launch_dxdb_impl(const BwdArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2)
    if (a.hs_dxdb == 4) return launch_dxdb_hs<T, P, N, 4>(a, s);
  return a.hs_dxdb == 1 ? launch_dxdb_hs<T, P, N, 1>(a, s) : hipErrorInvalidValue;
}

template <typename T, int P, int N>
static hipError_t launch_dc_impl(const BwdArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2)
    if (a.hs_dc == 4) return launch_dc_hs<T, P, N, 4>(a, s);
  return a.hs_dc == 1 ? launch_dc_hs<T, P, N, 1>(a, s) : hipErrorInvalidValue;
}

template <typename T, int P, int N>
static hipError_t launch_finalize_impl(const BwdArgs& a, hipStream_t s) {
  const FwdArgs& f = a.f;
  const uint32_t nblocks = (uint32_t)f.B * f.nc * f.H;
  hipExtLaunchKernelGGL(bwd_finalize_kernel<T, P, N>, dim3(nblocks), dim3(256), 0, s, f.ev0, f.ev1, 0,
      static_cast<const T*>(f.dt), f.dt_bias, f.A, f.dtp, f.dAcs, f.states, a.gstates, a.ddir, a.dSa, a.dSc, a.Ub,
      static_cast<T*>(a.ddt), a.pA, a.pbias, f.L, f.H, f.nc, f.Q, f.clamp, f.dt_lo, f.dt_hi);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_reduce_impl(const BwdArgs& a, hipStream_t s) {
  const FwdArgs& f = a.f;
  const size_t total = (size_t)f.B * f.L * f.G * f.N;
  // the start event goes with the first launch and the stop event with the second
  hipEvent_t start = f.ev0;
  if (total > 0) {
    const size_t total4 = total / 4;                // N is a multiple of 16
    hipExtLaunchKernelGGL(bwd_reduce_bc_kernel<T>, dim3((unsigned)((total4 + 255) / 256)), dim3(256), 0, s, start,
                          nullptr, 0, a.dBh, a.dCh, static_cast<T*>(a.dB), static_cast<T*>(a.dC), f.H, f.G, f.N,
                          total4, f.H / a.hs_dxdb, f.H / a.hs_dc);
    start = nullptr;
  }
  hipExtLaunchKernelGGL(bwd_reduce_params_kernel, dim3(f.H), dim3(256), 0, s, start, f.ev1, 0, a.pA, a.pbias, a.pD,
                        a.dA, a.ddt_bias, a.dD, f.H, f.P, f.B * f.nc, f.B * f.nc * (f.Q / KT));
  return hipGetLastError();
}

hipError_t launch_bwd_dxdb(const BwdArgs& a, hipStream_t s) {
#define SSD_CASE(T, P_, N_) \
  if (a.f.dtype == SSD_DTYPE_CODE_##T && a.f.P == P_ && a.f.N == N_) return launch_dxdb_impl<T, P_, N_>(a, s);
  SSD_FOR_EACH_SHAPE(SSD_CASE)
#undef SSD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dc(const BwdArgs& a, hipStream_t s) {
#define SSD_CASE(T, P_, N_) \
  if (a.f.dtype == SSD_DTYPE_CODE_##T && a.f.P == P_ && a.f.N == N_) return launch_dc_impl<T, P_, N_>(a, s);
  SSD_FOR_EACH_SHAPE(SSD_CASE)
#undef SSD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_finalize(const BwdArgs& a, hipStream_t s) {
#define SSD_CASE(T, P_, N_) \
  if (a.f.dtype == SSD_DTYPE_CODE_##T && a.f.P == P_ && a.f.N == N_) return launch_finalize_impl<T, P_, N_>(a, s);
  SSD_FOR_EACH_SHAPE(SSD_CASE)
#undef SSD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_reduce(const BwdArgs& a, hipStream_t s) {
  return a.f.dtype == DT_F32 ? launch_reduce_impl<float>(a, s) : launch_reduce_impl<__bf16>(a, s);
}

hipError_t launch_gate_bwd(const GateArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;   // unreachable with a gate: a sequence has at least one token
  const unsigned nb = (unsigned)((a.n + 255) / 256);
  if (a.dtype == DT_F32)
    hipExtLaunchKernelGGL(gate_bwd_kernel<float>, dim3(nb), dim3(256), 0, s, a.ev0, a.ev1, 0,
                          static_cast<const float*>(a.dout), static_cast<const float*>(a.z),
                          static_cast<const float*>(a.ypre), static_cast<float*>(a.dy), static_cast<float*>(a.dz),
                          a.n);
  else
    hipExtLaunchKernelGGL(gate_bwd_kernel<__bf16>, dim3(nb), dim3(256), 0, s, a.ev0, a.ev1, 0,
                          static_cast<const __bf16*>(a.dout), static_cast<const __bf16*>(a.z),
                          static_cast<const __bf16*>(a.ypre), static_cast<__bf16*>(a.dy), static_cast<__bf16*>(a.dz),
                          a.n);
  return hipGetLastError();
}

}  // namespace ssd
