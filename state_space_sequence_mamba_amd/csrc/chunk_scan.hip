// chunk_scan: the output of every position of a chunk,
//   y[i,p] = sum_{j<=i} CB[i,j] exp(dAcs[i] - dAcs[j]) dt'_j x[j,p]        (diagonal block)
//          + exp(dAcs[i]) sum_n C[i,n] Hprev[p,n]                            (carried state)
//          + D[p] x[i,p]                                                     (skip term)
// times silu(z[i,p]) when a gate is given, with CB[i,j] = sum_n C[i,n] B[j,n] and Hprev the
// state entering the chunk.
// Sources: "Agent 228: MAMBA-2 Reference Implementations Comparison", section 2.2 (the SSD
// output as a 1-semiseparable causal mask applied to attention-like C B^T scores) and
// section 3.2 (chunked evaluation: diagonal blocks plus the inter-chunk carry); "Agent 228:
// MAMBA-2 Implementation Gaps", Gap 1 (off-diagonal block from the previous state) and
// Gap 4 (D skip); the gate is the output gating of the reference-comparison page, 3.1.
//
// Per 16-row strip and 16-column causal sub-tile, CB^T (16x16) is contracted on MFMA and
// consumed at once by every head of the workgroup's head block: each head applies its decay
// exp(dAcs_i - dAcs_j) dt'_j and the causal mask in registers (CB^T, not CB, so that the MFMA
// result layout -- four consecutive columns of one row per lane -- is directly the A operand
// of the (L o CB) X product), then accumulates into its own (16 x P) tile.  On the diagonal
// sub-tile the x values a lane loads for that product are exactly its own output rows, so
// the D x skip term is added there without another read.  Contractions over dstate use the
// k permutation n = (N/4) qd + kk (fp32) so every lane reads 128 bits of LDS at a time; only
// consistency between the A and B operands matters for a sum over k.
//
// Two decompositions share these pieces:
//  * rows : one workgroup (4 wavefronts, one strip each) per 64-row block of a chunk and
//           head; each XCD takes a contiguous run of units in groups whose row blocks are
//           dispatched together (heaviest first), so that their re-reads of x and of the
//           entering state hit L2.  The default for both dtypes.
//  * chunk: one workgroup (8 wavefronts) per whole chunk and head block; wavefront w owns
//           the strip pair (w, S-1-w), S+1 sub-tiles each.  x, the carried state and y move
//           exactly once, but its registers allow one workgroup per CU.
// Token tiles (64 tokens of B and of x for every head) are loaded into registers one tile
// ahead of the MFMA work, then written to LDS.  y leaves through LDS as 16-byte row stores.
// Row blocks read C B^T precomputed once per group when chunk_state formed it (cb_block, in
// the A-operand lane order; always for fp32, for bf16 with many heads per group): each
// wavefront loads its own four sub-tiles of a column tile straight into registers, one tile
// ahead, with no LDS copy; the B tile is then not staged at all.
//
// MFMA: fp32 inputs -> v_mfma_f32_16x16x4_f32 for all three products; bf16 inputs ->
// 16x16x32 bf16 for C B^T and C Hprev^T, 16x16x16 bf16 for (L o CB) X.  Decay factors use
// the hardware base-2 exponential on log2(e)-scaled cumsums; factors below 2^-126 become 0.
// Below the diagonal the decay is split at each column tile's last position into a row
// factor and a per-column weight (both <= 1), so a lane takes one exponential per sub-tile.
#include "cb_tiles.h"
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kKT = 64;                       // tokens per staged tile == rows per row block
constexpr float kLog2e = 1.4426950408889634f;

template <int P> struct TPof { static constexpr int v = P / 16; };


template <typename T, int P, int N, int HB, int ROWS, bool NOB = false>
struct ScanLds {
  static constexpr bool F32 = sizeof(T) == 4;
  static constexpr int BP = N + (F32 ? 4 : 8);   // B tile / Hprev rows (n-contiguous), 16-byte rows
  static constexpr int XP = kKT + 4;              // x^T rows (token-contiguous)
  static constexpr int YP = P + (F32 ? 4 : 8);   // y staging rows
  // B tile (none when C B^T comes precomputed)
  static constexpr int B_ELEMS = NOB ? 0 : kKT * BP;
  static constexpr int X_ELEMS = HB * P * XP;
  static constexpr int PREV_ELEMS = P * BP;
  static constexpr int XU_ELEMS = X_ELEMS > PREV_ELEMS ? X_ELEMS : PREV_ELEMS;  // x tiles alias Hprev
  static constexpr int MAIN = B_ELEMS + XU_ELEMS;
  static constexpr int Y_ELEMS = ROWS * YP;                                      // y staging aliases both
  static constexpr int TOTAL = MAIN > Y_ELEMS ? MAIN : Y_ELEMS;
};

// One 64-token tile of B rows and of x for every head of the block, held in registers
// between its global loads and its LDS stores.  Loads read clamped in-bounds addresses and
// only record which tokens are real; the zeroing selects happen at store time, so nothing
// waits for the loads until the tile is written to LDS (after the current tile's MFMAs).
// PRECB: C B^T comes precomputed (each wavefront loads its own sub-tiles into registers), and
// the tile is x alone.

template <typename T, int P, int N, int HB, int NTHR, bool PRECB = false>
struct TileRegs {
  static constexpr int VEC = Vec16<T>::n;
  static constexpr int NVR = N / VEC, PV = P / VEC;
  static constexpr int BU = PRECB ? 0 : kKT * NVR;      // 16-byte vectors of B (none with PRECB)
  static constexpr int XU = HB * (kKT / 2) * PV;       // token-pair units of x
  // x unit order: for bf16 the 16-byte vectors of one token row sit on consecutive lanes, so
  // every load instruction reads whole rows (the transposing LDS stores then meet two-way bank
  // conflicts); for fp32 consecutive token pairs sit on consecutive lanes (conflict-free stores,
  // each load instruction touching 32 rows).  Measured: bf16 B8 L4096 H32 N128 169-172 us in
  // row order against 174-177 us; fp32 B4 L1024 H24 39-40 us in pair order against 40-42 us.
  static constexpr bool kXRows = sizeof(T) == 2;
  static constexpr int BPT = (BU + NTHR - 1) / NTHR, XPT = (XU + NTHR - 1) / NTHR;
  static_assert(BPT + 2 * XPT <= 32, "validity mask");
  Vec16<T> b[BPT > 0 ? BPT : 1];
  Vec16<T> x[XPT][2];
  uint32_t okm;

  __device__ __forceinline__ void load(const T* Bb, const T* xb, uint32_t bc_tok, uint32_t x_tok, int J, int len,
                                       int tid) {
    okm = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const int v = min(tid + NTHR * u, BU - 1);
      const int i = v / NVR, nv = (v % NVR) * VEC;
      const int tok = J * kKT + i;
      const bool ok = tok < len;
      b[u] = load16(Bb + (uint32_t)(ok ? tok : 0) * bc_tok + nv);
      okm |= (uint32_t)ok << u;
    }
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int v = min(tid + NTHR * u, XU - 1);
      const int m = kXRows ? (v / PV) % (kKT / 2) : v % (kKT / 2);
      const int pv = (kXRows ? v % PV : (v / (kKT / 2)) % PV) * VEC;
      const int hh = kXRows ? v / (PV * (kKT / 2)) : v / ((kKT / 2) * PV);
      const int tok = J * kKT + 2 * m;
      const bool ok0 = tok < len, ok1 = tok + 1 < len;
      const T* src = xb + hh * P + pv;
      x[u][0] = load16(src + (uint32_t)(ok0 ? tok : 0) * x_tok);
      x[u][1] = load16(src + (uint32_t)(ok1 ? tok + 1 : 0) * x_tok);
      okm |= ((uint32_t)ok0 << (BPT + 2 * u)) | ((uint32_t)ok1 << (BPT + 2 * u + 1));
    }
  }
  // B rows n-contiguous; x^T token-contiguous, one packed pair of consecutive tokens per store
  template <int BP, int XP>
  __device__ __forceinline__ void store(T* s_b, T* s_x, int tid) const {
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const int v = tid + NTHR * u;
      if (BU % NTHR == 0 || v < BU) {
        const int i = v / NVR, nv = (v % NVR) * VEC;
        *reinterpret_cast<Vec16<T>*>(&s_b[i * BP + nv]) = keep_if(b[u], (okm >> u) & 1u);
      }
    }
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int v = tid + NTHR * u;
      if (XU % NTHR == 0 || v < XU) {
        const int m = kXRows ? (v / PV) % (kKT / 2) : v % (kKT / 2);
        const int pv = (kXRows ? v % PV : (v / (kKT / 2)) % PV) * VEC;
        const int hh = kXRows ? v / (PV * (kKT / 2)) : v / ((kKT / 2) * PV);
        const Vec16<T> x0 = keep_if(x[u][0], (okm >> (BPT + 2 * u)) & 1u);
        const Vec16<T> x1 = keep_if(x[u][1], (okm >> (BPT + 2 * u + 1)) & 1u);
        T* dst = &s_x[(hh * P + pv) * XP + 2 * m];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          T pair[2] = {x0.v[e], x1.v[e]};
          __builtin_memcpy(dst + e * XP, pair, sizeof(pair));
        }
      }
    }
  }
};

// Stage the (P x N) state entering the chunk (already in T: fp32 states, or the bf16 copy
// state_passing writes for bf16 inputs) into LDS, n-contiguous rows.
template <typename T, int P, int N, int BP>
__device__ __forceinline__ void stage_prev(T* s_prev, const T* hp, int tid, int nthr) {
  constexpr int VEC = Vec16<T>::n;
  for (int v = tid; v < P * N / VEC; v += nthr) {
    const int p = (v * VEC) / N, n = (v * VEC) % N;
    *reinterpret_cast<Vec16<T>*>(&s_prev[p * BP + n]) = load16(hp + (size_t)p * N + n);
  }
}

// acc += exp(dAcs_i) * C_strip . Hprev^T   (Hprev staged in s_prev)
template <typename T, int P, int N, int BP>
__device__ __forceinline__ void carried_term(f32x4 (&acc)[TPof<P>::v], const typename NDot<T, N>::frag& cf,
                                             const T* s_prev, const float* s_da_h, int strip, int r, int qd) {
  typedef NDot<T, N> ND;
  constexpr int TP = P / 16;
  f32x4 t[TP];
#pragma unroll
  for (int pt = 0; pt < TP; ++pt) {
    typename ND::frag pf;
    ND::load(pf, &s_prev[(pt * 16 + r) * BP], qd);
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

// One causal 16x16 sub-tile (column tile jt, local index js in the staged tile) of one strip,
// for every head of the block.  EDGE: the sub-tile may be the diagonal one, whose columns past
// the diagonal are masked and which adds the skip term.
template <typename T, int P, int N, int HB, int BP, int XP, bool EDGE, bool PRECB>
__device__ __forceinline__ void sub_tile(f32x4 (&acc)[HB][TPof<P>::v], const typename NDot<T, N>::frag& cf,
                                         const float (&dco)[HB][TPof<P>::v], const T* s_b, const T* s_x,
                                         const float (*s_da)[256], const float (*s_dt)[256],
                                         const float (*s_w)[256], int strip, int jt, int js, int lstrip, int r,
                                         int qd, const f32x4& cbr) {
  typedef NDot<T, N> ND;
  constexpr int TP = P / 16;
  constexpr bool F32 = sizeof(T) == 4;
  const int i_row = 16 * strip + r;
  const bool diag = EDGE && jt == strip;
  // CB^T sub-tile: lane holds CB[i = 16 strip + r][j = 16 jt + 4 qd + e]
  f32x4 cbt;
  if constexpr (PRECB) {
    cbt = cbr;                                   // lane (r, qd) of sub-tile (lstrip, js)
  } else {
    typename ND::frag bfr;
    ND::load(bfr, &s_b[(js * 16 + r) * BP], qd);
    cbt = ND::dot(bfr, cf, zero4());
  }
  const int j0 = 16 * jt + 4 * qd;
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    float lw[4];
    if (diag) {
      // the diagonal sub-tile: the decay of each (i, j) on its own, then the causal mask (a
      // select, so an overflowed factor above the diagonal is dropped)
      const float da_i = s_da[hh][i_row];
      const float4 daj = *reinterpret_cast<const float4*>(&s_da[hh][j0]);
      const float4 dtj = *reinterpret_cast<const float4*>(&s_dt[hh][j0]);
      lw[0] = cbt[0] * __builtin_amdgcn_exp2f(da_i - daj.x) * dtj.x;
      lw[1] = cbt[1] * __builtin_amdgcn_exp2f(da_i - daj.y) * dtj.y;
      lw[2] = cbt[2] * __builtin_amdgcn_exp2f(da_i - daj.z) * dtj.z;
      lw[3] = cbt[3] * __builtin_amdgcn_exp2f(da_i - daj.w) * dtj.w;
      if (EDGE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) lw[e] = (j0 + e <= i_row) ? lw[e] : 0.f;
      }
    } else {
      // below the diagonal every j precedes every i: the decay splits at c, the tile's last
      // column, into a row factor exp2(dAcs_i - dAcs_c) and the column weight
      // W_j = exp2(dAcs_c - dAcs_j) dt'_j (both factors <= 1: no overflow), one exponential per
      // lane instead of four
      const float ri = __builtin_amdgcn_exp2f(s_da[hh][i_row] - s_da[hh][16 * jt + 15]);
      const float4 wj = *reinterpret_cast<const float4*>(&s_w[hh][j0]);
      lw[0] = cbt[0] * wj.x * ri;
      lw[1] = cbt[1] * wj.y * ri;
      lw[2] = cbt[2] * wj.z * ri;
      lw[3] = cbt[3] * wj.w * ri;
    }
    const T* xt = &s_x[(hh * P + r) * XP + js * 16 + 4 * qd];
    if (F32) {
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        const float4 xv = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(xt) + pt * 16 * XP);
        acc[hh][pt] = mfma_16x16x4_f32(lw[0], xv.x, acc[hh][pt]);
        acc[hh][pt] = mfma_16x16x4_f32(lw[1], xv.y, acc[hh][pt]);
        acc[hh][pt] = mfma_16x16x4_f32(lw[2], xv.z, acc[hh][pt]);
        acc[hh][pt] = mfma_16x16x4_f32(lw[3], xv.w, acc[hh][pt]);
        if (diag) {  // x rows 16 jt + 4 qd + e are this lane's output rows
          acc[hh][pt][0] += dco[hh][pt] * xv.x;
          acc[hh][pt][1] += dco[hh][pt] * xv.y;
          acc[hh][pt][2] += dco[hh][pt] * xv.z;
          acc[hh][pt][3] += dco[hh][pt] * xv.w;
        }
      }
    } else {
      bf16x4 a;
      a[0] = static_cast<__bf16>(lw[0]);
      a[1] = static_cast<__bf16>(lw[1]);
      a[2] = static_cast<__bf16>(lw[2]);
      a[3] = static_cast<__bf16>(lw[3]);
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        const bf16x4 xv = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(xt) + pt * 16 * XP);
        acc[hh][pt] = mfma_16x16x16_bf16(a, xv, acc[hh][pt]);
        if (diag) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[hh][pt][e] += dco[hh][pt] * static_cast<float>(xv[e]);
        }
      }
    }
  }
}

// Diagonal-block contributions of staged tile J to one strip: its causal sub-tiles, the one
// on the diagonal masked and carrying the skip term.
template <typename T, int P, int N, int HB, int BP, int XP, bool PRECB = false>
__device__ __forceinline__ void diag_tile(f32x4 (&acc)[HB][TPof<P>::v], const typename NDot<T, N>::frag& cf,
                                          const float (&dco)[HB][TPof<P>::v], const T* s_b, const T* s_x,
                                          const float (*s_da)[256], const float (*s_dt)[256],
                                          const float (*s_w)[256], int strip, int J, int lstrip, int r, int qd,
                                          const f32x4 (&cbr)[4]) {
#pragma unroll
  for (int js = 0; js < 4; ++js) {
    const int jt = 4 * J + js;
    if (jt > strip) break;
    sub_tile<T, P, N, HB, BP, XP, true, PRECB>(acc, cf, dco, s_b, s_x, s_da, s_dt, s_w, strip, jt, js, lstrip, r,
                                               qd, cbr[js]);
  }
}

// Staged tile J entirely below the diagonal of one strip (4 J + 3 < strip): four unmasked
// sub-tiles in one straight-line block, so the LDS reads of one sub-tile overlap the MFMAs of
// the one before.
template <typename T, int P, int N, int HB, int BP, int XP, bool PRECB = false>
__device__ __forceinline__ void full_tile(f32x4 (&acc)[HB][TPof<P>::v], const typename NDot<T, N>::frag& cf,
                                          const float (&dco)[HB][TPof<P>::v], const T* s_b, const T* s_x,
                                          const float (*s_da)[256], const float (*s_dt)[256],
                                          const float (*s_w)[256], int strip, int J, int lstrip, int r, int qd,
                                          f32x4 (&cbr)[4], const float* cb_next) {
#pragma unroll
  for (int js = 0; js < 4; ++js) {
    sub_tile<T, P, N, HB, BP, XP, false, PRECB>(acc, cf, dco, s_b, s_x, s_da, s_dt, s_w, strip, 4 * J + js, js,
                                                lstrip, r, qd, cbr[js]);
    // the next block's sub-tile into the register this one has just released
    if constexpr (PRECB) cbr[js] = *reinterpret_cast<const f32x4*>(cb_next + 256 * js);
  }
}

// Output gate y * silu(z) on one strip's registers (rows 16 strip + 4 qd + e, column 16 pt + r).
// All z loads are issued before use; rows past the sequence read a clamped address.
template <typename T, int P, int HB>
__device__ __forceinline__ void apply_gate(f32x4 (&acc)[HB][TPof<P>::v], const T* z, size_t row0, size_t x_tok,
                                           int h0, int strip, int len, int r, int qd) {
  constexpr int TP = P / 16;
  float zv[HB][TP][4];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * strip + 4 * qd + e;
        const size_t o = (row0 + (i < len ? i : 0)) * x_tok + (size_t)(h0 + hh) * P + pt * 16 + r;
        zv[hh][pt][e] = to_f32(z[o]);
      }
#pragma unroll
  for (int hh = 0; hh < HB; ++hh)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[hh][pt][e] *= silu(zv[hh][pt][e]);
}

// Write one strip's (16 x P) results of head hh into the y staging rows.
template <typename T, int P, int HB, int YP>
__device__ __forceinline__ void put_strip(T* s_y, const f32x4 (&acc)[HB][TPof<P>::v], int hh, int lstrip, int r,
                                          int qd) {
#pragma unroll
  for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_y[(16 * lstrip + 4 * qd + e) * YP + pt * 16 + r] = from_f32<T>(acc[hh][pt][e]);
}

// Copy staged rows [0, rows) of y (head h) to global memory as 16-byte row segments.
template <typename T, int P, int YP>
__device__ __forceinline__ void flush_rows(T* y, const T* s_y, size_t row0, size_t x_tok, int h, int rows,
                                           int tid, int nthr) {
  constexpr int VEC = Vec16<T>::n, PV = P / VEC;
  for (int v = tid; v < rows * PV; v += nthr) {
    const int i = v / PV, cv = (v % PV) * VEC;
    *reinterpret_cast<uint4*>(y + (row0 + i) * x_tok + (size_t)h * P + cv) =
        *reinterpret_cast<const uint4*>(&s_y[i * YP + cv]);
  }
}

// The chunk's dt' and (log2e-scaled) cumsum of HB heads, and head 0's entering state, held in
// registers from their loads to their LDS stores, so that every global load of a workgroup's
// prologue is in flight at once (one memory latency instead of one per phase).
// Every slot i < 256 of every head is written (positions past Q repeat position Q - 1 and are
// never read), so neither the loads nor the stores sit behind a branch: a conditional store
// lets the compiler sink its load into the branch and wait for it there.
// Column weights of the below-diagonal sub-tiles, W_j = exp2(dAcs_c - dAcs_j) dt'_j with c the
// last column of j's 16-column tile (c = j | 15), for every slot of every head of the block.
template <typename T, int HB, int NTHR>
__device__ __forceinline__ void column_weights(float (*s_w)[256], const float (*s_da)[256],
                                               const float (*s_dt)[256], int tid) {
#pragma unroll
  for (int hh = 0; hh < HB; ++hh)
    for (int i = tid; i < 256; i += NTHR)
      s_w[hh][i] = __builtin_amdgcn_exp2f(s_da[hh][i | 15] - s_da[hh][i]) * s_dt[hh][i];
}

template <int HB, int NTHR>
struct ScalarRegs {
  static constexpr int K = (256 + NTHR - 1) / NTHR;
  float da[HB][K], dt[HB][K];
  __device__ __forceinline__ void load(const float* dtp, const float* dAcs, int b, int H, int h0, int nc, int c,
                                       int Q, int tid) {
#pragma unroll
    for (int hh = 0; hh < HB; ++hh)
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int i = min(tid + NTHR * k, Q - 1);
        const size_t off = (((size_t)b * H + h0 + hh) * nc + c) * Q + i;
        dt[hh][k] = dtp[off];
        da[hh][k] = dAcs[off];
      }
  }
  __device__ __forceinline__ void store(float (*s_da)[256], float (*s_dt)[256], int tid) const {
#pragma unroll
    for (int hh = 0; hh < HB; ++hh)
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int i = tid + NTHR * k;
        if (NTHR * K == 256 || i < 256) {
          s_dt[hh][i] = dt[hh][k];
          s_da[hh][i] = da[hh][k] * kLog2e;
        }
      }
  }
};

template <typename T, int P, int N, int NTHR>
struct PrevRegs {
  static constexpr int VEC = Vec16<T>::n;
  static constexpr int U = P * N / VEC, K = (U + NTHR - 1) / NTHR;
  Vec16<T> v[K];
  __device__ __forceinline__ void load(const T* hp, int tid) {
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = load16(hp + (size_t)min(tid + NTHR * k, U - 1) * VEC);
  }
  template <int BP>
  __device__ __forceinline__ void store(T* s_prev, int tid) const {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int u = tid + NTHR * k;
      if (U % NTHR == 0 || u < U) {              // compile-time true for most instantiated shapes
        const int p = (VEC * u) / N, n = (VEC * u) % N;
        *reinterpret_cast<Vec16<T>*>(&s_prev[p * BP + n]) = v[k];
      }
    }
  }
};

// ---------------------------------------------------------------- row-block decomposition
template <typename T, int P, int N, int HB, bool PRECB>
__global__ __launch_bounds__(256, HB == 1 ? (sizeof(T) == 2 && PRECB && N >= 128 ? 5 : 4) : 2) void chunk_scan_rows_kernel(const T* __restrict__ x,
                                                                 const T* __restrict__ Bm,
                                                                 const float* __restrict__ cbp,
                                                                 const T* __restrict__ Cm,
                                                                 const float* __restrict__ dtp,
                                                                 const float* __restrict__ dAcs,
                                                                 const T* __restrict__ states,
                                                                 const float* __restrict__ Dw,
                                                                 const T* __restrict__ Z,
                                                                 T* __restrict__ y,
                                                                 int L, int H, int G, int nc, int Q, int B,
                                                                 int group_units) {
  constexpr int NTHR = 256;
  // PRECB: C B^T sub-tiles come precomputed, straight into each wavefront's registers
  typedef ScanLds<T, P, N, HB, kKT, PRECB> SL;
  typedef NDot<T, N> ND;
  constexpr int TP = P / 16;

  __shared__ __attribute__((aligned(16))) T s_mem[SL::TOTAL];
  __shared__ __attribute__((aligned(16))) float s_da[HB][256];     // dAcs * log2(e)
  __shared__ __attribute__((aligned(16))) float s_dt[HB][256];
  __shared__ __attribute__((aligned(16))) float s_w[HB][256];     // column weights
  T* s_b = s_mem;
  T* s_xu = s_mem + SL::B_ELEMS;                                   // Hprev, then x^T tiles
  T* s_y = s_mem;                                                  // y staging, at the end

  // work unit: row-block class (heaviest first), then XCD-local (b, c, head block)
  const int nrb = Q / kKT;
  const int nhb = H / HB;
  const uint32_t U = (uint32_t)B * nc * nhb;          // units per row-block class
  const uint32_t hw = blockIdx.x;
  uint32_t cls, unit;
  if ((U & 7u) == 0 && group_units > 0) {
    // every XCD a contiguous run of units, taken in groups of group_units whose row blocks
    // are dispatched together (heaviest class first within the group): the group's row blocks
    // share their x tiles and entering states in that XCD's L2
    const uint32_t per = U >> 3, seq = hw >> 3, k = (uint32_t)group_units;
    const uint32_t gi = seq / (nrb * k), gsize = min(k, per - gi * k), pos = seq - gi * nrb * k;
    cls = pos / gsize;
    unit = (hw & 7u) * per + gi * k + pos % gsize;
  } else if ((U & 7u) == 0) {
    // heaviest row blocks first, every XCD an equal share of each class
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

  const size_t bc_tok = (size_t)G * N, x_tok = (size_t)H * P;
  const T* Cb = Cm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  // PRECB: the C B^T sub-tiles of this row block come precomputed (once per group) by cb_block
  const T* Bb = PRECB ? reinterpret_cast<const T*>(cbp + (((size_t)b * nc + c) * G + g) *
                                                             (size_t)(nrb * (nrb + 1) / 2) * kCbBlock +
                                                   (size_t)(rb * (rb + 1) / 2) * kCbBlock)
                      : Bm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  const T* xb = x + ((size_t)b * L + t0) * x_tok + (size_t)h0 * P;

  // prologue: every global load in flight before the first wait, those of the carried term
  // first: loads complete in order, so the carried term's MFMAs need not wait for tile 0.
  // C rows past the sequence read row 0 unmasked: they only reach output rows that are
  // never stored.
  ScalarRegs<HB, NTHR> sr;
  sr.load(dtp, dAcs, b, H, h0, nc, c, Q, tid);
  PrevRegs<T, P, N, NTHR> pr;
  pr.load(states + (((size_t)b * nc + c) * H + h0) * (size_t)(P * N), tid);
  typename ND::frag cf;
  {
    const int i = 16 * s + r;
    ND::load(cf, Cb + (size_t)(i < len ? i : 0) * bc_tok, qd);
  }
  float dco[HB][TP];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) dco[hh][pt] = Dw ? Dw[(size_t)(h0 + hh) * P + pt * 16 + r] : 0.f;
  TileRegs<T, P, N, HB, NTHR, PRECB> tr;
  tr.load(Bb, xb, (uint32_t)bc_tok, (uint32_t)x_tok, 0, len, tid);
  // this wavefront's four C B^T sub-tiles of block (rb, 0), in the lane order cb_block wrote
  const float* cb_lane = reinterpret_cast<const float*>(Bb) + ((size_t)(wave * 4) * 64 + lane) * 4;
  f32x4 cbr[4] = {};
  if constexpr (PRECB) {
#pragma unroll
    for (int js = 0; js < 4; ++js) cbr[js] = *reinterpret_cast<const f32x4*>(cb_lane + 256 * js);
  }

  f32x4 acc[HB][TP];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) acc[hh][pt] = zero4();

  sr.store(s_da, s_dt, tid);
  pr.template store<SL::BP>(s_xu, tid);
  __syncthreads();
  column_weights<T, HB, NTHR>(s_w, s_da, s_dt, tid);          // read after the J loop's first barrier
  if (strip_ok) carried_term<T, P, N, SL::BP>(acc[0], cf, s_xu, s_da[0], s, r, qd);
#pragma unroll
  for (int hh = 1; hh < HB; ++hh) {
    __syncthreads();
    stage_prev<T, P, N, SL::BP>(s_xu, states + (((size_t)b * nc + c) * H + h0 + hh) * (size_t)(P * N), tid, NTHR);
    __syncthreads();
    if (strip_ok) carried_term<T, P, N, SL::BP>(acc[hh], cf, s_xu, s_da[hh], s, r, qd);
  }
  for (int J = 0; J <= rb; ++J) {
    __syncthreads();
    tr.template store<SL::BP, SL::XP>(s_b, s_xu, tid);
    if (J < rb) tr.load(Bb, xb, (uint32_t)bc_tok, (uint32_t)x_tok, J + 1, len, tid);
    __syncthreads();
    if (strip_ok) {
      if (J < rb)
        full_tile<T, P, N, HB, SL::BP, SL::XP, PRECB>(acc, cf, dco, s_b, s_xu, s_da, s_dt, s_w, s, J, wave, r, qd,
                                                      cbr, cb_lane + (size_t)(J + 1) * kCbBlock);
      else
        diag_tile<T, P, N, HB, SL::BP, SL::XP, PRECB>(acc, cf, dco, s_b, s_xu, s_da, s_dt, s_w, s, J, wave, r, qd,
                                                      cbr);
    }
  }
  if (Z && strip_ok) apply_gate<T, P, HB>(acc, Z, (size_t)b * L + t0, x_tok, h0, s, len, r, qd);
  const int rows = min(kKT, len - rb * kKT);
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    __syncthreads();
    if (strip_ok) put_strip<T, P, HB, SL::YP>(s_y, acc, hh, wave, r, qd);
    __syncthreads();
    flush_rows<T, P, SL::YP>(y, s_y, (size_t)b * L + t0 + rb * kKT, x_tok, h0 + hh, rows, tid, NTHR);
  }
}

// ---------------------------------------------------------------- whole-chunk decomposition
template <typename T, int P, int N, int HB>
__global__ __launch_bounds__(512) void chunk_scan_chunk_kernel(const T* __restrict__ x,
                                                               const T* __restrict__ Bm,
                                                               const T* __restrict__ Cm,
                                                               const float* __restrict__ dtp,
                                                               const float* __restrict__ dAcs,
                                                               const T* __restrict__ states,
                                                               const float* __restrict__ Dw,
                                                               const T* __restrict__ Z,
                                                               T* __restrict__ y,
                                                               int L, int H, int G, int nc, int Q, uint32_t nblocks) {
  constexpr int NTHR = 512;
  typedef ScanLds<T, P, N, HB, 256> SL;
  typedef NDot<T, N> ND;
  constexpr int TP = P / 16;

  __shared__ __attribute__((aligned(16))) T s_mem[SL::TOTAL];
  __shared__ __attribute__((aligned(16))) float s_da[HB][256];
  __shared__ __attribute__((aligned(16))) float s_dt[HB][256];
  __shared__ __attribute__((aligned(16))) float s_w[HB][256];
  T* s_b = s_mem;
  T* s_xu = s_mem + SL::B_ELEMS;
  T* s_y = s_mem;

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

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, qd = lane >> 4;
  const bool active = wave < (S >> 1);                  // wavefronts past Q/32 only stage data
  int strip[2];
  strip[0] = wave;                                      // short strip
  strip[1] = S - 1 - wave;                              // long strip
  bool ok[2];
  ok[0] = active && 16 * strip[0] < len;
  ok[1] = active && 16 * strip[1] < len;

  const size_t bc_tok = (size_t)G * N, x_tok = (size_t)H * P;
  const T* Cb = Cm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  const T* Bb = Bm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  const T* xb = x + ((size_t)b * L + t0) * x_tok + (size_t)h0 * P;

  // prologue: every global load in flight before the first wait, those of the carried term
  // first (as in the row-block kernel)
  ScalarRegs<HB, NTHR> sr;
  sr.load(dtp, dAcs, b, H, h0, nc, c, Q, tid);
  PrevRegs<T, P, N, NTHR> pr;
  pr.load(states + (((size_t)b * nc + c) * H + h0) * (size_t)(P * N), tid);
  typename ND::frag cf[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int i = 16 * strip[st] + r;
    const bool in = active && i < len;
    ND::load(cf[st], Cb + (size_t)(in ? i : 0) * bc_tok, qd);
  }
  float dco[HB][TP];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) dco[hh][pt] = Dw ? Dw[(size_t)(h0 + hh) * P + pt * 16 + r] : 0.f;
  TileRegs<T, P, N, HB, NTHR> tr;
  tr.load(Bb, xb, (uint32_t)bc_tok, (uint32_t)x_tok, 0, len, tid);

  f32x4 acc[2][HB][TP];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int hh = 0; hh < HB; ++hh)
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) acc[st][hh][pt] = zero4();

  sr.store(s_da, s_dt, tid);
  pr.template store<SL::BP>(s_xu, tid);
  __syncthreads();
  column_weights<T, HB, NTHR>(s_w, s_da, s_dt, tid);          // read after the J loop's first barrier
#pragma unroll
  for (int st = 0; st < 2; ++st)
    if (ok[st]) carried_term<T, P, N, SL::BP>(acc[st][0], cf[st], s_xu, s_da[0], strip[st], r, qd);
#pragma unroll
  for (int hh = 1; hh < HB; ++hh) {
    __syncthreads();
    stage_prev<T, P, N, SL::BP>(s_xu, states + (((size_t)b * nc + c) * H + h0 + hh) * (size_t)(P * N), tid, NTHR);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 2; ++st)
      if (ok[st]) carried_term<T, P, N, SL::BP>(acc[st][hh], cf[st], s_xu, s_da[hh], strip[st], r, qd);
  }
  const int ntiles = (len + kKT - 1) / kKT;
  f32x4 no_cb[4] = {};                                  // (C B^T is formed here, not read)
  for (int J = 0; J < ntiles; ++J) {
    __syncthreads();
    tr.template store<SL::BP, SL::XP>(s_b, s_xu, tid);
    if (J + 1 < ntiles) tr.load(Bb, xb, (uint32_t)bc_tok, (uint32_t)x_tok, J + 1, len, tid);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (ok[st] && 4 * J + 3 < strip[st])
        full_tile<T, P, N, HB, SL::BP, SL::XP>(acc[st], cf[st], dco, s_b, s_xu, s_da, s_dt, s_w, strip[st], J, 0, r,
                                               qd, no_cb, nullptr);
      else if (ok[st] && 4 * J <= strip[st])
        diag_tile<T, P, N, HB, SL::BP, SL::XP>(acc[st], cf[st], dco, s_b, s_xu, s_da, s_dt, s_w, strip[st], J, 0, r,
                                               qd, no_cb);
    }
  }
  if (Z) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
      if (ok[st]) apply_gate<T, P, HB>(acc[st], Z, (size_t)b * L + t0, x_tok, h0, strip[st], len, r, qd);
  }
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 2; ++st)
      if (ok[st]) put_strip<T, P, HB, SL::YP>(s_y, acc[st], hh, strip[st], r, qd);
    __syncthreads();
    flush_rows<T, P, SL::YP>(y, s_y, (size_t)b * L + t0, x_tok, h0 + hh, len, tid, NTHR);
  }
}

template <typename T, int P, int N, int HB>
static hipError_t launch_scan_hb(const FwdArgs& a, hipStream_t s) {
  const T* prevT = sizeof(T) == 4 ? reinterpret_cast<const T*>(a.states) : static_cast<const T*>(a.prev16);
  if (a.scan_variant == 2) {
    const uint32_t nblocks = (uint32_t)a.B * a.nc * (a.H / HB);
    hipExtLaunchKernelGGL(chunk_scan_chunk_kernel<T, P, N, HB>, dim3(nblocks), dim3(512), 0, s, a.ev0, a.ev1, 0,
        static_cast<const T*>(a.x), static_cast<const T*>(a.Bm), static_cast<const T*>(a.Cm), a.dtp, a.dAcs,
        prevT, a.D, static_cast<const T*>(a.z), static_cast<T*>(a.y), a.L, a.H, a.G, a.nc, a.Q, nblocks);
  } else {
    const uint32_t nblocks = (uint32_t)a.B * a.nc * (a.H / HB) * (a.Q / kKT);
    // C B^T precomputed whenever chunk_state formed it (always for fp32)
    auto kern = chunk_scan_rows_kernel<T, P, N, HB, true>;
    if constexpr (sizeof(T) == 4) {
      if (!a.cb) return hipErrorInvalidValue;
    } else {
      if (!a.cb) kern = chunk_scan_rows_kernel<T, P, N, HB, false>;
    }
    hipExtLaunchKernelGGL(kern, dim3(nblocks), dim3(256), 0, s, a.ev0, a.ev1, 0,
        static_cast<const T*>(a.x), static_cast<const T*>(a.Bm), a.cb, static_cast<const T*>(a.Cm), a.dtp, a.dAcs,
        prevT, a.D, static_cast<const T*>(a.z), static_cast<T*>(a.y), a.L, a.H, a.G, a.nc, a.Q, a.B,
        a.rows_group);
  }
  return hipGetLastError();
}

template <typename T, int P, int N>
static hipError_t launch_scan_impl(const FwdArgs& a, hipStream_t s) {
  // instantiated head-block sizes: 1 and 2 (larger blocks need more registers than they save)
  return a.heads_per_block == 2 ? launch_scan_hb<T, P, N, 2>(a, s) : launch_scan_hb<T, P, N, 1>(a, s);
}

hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t s) {
  if (a.scan_variant == 3) return launch_chunk_scan_group(a, a.heads_per_block, s);
#define SSD_CASE(T, P_, N_) \
  if (a.dtype == SSD_DTYPE_CODE_##T && a.P == P_ && a.N == N_) return launch_scan_impl<T, P_, N_>(a, s);
  SSD_FOR_EACH_SHAPE(SSD_CASE)
#undef SSD_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
