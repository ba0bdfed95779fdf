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
//   bwd_dxdb   per (b, c, 64-row block R, h): the anti-causal sums over row blocks I >= R
//   bwd_dc     per (b, c, R, h): the causal sums over row blocks J <= R
//   bwd_finalize per (b, c, h): dS, its reverse cumsum, d(dt), and the dA / d dt_bias partials
//   bwd_reduce_*: per-head dB, dC summed over the heads of each group; parameter partials
//                 summed in a fixed order (results are run-to-run deterministic)
//   gate_bwd:  dy = dout silu(z) and dz = dout y~ silu'(z)
// Tiles are staged in LDS as fp32 with an odd row pitch, so that both the row-broadcast
// and the column-stride reads of the 64 x 64 products are free of bank conflicts.  A
// thread (tr, tc) = (tid / 16, tid % 16) owns rows 4 tr .. 4 tr + 3 and the columns
// tc + 16 m of every 64-row product.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

namespace {
constexpr int KT = 64;   // tokens per tile (row block)
constexpr int KP = KT + 1;

// Stage `nvalid` token rows of width W (row stride `stride` elements) as fp32, zero rows after.
template <typename T, int W>
__device__ __forceinline__ void stage_rows(float* dst, const T* src, size_t stride, int nvalid, int tid) {
  constexpr int VEC = Vec16<T>::n, WV = W / VEC, UNITS = KT * WV, NIT = (UNITS + 255) / 256;
  Vec16<T> v[NIT];
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int u = min(tid + 256 * k, UNITS - 1);
    const int tok = u / WV, cv = (u % WV) * VEC;
    v[k] = load16_if(src + (size_t)(tok < nvalid ? tok : 0) * stride + cv, tok < nvalid);
  }
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int u = tid + 256 * k;
    if (u < UNITS) {
      const int tok = u / WV, cv = (u % WV) * VEC;
#pragma unroll
      for (int e = 0; e < VEC; ++e) dst[tok * (W + 1) + cv + e] = to_f32(v[k].v[e]);
    }
  }
}

// Stage a (P x N) fp32 state as rows of pitch N + 1.
template <int P, int N>
__device__ __forceinline__ void stage_state(float* dst, const float* src, int tid) {
  constexpr int UNITS = P * N / 4, NIT = (UNITS + 255) / 256;
  float4 v[NIT];
#pragma unroll
  for (int k = 0; k < NIT; ++k) v[k] = reinterpret_cast<const float4*>(src)[min(tid + 256 * k, UNITS - 1)];
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int u = tid + 256 * k;
    if (u < UNITS) {
      const int p = (4 * u) / N, n = (4 * u) % N;
      float* d = dst + p * (N + 1) + n;
      d[0] = v[k].x;
      d[1] = v[k].y;
      d[2] = v[k].z;
      d[3] = v[k].w;
    }
  }
}

// Sum over the 16 lanes of a row group (lanes 16 tr .. 16 tr + 15 of a wavefront).
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// 4 x 4 block of the product of two row sets over a shared width W:
// out[r][m] = sum_k A[(4 tr + r)][k] * Bt[(tc + 16 m)][k]   (both row-major, pitch W + 1)
template <int W>
__device__ __forceinline__ void rows_dot(float (&out)[4][4], const float* A, const float* Bt, int tr, int tc) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int m = 0; m < 4; ++m) out[r][m] = 0.f;
#pragma unroll 4
  for (int k = 0; k < W; ++k) {
    float a[4], b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = A[(4 * tr + r) * (W + 1) + k];
#pragma unroll
    for (int m = 0; m < 4; ++m) b[m] = Bt[(tc + 16 * m) * (W + 1) + k];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int m = 0; m < 4; ++m) out[r][m] += a[r] * b[m];
  }
}

// acc[r][m] += sum_k M[k][4 tr + r] * V[k][tc + 16 m]   (M pitch KP, V pitch W + 1), k < KT
template <int W>
__device__ __forceinline__ void acc_tn(float (&acc)[4][W / 16], const float* M, const float* V, int tr, int tc) {
#pragma unroll 4
  for (int k = 0; k < KT; ++k) {
    float a[4], b[W / 16];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = M[k * KP + 4 * tr + r];
#pragma unroll
    for (int m = 0; m < W / 16; ++m) b[m] = V[k * (W + 1) + tc + 16 * m];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int m = 0; m < W / 16; ++m) acc[r][m] += a[r] * b[m];
  }
}

// acc[r][m] += sum_k M[4 tr + r][k] * V[k][tc + 16 m]   (M pitch MP, V pitch W + 1), k < K
template <int K, int MP, int W>
__device__ __forceinline__ void acc_nn(float (&acc)[4][W / 16], const float* M, const float* V, int tr, int tc) {
#pragma unroll 4
  for (int k = 0; k < K; ++k) {
    float a[4], b[W / 16];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = M[(4 * tr + r) * MP + k];
#pragma unroll
    for (int m = 0; m < W / 16; ++m) b[m] = V[k * (W + 1) + tc + 16 * m];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int m = 0; m < W / 16; ++m) acc[r][m] += a[r] * b[m];
  }
}
}  // namespace

// ------------------------------------------------------------------ anti-causal: dx, dB
template <typename T, int P, int N>
__global__ __launch_bounds__(256) void bwd_dxdb_kernel(const T* __restrict__ x, const T* __restrict__ Bm,
                                                       const T* __restrict__ Cm, const T* __restrict__ dy,
                                                       const float* __restrict__ dtp, const float* __restrict__ dAcs,
                                                       const float* __restrict__ gstates,
                                                       const float* __restrict__ Dw, T* __restrict__ dx,
                                                       float* __restrict__ dBh, float* __restrict__ ddir,
                                                       float* __restrict__ dSa, float* __restrict__ Ub,
                                                       float* __restrict__ pD, int L, int H, int G, int nc, int Q,
                                                       uint32_t nblocks) {
  constexpr int PP = P + 1, NP = N + 1, TPm = P / 16, TNm = N / 16;
  __shared__ float s_b[KT * NP];                 // B of the own block R
  __shared__ float s_x[KT * PP];                 // x of R
  __shared__ float s_c[KT * NP];                 // C of block I; later Gnext (P x N)
  __shared__ float s_dy[KT * PP];                // dy of block I
  __shared__ float s_m1[KT * KP];                // e^(S_i - S_j) CB_ij   [i][j]
  __shared__ float s_m2[KT * KP];                // e^(S_i - S_j) DX_ij   [i][j]
  __shared__ float s_red[16 * KT];
  __shared__ float s_SR[KT], s_dR[KT], s_SI[KT];

  const int nrb = Q / KT;
  uint32_t id = xcd_swizzle(blockIdx.x, nblocks);
  const int h = id % H;
  id /= H;
  const int R = id % nrb;
  id /= nrb;
  const int c = id % nc, b = id / nc;
  const int g = h / (H / G);
  const int t0 = c * Q, len = min(Q, L - t0);
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  if (R * KT >= len) {                 // a row block past the end of the sequence: no rows,
    if (tid < P)                       // but its dD partial is still summed
      pD[(((size_t)b * nc + c) * nrb + R) * (size_t)(H * P) + (size_t)h * P + tid] = 0.f;
    return;
  }
  const int lenR = min(KT, len - R * KT);
  const size_t xs = (size_t)H * P, bs = (size_t)G * N;
  const size_t cq = (((size_t)b * H + h) * nc + c) * Q;
  const float Slast = dAcs[cq + Q - 1];

  stage_rows<T, N>(s_b, Bm + ((size_t)b * L + t0 + R * KT) * bs + (size_t)g * N, bs, lenR, tid);
  stage_rows<T, P>(s_x, x + ((size_t)b * L + t0 + R * KT) * xs + (size_t)h * P, xs, lenR, tid);
  if (tid < KT) {
    s_SR[tid] = dAcs[cq + R * KT + tid];
    s_dR[tid] = dtp[cq + R * KT + tid];
  }

  float xi[4][TPm], db[4][TNm], cs[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    cs[r] = 0.f;
#pragma unroll
    for (int m = 0; m < TPm; ++m) xi[r][m] = 0.f;
#pragma unroll
    for (int m = 0; m < TNm; ++m) db[r][m] = 0.f;
  }

  const int nI = (len + KT - 1) / KT;
  for (int I = R; I < nI; ++I) {
    const int lenI = min(KT, len - I * KT);
    __syncthreads();
    stage_rows<T, N>(s_c, Cm + ((size_t)b * L + t0 + I * KT) * bs + (size_t)g * N, bs, lenI, tid);
    stage_rows<T, P>(s_dy, dy + ((size_t)b * L + t0 + I * KT) * xs + (size_t)h * P, xs, lenI, tid);
    if (tid < KT) s_SI[tid] = dAcs[cq + I * KT + tid];
    __syncthreads();
    float cb[4][4], dxv[4][4];
    rows_dot<N>(cb, s_c, s_b, tr, tc);      // rows i of I, columns j of R
    rows_dot<P>(dxv, s_dy, s_x, tr, tc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * tr + r;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int j = tc + 16 * m;
        const bool ok = (I * KT + i >= R * KT + j) && i < lenI && j < lenR;
        const float e = ok ? expf(s_SI[i] - s_SR[j]) : 0.f;
        const float m1 = e * cb[r][m];
        cs[m] += m1 * dxv[r][m];
        s_m1[i * KP + j] = m1;
        s_m2[i * KP + j] = e * dxv[r][m];
      }
    }
    __syncthreads();
    acc_tn<P>(xi, s_m1, s_dy, tr, tc);      // xi[j][p] += sum_i m1[i][j] dy[i][p]
    acc_tn<N>(db, s_m2, s_c, tr, tc);       // db[j][n] += sum_i m2[i][j] C[i][n]
  }

  // carried terms through the gradient of the state leaving the chunk
  __syncthreads();
  stage_state<P, N>(s_c, gstates + (((size_t)b * nc + c) * H + h) * (size_t)(P * N), tid);
  // column partial sums of T (over this thread's rows i) -> per column j
#pragma unroll
  for (int m = 0; m < 4; ++m) s_red[tr * KT + tc + 16 * m] = cs[m];
  __syncthreads();
  float tmp[4][TPm];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int m = 0; m < TPm; ++m) tmp[r][m] = 0.f;
  // tmp[j][p] = sum_n B[j][n] Gnext[p][n]
#pragma unroll 4
  for (int n = 0; n < N; ++n) {
    float a[4], gv[TPm];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = s_b[(4 * tr + r) * NP + n];
#pragma unroll
    for (int m = 0; m < TPm; ++m) gv[m] = s_c[(tc + 16 * m) * NP + n];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int m = 0; m < TPm; ++m) tmp[r][m] += a[r] * gv[m];
  }
  float f[4], dj[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f[r] = expf(Slast - s_SR[4 * tr + r]);
    dj[r] = s_dR[4 * tr + r];
  }
  // db[j][n] += f_j sum_p x[j][p] Gnext[p][n]
  {
    float xg[4][TNm];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int m = 0; m < TNm; ++m) xg[r][m] = 0.f;
    acc_nn<P, PP, N>(xg, s_x, s_c, tr, tc);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int m = 0; m < TNm; ++m) db[r][m] += f[r] * xg[r][m];
  }
  float U[4], dd[4], dDp[TPm];
#pragma unroll
  for (int m = 0; m < TPm; ++m) dDp[m] = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = 4 * tr + r;
    float u = 0.f, q = 0.f;
#pragma unroll
    for (int m = 0; m < TPm; ++m) {
      const float xv = s_x[j * PP + tc + 16 * m];
      u += xv * tmp[r][m];
      xi[r][m] += f[r] * tmp[r][m];
      q += xv * xi[r][m];
    }
    U[r] = f[r] * dj[r] * sum16(u);
    dd[r] = sum16(q);
  }
  // outputs of the own block R
  const size_t row0 = (size_t)b * L + t0 + R * KT;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = 4 * tr + r;
    const bool ok = j < lenR;
    const size_t tok = row0 + (ok ? j : 0);
#pragma unroll
    for (int m = 0; m < TPm; ++m) {
      const int p = tc + 16 * m;
      const float dyv = ok ? to_f32(dy[tok * xs + (size_t)h * P + p]) : 0.f;
      const float dw = Dw ? Dw[(size_t)h * P + p] : 0.f;
      if (ok) dx[tok * xs + (size_t)h * P + p] = from_f32<T>(dw * dyv + dj[r] * xi[r][m]);
      dDp[m] += dyv * s_x[j * PP + p];
    }
    if (ok) {
#pragma unroll
      for (int m = 0; m < TNm; ++m) dBh[(tok * H + h) * (size_t)N + tc + 16 * m] = dj[r] * db[r][m];
    }
  }
  if (tc == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * tr + r;
      if (j < lenR) {
        float colsum = 0.f;
        for (int q = 0; q < 16; ++q) colsum += s_red[q * KT + j];
        colsum *= dj[r];
        ddir[cq + R * KT + j] = dd[r];
        dSa[cq + R * KT + j] = -colsum - U[r];
        Ub[cq + R * KT + j] = U[r];
      }
    }
  }
  // dD partial of this block: sum over the block's rows, per channel p
  __syncthreads();
#pragma unroll
  for (int m = 0; m < TPm; ++m) s_red[tr * KT + tc + 16 * m] = dDp[m];
  __syncthreads();
  if (tid < P) {
    float sD = 0.f;
    for (int q = 0; q < 16; ++q) sD += s_red[q * KT + tid];
    pD[(((size_t)b * nc + c) * nrb + R) * (size_t)(H * P) + (size_t)h * P + tid] = sD;
  }
}

// ------------------------------------------------------------------ causal: dC
template <typename T, int P, int N>
__global__ __launch_bounds__(256) void bwd_dc_kernel(const T* __restrict__ x, const T* __restrict__ Bm,
                                                     const T* __restrict__ Cm, const T* __restrict__ dy,
                                                     const float* __restrict__ dtp, const float* __restrict__ dAcs,
                                                     const float* __restrict__ states, float* __restrict__ dCh,
                                                     float* __restrict__ dSc, int L, int H, int G, int nc, int Q,
                                                     uint32_t nblocks) {
  constexpr int PP = P + 1, NP = N + 1, TNm = N / 16;
  __shared__ float s_c[KT * NP];                 // C of the own block R
  __shared__ float s_dy[KT * PP];                // dy of R
  __shared__ float s_b[KT * NP];                 // B of block J; later Hprev (P x N)
  __shared__ float s_x[KT * PP];                 // x of J
  __shared__ float s_w[KT * KP];                 // e^(S_i - S_j) d_j DX_ij   [i][j]
  __shared__ float s_SR[KT], s_SJ[KT], s_dJ[KT];

  const int nrb = Q / KT;
  uint32_t id = xcd_swizzle(blockIdx.x, nblocks);
  const int h = id % H;
  id /= H;
  const int R = id % nrb;
  id /= nrb;
  const int c = id % nc, b = id / nc;
  const int g = h / (H / G);
  const int t0 = c * Q, len = min(Q, L - t0);
  if (R * KT >= len) return;
  const int lenR = min(KT, len - R * KT);
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  const size_t xs = (size_t)H * P, bs = (size_t)G * N;
  const size_t cq = (((size_t)b * H + h) * nc + c) * Q;

  stage_rows<T, N>(s_c, Cm + ((size_t)b * L + t0 + R * KT) * bs + (size_t)g * N, bs, lenR, tid);
  stage_rows<T, P>(s_dy, dy + ((size_t)b * L + t0 + R * KT) * xs + (size_t)h * P, xs, lenR, tid);
  if (tid < KT) s_SR[tid] = dAcs[cq + R * KT + tid];

  float dc[4][TNm], rs[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    rs[r] = 0.f;
#pragma unroll
    for (int m = 0; m < TNm; ++m) dc[r][m] = 0.f;
  }
  for (int J = 0; J <= R; ++J) {
    const int lenJ = min(KT, len - J * KT);
    __syncthreads();
    stage_rows<T, N>(s_b, Bm + ((size_t)b * L + t0 + J * KT) * bs + (size_t)g * N, bs, lenJ, tid);
    stage_rows<T, P>(s_x, x + ((size_t)b * L + t0 + J * KT) * xs + (size_t)h * P, xs, lenJ, tid);
    if (tid < KT) {
      s_SJ[tid] = dAcs[cq + J * KT + tid];
      s_dJ[tid] = dtp[cq + J * KT + tid];
    }
    __syncthreads();
    float cb[4][4], dxv[4][4];
    rows_dot<N>(cb, s_c, s_b, tr, tc);       // rows i of R, columns j of J
    rows_dot<P>(dxv, s_dy, s_x, tr, tc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * tr + r;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int j = tc + 16 * m;
        const bool ok = (R * KT + i >= J * KT + j) && i < lenR && j < lenJ;
        const float w = ok ? expf(s_SR[i] - s_SJ[j]) * s_dJ[j] * dxv[r][m] : 0.f;
        rs[r] += w * cb[r][m];
        s_w[i * KP + j] = w;
      }
    }
    __syncthreads();
    acc_nn<KT, KP, N>(dc, s_w, s_b, tr, tc);  // dc[i][n] += sum_j w[i][j] B[j][n]
  }
  __syncthreads();
  stage_state<P, N>(s_b, states + (((size_t)b * nc + c) * H + h) * (size_t)(P * N), tid);
  __syncthreads();
  float cr[4][TNm];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int m = 0; m < TNm; ++m) cr[r][m] = 0.f;
  acc_nn<P, PP, N>(cr, s_dy, s_b, tr, tc);   // cr[i][n] = sum_p dy[i][p] Hprev[p][n]
  const size_t row0 = (size_t)b * L + t0 + R * KT;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * tr + r;
    const float ei = expf(s_SR[i]);
    float rr = 0.f;
#pragma unroll
    for (int m = 0; m < TNm; ++m) rr += cr[r][m] * s_c[i * NP + tc + 16 * m];
    rr = ei * sum16(rr);
    const float rsum = sum16(rs[r]);
    if (i < lenR) {
      const size_t tok = row0 + i;
#pragma unroll
      for (int m = 0; m < TNm; ++m) dCh[(tok * H + h) * (size_t)N + tc + 16 * m] = dc[r][m] + ei * cr[r][m];
      if (tc == 0) dSc[cq + R * KT + i] = rsum + rr;
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
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ dBh,
                                                            const float* __restrict__ dCh, T* __restrict__ dB,
                                                            T* __restrict__ dC, int H, int G, int N, size_t total) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;   // index into (B, L, G, N)
  if (e >= total) return;
  const int n = (int)(e % N);
  const size_t bg = e / N;
  const int g = (int)(bg % G);
  const size_t bl = bg / G;
  const int hpg = H / G;
  float sb = 0.f, sc = 0.f;
  for (int k = 0; k < hpg; ++k) {
    const size_t o = (bl * H + (size_t)g * hpg + k) * N + n;
    sb += dBh[o];
    sc += dCh[o];
  }
  dB[e] = from_f32<T>(sb);
  dC[e] = from_f32<T>(sc);
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
  if (dD && tid < P) {
    float sD = 0.f;
    for (int k = 0; k < nbr; ++k) sD += pD[((size_t)k * H + h) * P + tid];
    dD[(size_t)h * P + tid] = sD;
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
template <typename T, int P, int N>
static hipError_t launch_dxdb_impl(const BwdArgs& a, hipStream_t s) {
  const FwdArgs& f = a.f;
  const uint32_t nblocks = (uint32_t)f.B * f.nc * (f.Q / KT) * f.H;
  bwd_dxdb_kernel<T, P, N><<<nblocks, 256, 0, s>>>(
      static_cast<const T*>(f.x), static_cast<const T*>(f.Bm), static_cast<const T*>(f.Cm),
      static_cast<const T*>(a.dy), f.dtp, f.dAcs, a.gstates, f.D, static_cast<T*>(a.dx), a.dBh, a.ddir, a.dSa, a.Ub,
      a.pD, f.L, f.H, f.G, f.nc, f.Q, nblocks);
  return hipGetLastError();
}

template <typename T, int P, int N>
static hipError_t launch_dc_impl(const BwdArgs& a, hipStream_t s) {
  const FwdArgs& f = a.f;
  const uint32_t nblocks = (uint32_t)f.B * f.nc * (f.Q / KT) * f.H;
  bwd_dc_kernel<T, P, N><<<nblocks, 256, 0, s>>>(
      static_cast<const T*>(f.x), static_cast<const T*>(f.Bm), static_cast<const T*>(f.Cm),
      static_cast<const T*>(a.dy), f.dtp, f.dAcs, f.states, a.dCh, a.dSc, f.L, f.H, f.G, f.nc, f.Q, nblocks);
  return hipGetLastError();
}

template <typename T, int P, int N>
static hipError_t launch_finalize_impl(const BwdArgs& a, hipStream_t s) {
  const FwdArgs& f = a.f;
  const uint32_t nblocks = (uint32_t)f.B * f.nc * f.H;
  bwd_finalize_kernel<T, P, N><<<nblocks, 256, 0, s>>>(
      static_cast<const T*>(f.dt), f.dt_bias, f.A, f.dtp, f.dAcs, f.states, a.gstates, a.ddir, a.dSa, a.dSc, a.Ub,
      static_cast<T*>(a.ddt), a.pA, a.pbias, f.L, f.H, f.nc, f.Q, f.clamp, f.dt_lo, f.dt_hi);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_reduce_impl(const BwdArgs& a, hipStream_t s) {
  const FwdArgs& f = a.f;
  const size_t total = (size_t)f.B * f.L * f.G * f.N;
  if (total > 0)
    bwd_reduce_bc_kernel<T><<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
        a.dBh, a.dCh, static_cast<T*>(a.dB), static_cast<T*>(a.dC), f.H, f.G, f.N, total);
  bwd_reduce_params_kernel<<<f.H, 256, 0, s>>>(a.pA, a.pbias, a.pD, a.dA, a.ddt_bias, a.dD, f.H, f.P, f.B * f.nc,
                                               f.B * f.nc * (f.Q / KT));
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
  if (a.n == 0) return hipSuccess;
  const unsigned nb = (unsigned)((a.n + 255) / 256);
  if (a.dtype == DT_F32)
    gate_bwd_kernel<float><<<nb, 256, 0, s>>>(static_cast<const float*>(a.dout), static_cast<const float*>(a.z),
                                              static_cast<const float*>(a.ypre), static_cast<float*>(a.dy),
                                              static_cast<float*>(a.dz), a.n);
  else
    gate_bwd_kernel<__bf16><<<nb, 256, 0, s>>>(static_cast<const __bf16*>(a.dout), static_cast<const __bf16*>(a.z),
                                               static_cast<const __bf16*>(a.ypre), static_cast<__bf16*>(a.dy),
                                               static_cast<__bf16*>(a.dz), a.n);
  return hipGetLastError();
}

}  // namespace ssd
