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
// chunk: dt' and the in-chunk cumsum of dt' A for every head of the slice (wavefront hh: a DPP
// prefix scan over 64 lanes), written to the workspace for chunk_scan;
// B staged once in LDS for all the slice's heads; each wavefront owns a 32 x 32 block of S^T and
// holds its 32 dstate rows of B^T in registers for the chunk.  Per head: x times the token weights staged in LDS, L_c written
// (rounded to bf16) unless c opens the segment, the state scaled by the chunk's decay and the
// chunk's B^T diag(w) x added on 16x16x32 bf16 MFMA, the state of each head held in the
// accumulators of the whole segment.  B and x stay token-major in LDS (16 x 16 tiles, 16-byte
// stores) and reach the MFMA through transpose reads (ds_read_b64_tr_b16); the state is formed
// transposed (S^T[n][p]), so each lane holds four consecutive dstate values of one headdim row
// and L_c and E_s leave as 8- and 16-byte row stores.  The next chunk's B and dt are loaded into
// registers while the current ones are in use, and the next head's x in parts between the
// MFMAs.  At the segment's end E_s goes out in fp32 with the segment's total exponent; D_c goes
// out for every chunk.
#include <type_traits>
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kSQ = 256;                       // chunk length
constexpr int kSThreads = 512;
constexpr int kST = 16 * 16 + 16;              // one 16 x 16 tile (token-major) plus 32 bytes of padding,
                                               // which put the tiles of one token row in different banks

typedef short si16x4 __attribute__((ext_vector_type(4)));
// LDS transpose read: in each group of 16 lanes, with M[j][q] the q-th 16-bit element at lane j's
// address, lane i receives element k = M[4 k + i / 4][i % 4]; a 16 x 16 row-major tile read with
// lane (i, g) at offset 4 (16 g + i) gives lane (i, g) the tile's column i, rows 4 g .. 4 g + 3
__device__ __forceinline__ uint2 tr16(const __bf16* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) si16x4*)(p)));
}
// 32 tokens of column i of two vertically adjacent tiles as one 16x16x32 operand: k = 8 g + e
// stands for token 4 g + e of the first tile (e < 4) and 4 g + e - 4 of the second
__device__ __forceinline__ bf16x8 tr16x2(const __bf16* t0, const __bf16* t1) {
  const uint2 a = tr16(t0), b = tr16(t1);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// A workgroup barrier for LDS data only: this wavefront's LDS accesses complete, then s_barrier,
// with no memory fence.  (__syncthreads' fence would also wait for the direct-to-LDS loads of the
// next chunk's B in flight and, loads completing in order, for the x loads issued before them.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// f(integral_constant<int, i>) for i = 0 .. N - 1, unrolled at compile time
template <int... I, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>()), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>(), f);
}
// every vector memory operation of this wavefront complete but the last N: s_waitcnt vmcnt(N)
// (loads complete in order, so a load issued before N more loads and stores has landed, while
// these stay in flight; the compiler takes an explicit wait into account and adds none of its own
// for what it covers)
template <int N>
__device__ __forceinline__ void vm_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | ((N >> 4) << 14));
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{lo, hi}), b2));
}

// Token rows of a (256 token x VECS 16-byte vector) tile in registers: consecutive lanes take
// consecutive 16-byte vectors of one token row (coalesced loads), and the stores into the
// 16 x 16 LDS tiles are conflict-free.  Tokens past `len` read row 0 and are stored as zeros.
template <int VECS>
struct RowTile {
  static constexpr int U = kSQ * VECS;
  static constexpr int UPT = U / kSThreads;
  static_assert(U % kSThreads == 0, "shape");
  uint4 v[UPT];
  uint32_t okm;

  __device__ __forceinline__ void load_one(int u, const __bf16* base, uint32_t stride, int len, int tid) {
    const int q = tid + kSThreads * u;
    const int t = q / VECS, vec = (q % VECS) * 8;
    const bool ok = t < len;
    uint32_t o = ((uint32_t)(ok ? t : 0) * stride + vec) * 2;
    asm volatile("" : "+v"(o));
    v[u] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + o);
    okm = (okm & ~(1u << u)) | ((uint32_t)ok << u);
  }
  __device__ __forceinline__ void load(const __bf16* base, uint32_t stride, int len, int tid) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) load_one(u, base, stride, len, tid);
  }
  // into tiles (jt, ct) at (jt VECS / 2 + ct) kST, each value times its token's weight wt[t]
  // (straight-line: every weight read issued before the first is used, out-of-range tokens
  // masked by bits, not branches)
  __device__ __forceinline__ void store(__bf16* dst, const float* wt, int tid) const {
    float wv[UPT];
#pragma unroll
    for (int u = 0; u < UPT; ++u) wv[u] = wt[(tid + kSThreads * u) / VECS];
    // (the mask bits made opaque here: known at the load, the masking would be folded into a
    // select right behind it, which waits for the load on the spot)
    uint32_t om = okm;
    asm volatile("" : "+v"(om));
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int q = tid + kSThreads * u;
      const int t = q / VECS, vec = (q % VECS) * 8;
      const uint32_t m = 0u - ((om >> u) & 1u);
      const uint32_t av[4] = {v[u].x & m, v[u].y & m, v[u].z & m, v[u].w & m};
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = pack2(__builtin_bit_cast(float, av[k] << 16) * wv[u], __builtin_bit_cast(float, av[k] & 0xffff0000u) * wv[u]);
      const uint4 a = make_uint4(o[0], o[1], o[2], o[3]);
      const int off = ((t >> 4) * (VECS / 2) + (vec >> 4)) * kST + (t & 15) * 16 + (vec & 15);
      // (an inline-asm LDS store: the compiler does not order it behind the direct-to-LDS B loads
      // in flight, which write other tiles, as it would a plain store; their landing is waited
      // for only before the next chunk's B^T reads)
      typedef unsigned su32x4 __attribute__((ext_vector_type(4)));
      const uint32_t la = (uint32_t)reinterpret_cast<uintptr_t>(&dst[off]);
      asm volatile("ds_write_b128 %0, %1" ::"v"(la), "v"(su32x4{a.x, a.y, a.z, a.w}) : "memory");
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
  constexpr int P = 64, N = 128, Q = kSQ, KS = Q / 32;
  constexpr int EPL = Q / 64;                      // cumsum positions per lane
  constexpr int XV = P / 8;                        // 16-byte vectors per x token row

  __shared__ __attribute__((aligned(16))) __bf16 s_b[(Q / 16) * (N / 16) * kST];   // B of the chunk
  __shared__ __attribute__((aligned(16))) __bf16 s_x[(Q / 16) * (P / 16) * kST];   // x w of one head
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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // this wavefront's 32 x 32 block of S^T: dstate tiles 2 nb, 2 nb + 1 and headdim tiles 2 pb, 2 pb + 1
  // (each x operand read from LDS feeds two MFMAs)
  const int nb = w >> 1, pb = w & 1;
  const uint32_t x_tok = (uint32_t)H * P, b_tok = (uint32_t)G * N;
  const size_t PN = (size_t)P * N;

  auto x_base = [&](int c, int hh) { return x + ((size_t)b * L + (size_t)c * Q) * x_tok + (size_t)(h0 + hh) * P; };
  auto b_base = [&](int c) { return Bm + ((size_t)b * L + (size_t)c * Q) * b_tok + (size_t)g * N; };
  // dt of the positions this lane scans (wavefront hh < HS: head h0 + hh), clamped in bounds, as
  // raw bf16 bits: widened only where the cumsum uses them (a conversion here would wait for
  // each load on the spot)
  auto load_dt = [&](int c, uint32_t (&dv)[EPL]) {
    const int hh = w < HS ? w : 0;
    // (through an opaque pointer: a load known not to alias any store would be moved down to
    // its use in the next chunk, inside the branch of the wavefronts that scan, and waited for
    // there on the spot)
    typedef const __attribute__((address_space(1))) unsigned short gu16;
    gu16* d16 = (gu16*)dt;
    asm volatile("" : "+s"(d16));
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int t = min(c * Q + lane * EPL + k, L - 1);
      dv[k] = d16[((size_t)b * L + t) * H + h0 + hh];
    }
  };

  // the states, transposed: st[hh][2 ni + pi] lane (r, qd) holds S^T[n = 16 (2 nb + ni) + 4 qd + e]
  // [p = 16 (2 pb + pi) + r]
  f32x4 st[HS][4];
#pragma unroll
  for (int hh = 0; hh < HS; ++hh)
#pragma unroll
    for (int j = 0; j < 4; ++j) st[hh][j] = zero4();
  float run = 0.f;                                 // wavefront hh: exponent sum since the segment start

  // B of a chunk straight into s_b (16-byte direct-to-LDS loads): block q (q = w, w + 8, ...) of
  // 64 consecutive 16-byte LDS slots per instruction; slot S is slot S % 34 of tile S / 34 (tile
  // (jt, ct) = 8 jt + ct: token row 16 jt + s / 2, dstate 16 ct + 8 (s % 2) for s < 32; slots 32
  // and 33 are the tile's padding and take a copy of its first vector).  Tokens past the end
  // read row 0: their weights and x are zero, so they add nothing.
  constexpr int BBLK = (Q / 16) * (N / 16) * kST / (64 * 8);       // 1 KiB blocks of s_b
  static_assert(kST * 2 == 34 * 16 && BBLK * 64 * 8 == (Q / 16) * (N / 16) * kST, "B tiles: 34 slots each");
  constexpr int BJ = (BBLK + 7) / 8;                               // blocks per wavefront (at most)
  auto b_block = [&](int j, int c, int t, bool idle) {
    int q = 8 * j + w;
    // (the last round of blocks: wavefronts past the end load the block eight before again, into
    // the same slots, so that no load is conditional)
    if (8 * (j + 1) > BBLK) q = q < BBLK ? q : q - 8;
    asm volatile("" : "+s"(q));
    {
      const int S = 64 * q + (t & 63);
      const int T = S / 34, si = S % 34;
      const int row = 16 * (T >> 3) + (si < 32 ? si >> 1 : 0);
      const int n = 16 * (T & 7) + (si < 32 ? (si & 1) * 8 : 0);
      const int lenc = min(Q, L - c * Q);
      uint32_t o = ((uint32_t)(row < lenc ? row : 0) * b_tok + n) * 2;
      asm volatile("" : "+v"(o));
      o = idle ? 0u : o;                           // (an idle load: one 16-byte vector for all lanes)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(reinterpret_cast<const char*>(b_base(c)) + o),
          (__attribute__((address_space(3))) void*)(s_b + q * 64 * 8), 16, 0, 0);
    }
  };

  // x two heads ahead: the heads of the segment in order (chunk-major) alternate between two
  // register tiles; head n's tile is stored into LDS at its start and then refilled with head
  // n + 2's x, in parts between head n's MFMAs
  RowTile<XV> xr[2];
  xr[0].okm = xr[1].okm = 0;
  // global head n + k after head hh of chunk c, clamped to the segment (a clamped load is unused)
  auto head_after = [&](int c, int hh, int k, int& cn, int& hn) {
    cn = c + (hh + k) / HS;
    hn = (hh + k) % HS;
    if (cn >= c1) {
      cn = c;
      hn = hh;
    }
  };
  uint32_t dtv[EPL];
#pragma unroll
  for (int j = 0; j < BJ; ++j) b_block(j, c0, tid, false);
  load_dt(c0, dtv);
  {
    int cn, hn;
    xr[0].load(x_base(c0, 0), x_tok, min(Q, L - c0 * Q), tid);
    head_after(c0, 0, 1, cn, hn);
    xr[1].load(x_base(cn, hn), x_tok, min(Q, L - cn * Q), tid);
  }

  // one chunk; CP: the chunk's parity in the segment (which register tile each head uses)
  auto chunk = [&](int c, auto cp_tag) {
    constexpr int CP = decltype(cp_tag)::value;
    const int len = min(Q, L - c * Q);
    // the B blocks of this chunk landed.  Every load and store of a chunk is unconditional (no
    // count the compiler tracks depends on a branch), in this order per head: its L_c stores, its
    // share of the next chunk's B (heads 0 .. HS - 2; one head: in it), its four x loads.  After
    // the last B block come head HS - 2's x loads and head HS - 1's stores and loads (one head:
    // its x loads); after the segment's first B, dt and two heads' x
    vm_keep<HS == 1 ? 4 : 12>();
    lds_barrier();                                 // the previous chunk's weights and exponents consumed
    if (w < HS) {
      // dt' and the inclusive in-chunk cumsum of dt' A of head h0 + w; weights to the chunk end
      const int h = h0 + w;
      const float bias = dt_bias[h], av = A[h];
      float d[EPL], cs[EPL], run_l = 0.f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        float v = softplus(__builtin_bit_cast(float, dtv[k] << 16) + bias);
        if (clamp) v = fminf(fmaxf(v, lo), hi);
        d[k] = lane * EPL + k < len ? v : 0.f;
        run_l += d[k] * av;
        cs[k] = run_l;
      }
      const float excl = wave_shr1(wave_incl_scan(run_l));   // sum over the lanes before this one
#pragma unroll
      for (int k = 0; k < EPL; ++k) cs[k] += excl;
      const float last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cs[EPL - 1]), 63));
      const size_t o = (((size_t)b * H + h) * nc + c) * Q + lane * EPL;
      static_assert(EPL == 4, "one 16-byte store per lane");
      *reinterpret_cast<float4*>(&dtp[o]) = make_float4(d[0], d[1], d[2], d[3]);
      *reinterpret_cast<float4*>(&dAcs[o]) = make_float4(cs[0], cs[1], cs[2], cs[3]);
      *reinterpret_cast<float4*>(&s_w[w][lane * EPL]) =
          make_float4(expf(last - cs[0]) * d[0], expf(last - cs[1]) * d[1], expf(last - cs[2]) * d[2],
                      expf(last - cs[3]) * d[3]);
      if (lane == 0) {
        s_last[w] = last;
        cdec[((size_t)b * H + h) * nc + c] = run;
      }
      run += last;
    }
    load_dt(min(c + 1, c1 - 1), dtv);
    lds_barrier();                                 // B (landed before the first barrier), weights and exponents in LDS
    // this wavefront's B^T rows n = 16 (2 nb + ni) + r for the whole chunk (A operands)
    bf16x8 bfr[2][KS];
    {
      int bo = 4 * lane;
      asm volatile("" : "+v"(bo));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          bfr[ni][kk] = tr16x2(&s_b[((2 * kk) * (N / 16) + 2 * nb + ni) * kST + bo],
                               &s_b[((2 * kk + 1) * (N / 16) + 2 * nb + ni) * kST + bo]);
    }

    static_for<HS>([&](auto hc) {
      constexpr int hh = decltype(hc)::value;
      RowTile<XV>& xb = xr[(CP * HS + hh) & 1];
      constexpr int NSTEP = 2 * KS, BH = HS > 1 ? HS - 1 : 1, BPH = (BJ + BH - 1) / BH;
      // B blocks issued in head k
      constexpr auto nbk = [](int k) { return k < BH ? (BJ - k * BPH < BPH ? (BJ - k * BPH > 0 ? BJ - k * BPH : 0) : BPH) : 0; };
      if constexpr (hh > 0) {
        // this head's x (loaded two heads back) landed: after it come, per head, the L_c stores,
        // the B blocks and the x loads (at head 1: the chunk start's dt loads and head 0's; the
        // scanning wavefronts' stores there only add to the count)
        constexpr int KEEP = hh == 1 ? 12 + nbk(0) : 8 + nbk(hh - 1);
        vm_keep<KEEP>();
        lds_barrier();                             // the previous head's x consumed
      }
      xb.store(s_x, s_w[hh], tid);
      lds_barrier();                               // (at head 0 also: every wavefront's B^T rows read)
      const int h = h0 + hh;
      // lane-dependent offsets recomputed per head (nothing lane-dependent is hoisted and kept)
      int lt = tid;
      asm volatile("" : "+v"(lt));
      const int rr = lt & 15, qq = (lt >> 4) & 3;
      {
        // L_c: the state this segment carried into chunk c, rounded to bf16 for the scan (none
        // for the segment's first chunk, whose slot the scan does not read: there every lane
        // stores into its first vector, so that no store is conditional)
        __bf16* dst = prev16 + (((size_t)b * nc + c) * H + h) * PN;
        uint32_t o = ((uint32_t)(32 * pb + rr) * N + 32 * nb + 4 * qq) * 2;
        asm volatile("" : "+v"(o));
        o = c > c0 ? o : 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint2*>(reinterpret_cast<char*>(dst) + o + ((j & 1) * 16 * N + (j >> 1) * 16) * 2) =
              make_uint2(pack2(st[hh][j][0], st[hh][j][1]), pack2(st[hh][j][2], st[hh][j][3]));
      }
      const float dec = expf(s_last[hh]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[hh][j][e] *= dec;
      // head n + 2's x into the tile just stored, a part every fourth MFMA step
      int cn, hn;
      head_after(c, hh, 2, cn, hn);
      const __bf16* xn = x_base(cn, hn);
      const int ln = min(Q, L - cn * Q);
      const int xo = 4 * (lt & 63);
      // the next chunk's B into s_b (free once every wavefront has read its B^T rows): BPH
      // blocks per head in every head but the last (one head: in it), at the head's first step,
      // before its x loads
      // the MFMA steps (pi outer, kk inner; two MFMAs per x operand), the operand of step + XD
      // read before step's MFMAs (LDS latency covered by XD steps)
      auto xop = [&](int kk, int pi) {
        const int pt = 2 * pb + pi;
        return tr16x2(&s_x[((2 * kk) * (P / 16) + pt) * kST + xo], &s_x[((2 * kk + 1) * (P / 16) + pt) * kST + xo]);
      };
      constexpr int XD = 3;
      bf16x8 xq[XD];
#pragma unroll
      for (int k = 0; k < XD; ++k) xq[k] = xop(k % KS, k / KS);
#pragma unroll
      for (int pi = 0; pi < 2; ++pi) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const int step = pi * KS + kk;
          const bf16x8 cur = xq[step % XD];
          if (step + XD < NSTEP) xq[step % XD] = xop((step + XD) % KS, (step + XD) / KS);
          st[hh][pi] = mfma_16x16x32_bf16(bfr[0][kk], cur, st[hh][pi]);
          st[hh][2 + pi] = mfma_16x16x32_bf16(bfr[1][kk], cur, st[hh][2 + pi]);
          if (step % 4 == 1) {
            const int part = step / 4;             // 0..3: head n + 2's x, in parts
            if (part < RowTile<XV>::UPT) xb.load_one(part, xn, x_tok, ln, lt);
          }
          if (step == 0) {
            // (at the segment's last chunk idle loads: s_b is no longer read)
#pragma unroll
            for (int j = 0; j < nbk(hh); ++j) b_block(hh * BPH + j, min(c + 1, c1 - 1), lt, c + 1 >= c1);
          }
          if (step == 0) asm volatile("" ::: "memory");   // (the B blocks issued before the x loads)
        }
      }
    });
  };

  // pairs of chunks (an even number of heads: the tiles have the same roles at every pair's
  // start), then a last single chunk; no chunk is conditional inside the loop, so that no
  // control-flow join makes the compiler copy (and so wait for) the x tiles in flight
  int c = c0;
  for (; c + 1 < c1; c += 2) {
    chunk(c, std::integral_constant<int, 0>());
    chunk(c + 1, std::integral_constant<int, 1>());
  }
  if (c < c1) chunk(c, std::integral_constant<int, 0>());
  // the last chunk's B loads into LDS (issued unconditionally, unused) land before the
  // workgroup ends
  vm_keep<0>();
  // the segment's end states and total exponents
  {
    int lt = tid;
    asm volatile("" : "+v"(lt));
    const int rr = lt & 15, qq = (lt >> 4) & 3;
#pragma unroll
    for (int hh = 0; hh < HS; ++hh) {
      float* dst = E + (((size_t)b * nseg + seg) * H + h0 + hh) * PN;
      uint32_t o = ((uint32_t)(32 * pb + rr) * N + 32 * nb + 4 * qq) * 4;
      asm volatile("" : "+v"(o));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(reinterpret_cast<char*>(dst) + o + ((j & 1) * 16 * N + (j >> 1) * 16) * 4) =
            make_float4(st[hh][j][0], st[hh][j][1], st[hh][j][2], st[hh][j][3]);
    }
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
