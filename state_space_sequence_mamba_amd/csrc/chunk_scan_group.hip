// chunk_scan, group-shared form for bf16 inputs (chunk 256): the same output as chunk_scan.hip,
//   y[i,p] = sum_{j<=i} CB[i,j] exp(dAcs[i] - dAcs[j]) dt'_j x[j,p]        (diagonal block)
//          + exp(dAcs[i]) sum_n C[i,n] Hprev[p,n]                            (carried state)
//          + D[p] x[i,p]                                                     (skip term)
// (times silu(z[i,p]) with a gate), CB[i,j] = sum_n C[i,n] B[j,n].  Sources as chunk_scan.hip:
// "Agent 228: MAMBA-2 Reference Implementations Comparison", sections 2.2 and 3.2; "Agent 228:
// MAMBA-2 Implementation Gaps", Gaps 1 and 4; the gate of section 3.1 of the first page.
//
// CB depends only on the chunk and the group, not on the head, so a workgroup takes one chunk of
// one group and a slice of that group's heads: it forms the chunk's causal CB once, keeps it in
// registers, and streams the heads of its slice through it.  Per head it reads x, the entering
// state and the cumsums once and writes y once, so a launch moves each input and output exactly
// once (B and C once per slice) and contracts CB once per slice instead of once per head.
//
// Eight wavefronts; wavefront w owns the strip pair (w, 15 - w) of the chunk's sixteen 16-row
// strips, i.e. w + 1 and 16 - w causal 16x16 sub-tiles, 17 for every wavefront.  The CB sub-tiles
// (16x16x32 bf16 MFMA over dstate, from the chunk's B and C rows staged in LDS) stay in registers
// for all heads; the C rows stay in LDS for the carried term.  Per head, every product formed
// transposed (y^T = x^T L^T, so that a lane's outputs are four consecutive headdims of one row):
// the carried terms Hprev C^T of both strips on MFMA (Hprev staged in LDS), then the 17 sub-tiles
// as one software pipeline (the next sub-tile's LDS operands in flight during the current one's
// MFMAs), each sub-tile's decay formed in registers (below the diagonal a row factor times a
// per-column weight, both <= 1: one exponential per lane; on the diagonal one per element and the
// causal mask) and rounded to bf16 as the B operand of the 16x16x16 bf16 MFMA whose A operand is
// the x tile read transposed from LDS (x stays token-major there); the skip term on the diagonal
// sub-tiles.  Global memory traffic is spread over the sub-tiles: the next head's inputs are
// loaded into registers in parts on every other sub-tile (in flight for the rest of the head),
// and y, staged in LDS after the head, leaves as 16-byte row stores in parts on the next head's
// sub-tiles in between (two barriers per head).
#include "cb_tiles.h"
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kGQ = 256;                        // chunk length of this form
constexpr int kGS = kGQ / 16;                   // 16-row strips per chunk
constexpr int kGThreads = 512;                  // eight wavefronts
constexpr int kGSub = kGS + 1;                  // causal sub-tiles per wavefront (strip pair)
constexpr float kGLog2e = 1.4426950408889634f;

typedef float gf32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 gbf16x2 __attribute__((ext_vector_type(2)));

// two fp32 values rounded to bf16 (nearest-even) in one 32-bit word (one two-source conversion
// instruction), and back
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((gf32x2{lo, hi}), gbf16x2));
}
// (the two words pass through an empty asm: otherwise the conversion is split into four
// one-source conversions and two byte permutes)
__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
  uint32_t lo = pack_bf16(a, b), hi = pack_bf16(c, d);
  asm volatile("" : "+v"(lo), "+v"(hi));
  return __builtin_bit_cast(bf16x4, (uint2{lo, hi}));
}
__device__ __forceinline__ float unpack_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float unpack_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xffff0000u); }

// 16 bytes at a byte offset from a wavefront-uniform base (scalar base + 32-bit vector offset)
__device__ __forceinline__ uint4 ld16(const void* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + off);
}

typedef short gi16x4 __attribute__((ext_vector_type(4)));
// LDS transpose read (ds_read_b64_tr_b16): every lane passes the address of 8 bytes; in each
// group of 16 lanes, with M[j][q] the q-th 16-bit element at lane j's address, lane i receives
// element k = M[4 k + i / 4][i % 4].  When lane j of group g points at row 4 g + j / 4, columns
// 4 (j % 4) .. + 3 of a row-major 16 x 16 tile T, lane (i, g) receives T[4 g + k][i], k = 0..3:
// the MFMA operand layout of the tile's transpose.
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                        (__attribute__((address_space(3))) gi16x4*)(p)));
}

template <int P, int N>
struct GroupLds {
  static constexpr int BP = N + 8;              // B rows / Hprev rows, n-contiguous (bf16)
  // x: 16 x 16 tiles (16 tokens x 16 headdims, row-major, 512 bytes), tile (jt, pt) at
  // (4 jt + pt) XT.  The 32 padding bytes per tile put the four headdim tiles of one token row
  // in different banks (16-byte stores conflict-free); a tile itself is read contiguously.
  static constexpr int XT = 16 * 16 + 16;
  static constexpr int YP = P + 8;              // y staging rows
  static constexpr int X_ELEMS = (kGQ / 16) * (P / 16) * XT;
  static constexpr int PREV_ELEMS = P * BP;
  static constexpr int Y_ELEMS = kGQ * YP;
  static constexpr int HEAD = X_ELEMS + PREV_ELEMS + Y_ELEMS;   // per-head regions, side by side
  static constexpr int B_ELEMS = kGQ * BP;                      // B rows of the chunk (CB phase only)
  static constexpr int TOTAL = HEAD > B_ELEMS ? HEAD : B_ELEMS;
  static constexpr int C_ELEMS = kGQ * BP;                      // C rows of the chunk, kept for every head
};

// One head's inputs between their global loads and their LDS stores: x as token pairs (each
// thread two 16-byte vectors of consecutive tokens at the same headdim offset; eight lanes cover
// one token row, so every load instruction reads whole rows), stored as they are into the x
// tiles; the bf16 entering state as 16-byte vectors, the chunk's dt' and cumsum (threads 0..255,
// one position each) and D (threads 0..P-1).
template <int P, int N>
struct HeadRegs {
  static constexpr int PV = P / 8;                          // 16-byte vectors per token row
  static constexpr int XU = (kGQ / 2) * PV;                 // token-pair units
  static constexpr int XPT = XU / kGThreads;
  static constexpr int PU = P * N / 8;                      // 16-byte vectors of the state
  static constexpr int PPT = PU / kGThreads;
  static_assert(XU % kGThreads == 0 && PU % kGThreads == 0, "shape");
  uint4 x[XPT][2];
  uint4 pv[PPT];
  uint4 hv[PPT];           // segmented states: the state entering the segment (else unused)
  float dt, da, dd;
  float ecdv;              // segmented states: the decay exponent since the segment start
  bool seg;                // segmented states
  bool pz;                 // segmented states, c opens its segment: no carried state of its own
  uint32_t okm;

  // Per-lane element offsets from the head's (wavefront-uniform) base pointers, 32-bit: the
  // loads take a scalar base plus a vector offset.  The offsets are made opaque at each call so
  // the compiler does not keep precomputed 64-bit addresses alive across the head loop.  The
  // loads come in parts (part = 0 .. kParts - 1) so that a caller can spread their issue.
  // hh: the segment's incoming state (null without segments); first: c opens its segment (no
  // carried part of its own); ecd: the decay exponent since the segment start
  static constexpr int kParts = XPT + 2;
  __device__ __forceinline__ void load_part(int part, const __bf16* xh, const __bf16* ph, const float* dth,
                                            const float* dah, const float* Dh, uint32_t x_tok, int len, int tid,
                                            const __bf16* hh, bool first, const float* ecd) {
    if (part < XPT) {
      const int u = part;
      const int v = tid + kGThreads * u;
      const int vec = (v % PV) * 8, m = v / PV;
      const int tok = 2 * m;
      const bool ok0 = tok < len, ok1 = tok + 1 < len;
      uint32_t xo0 = ((uint32_t)(ok0 ? tok : 0) * x_tok + vec) * 2;      // bytes
      uint32_t xo1 = ((uint32_t)(ok1 ? tok + 1 : 0) * x_tok + vec) * 2;
      const uint32_t bits = ((uint32_t)ok0 << (2 * u)) | ((uint32_t)ok1 << (2 * u + 1));
      okm = u == 0 ? bits : (okm | bits);
      asm volatile("" : "+v"(xo0), "+v"(xo1));
      x[u][0] = ld16(xh, xo0);
      x[u][1] = ld16(xh, xo1);
    } else if (part == XPT) {
      uint32_t po[PPT];
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        po[u] = (uint32_t)(tid + kGThreads * u) * 16;                     // bytes
        asm volatile("" : "+v"(po[u]));
      }
      // (a segment's first chunk has no carried state of its own: it drops the loaded one at the
      // store, since overwriting the registers here would wait for their loads, and loads it
      // from the incoming state's address, so that the bytes come from the L2)
      pz = hh && first;
      const __bf16* pp = pz ? hh : ph;
#pragma unroll
      for (int u = 0; u < PPT; ++u) pv[u] = ld16(pp, po[u]);
      if (hh) {
#pragma unroll
        for (int u = 0; u < PPT; ++u) hv[u] = ld16(hh, po[u]);
      }
    } else {
      // only the wavefronts that store them load the scalars (wavefront-uniform branches)
      const int wf = __builtin_amdgcn_readfirstlane(tid) / 64;
      uint32_t io = (tid & (kGQ - 1)) * 4, Do = (tid & (P - 1)) * 4;
      asm volatile("" : "+v"(io), "+v"(Do));
      // (the exponent is loaded by a vector load, opaque offset 0, and taken at the store: a
      // scalar load would be waited for, and the value moved to a vector register, right here
      // between the MFMAs)
      // (loaded on every path, without segments from the cumsum, so that no select or branch
      // on the loaded value pulls its use forward)
      seg = hh != nullptr;
      uint32_t zo = 0;
      asm volatile("" : "+v"(zo));
      ecdv = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(hh ? ecd : dah) + zo);
      if (wf < kGQ / 64) {
        dt = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(dth) + io);
        da = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(dah) + io);
      }
      if (wf < P / 64 || (P < 64 && wf == 0)) dd = Dh ? *reinterpret_cast<const float*>(reinterpret_cast<const char*>(Dh) + Do) : 0.f;
    }
  }

  // x into its tiles (16-byte stores), the state rows, and for threads 0..255 the log2e-scaled
  // cumsum, dt' and the column weights W_j = exp2(dAcs_c - dAcs_j) dt'_j, c = j | 15 (the last
  // column of j's 16-column tile)
  template <typename L>
  __device__ __forceinline__ void store(__bf16* s_x, __bf16* s_prev, float* s_da, float* s_dt, float* s_w,
                                        float* s_D, int tid) const {
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int v = tid + kGThreads * u;
      const int vec = (v % PV) * 8, m = v / PV;
      const int tok = 2 * m;                                   // (even: both tokens in one tile)
      const int o = ((tok >> 4) * (P / 16) + (vec >> 4)) * L::XT + (tok & 15) * 16 + (vec & 15);
      uint4 a = x[u][0], b = x[u][1];
      if (!((okm >> (2 * u)) & 1u)) a = make_uint4(0, 0, 0, 0);
      if (!((okm >> (2 * u + 1)) & 1u)) b = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&s_x[o]) = a;
      *reinterpret_cast<uint4*>(&s_x[o + 16]) = b;
    }
    const float sdec = __expf(ecdv);   // exp of the decay since the segment start (with segments)
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int v = tid + kGThreads * u;
      const int p = (v * 8) / N, n = (v * 8) % N;
      uint4 o = pv[u];
      if (pz) o = make_uint4(0, 0, 0, 0);            // (that slot holds no state of this segment)
      if (seg) {
        // segmented states: the entering state is the segment's own carry plus the decayed
        // state that entered the segment, rounded to bf16 as the scan reads it
        const uint32_t lv[4] = {o.x, o.y, o.z, o.w}, iv[4] = {hv[u].x, hv[u].y, hv[u].z, hv[u].w};
        uint32_t ov[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float l0 = __builtin_bit_cast(float, lv[q] << 16), l1 = __builtin_bit_cast(float, lv[q] & 0xffff0000u);
          const float i0 = __builtin_bit_cast(float, iv[q] << 16), i1 = __builtin_bit_cast(float, iv[q] & 0xffff0000u);
          ov[q] = pack_bf16(l0 + sdec * i0, l1 + sdec * i1);
        }
        o = make_uint4(ov[0], ov[1], ov[2], ov[3]);
      }
      *reinterpret_cast<uint4*>(&s_prev[p * L::BP + n]) = o;
    }
    if (tid < kGQ) {
      const float d2 = da * kGLog2e;
      const float dc = __shfl(d2, (tid & 63) | 15, 64);
      s_da[tid] = d2;
      s_dt[tid] = dt;
      s_w[tid] = __builtin_amdgcn_exp2f(dc - d2) * dt;
    }
    if (tid < P) s_D[tid] = dd;
  }
};

}  // namespace

// GATE: z is given (a separate instantiation, so that the ungated kernel carries none of the
// gate's registers)
template <int P, int N, bool GATE>
__global__ __launch_bounds__(kGThreads, 1) void chunk_scan_group_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ Bm, const __bf16* __restrict__ Cm,
    const float* __restrict__ dtp, const float* __restrict__ dAcs, const __bf16* __restrict__ prev16,
    const float* __restrict__ Dw, const __bf16* __restrict__ Z, __bf16* __restrict__ y, int L, int H, int G, int nc,
    int hs, uint32_t nblocks, const __bf16* __restrict__ hin16, const float* __restrict__ cdec, int seg_len) {
  typedef GroupLds<P, N> SL;
  typedef NDot<__bf16, N> ND;
  typedef HeadRegs<P, N> HR;
  constexpr int TP = P / 16;

  __shared__ __attribute__((aligned(16))) __bf16 s_mem[SL::TOTAL];
  __shared__ __attribute__((aligned(16))) __bf16 s_c[SL::C_ELEMS];   // C rows (carried term)
  __shared__ __attribute__((aligned(16))) float s_da[kGQ];   // dAcs * log2(e)
  __shared__ __attribute__((aligned(16))) float s_dt[kGQ];
  __shared__ __attribute__((aligned(16))) float s_w[kGQ];    // column weights
  __shared__ __attribute__((aligned(16))) float s_D[P];      // skip weights of the head
  __bf16* s_b = s_mem;                                       // CB phase: B rows
  __bf16* s_x = s_mem;                                       // per head: x^T, Hprev, y staging
  __bf16* s_prev = s_mem + SL::X_ELEMS;
  __bf16* s_y = s_mem + SL::X_ELEMS + SL::PREV_ELEMS;

  // work unit: (b, c, g, head slice); the slices of one (b, c, g) are consecutive, so they share
  // B and C in one XCD's L2
  uint32_t id = xcd_swizzle(blockIdx.x, nblocks);
  const int hpg = H / G, nsl = hpg / hs;
  const int sl = id % nsl;
  id /= nsl;
  const int g = id % G;
  id /= G;
  const int c = id % nc, b = id / nc;
  const int h0 = g * hpg + sl * hs;
  const int t0 = c * kGQ;
  const int len = min(kGQ, L - t0);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);    // wavefront-uniform: scalar branches below
  const int r = lane & 15, qd = lane >> 4;
  const int s0 = w, s1 = kGS - 1 - w;                        // this wavefront's strips

  const size_t bc_tok = (size_t)G * N, x_tok = (size_t)H * P;
  const __bf16* Cb = Cm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  const __bf16* Bb = Bm + ((size_t)b * L + t0) * bc_tok + (size_t)g * N;
  auto head_ptrs = [&](int h, const __bf16*& xh, const __bf16*& ph, const float*& dth, const float*& dah,
                       const float*& Dh) {
    xh = x + ((size_t)b * L + t0) * x_tok + (size_t)h * P;
    ph = prev16 + (((size_t)b * nc + c) * H + h) * (size_t)(P * N);
    const size_t o = (((size_t)b * H + h) * nc + c) * kGQ;
    dth = dtp + o;
    dah = dAcs + o;
    Dh = Dw ? Dw + (size_t)h * P : nullptr;
  };

  // segmented chunk states: the state entering c's segment and the decay since its start
  const bool seg_first = seg_len > 0 && c % seg_len == 0;
  auto seg_in = [&](int h) -> const __bf16* {
    return seg_len > 0 ? hin16 + (((size_t)b * ((nc + seg_len - 1) / seg_len) + c / seg_len) * H + h) * (size_t)(P * N)
                       : nullptr;
  };
  auto seg_dec = [&](int h) { return cdec + ((size_t)b * H + h) * nc + c; };

  // ---- prologue: B rows of the chunk, this wavefront's C rows, the first head's inputs
  constexpr int BU = kGQ * N / 8, BPT = BU / kGThreads;       // 16-byte vectors of B
  uint4 breg[BPT];
#pragma unroll
  for (int u = 0; u < BPT; ++u) {
    const int v = tid + kGThreads * u;
    const int row = v / (N / 8), nv = (v % (N / 8)) * 8;
    breg[u] = *reinterpret_cast<const uint4*>(Bb + (size_t)(row < len ? row : 0) * bc_tok + nv);
  }
  // C rows past the end read row 0 (they reach only output rows that are never stored).  (Read
  // through an opaque pointer and fenced: loads known to be invariant would be moved down to
  // their LDS stores, each then waited for on its own.)
  uint4 creg[BPT];
  {
    typedef unsigned gu32x4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(1))) gu32x4 gv4;
    gv4* cg = (gv4*)Cb;
    asm volatile("" : "+s"(cg));
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const int v = tid + kGThreads * u;
      const int row = v / (N / 8), nv = (v % (N / 8)) * 8;
      const gu32x4 t = cg[((size_t)(row < len ? row : 0) * bc_tok + nv) / 8];
      creg[u] = make_uint4(t.x, t.y, t.z, t.w);
    }
  }
  HR hr;
  // part `part` of head hn's inputs into hr
  auto load_part = [&](int part, int hn, int t) {
    const __bf16 *xh, *ph;
    const float *dth, *dah, *Dh;
    head_ptrs(hn, xh, ph, dth, dah, Dh);
    hr.load_part(part, xh, ph, dth, dah, Dh, (uint32_t)x_tok, len, t, seg_in(hn), seg_first, seg_dec(hn));
  };
#pragma unroll
  for (int part = 0; part < HR::kParts; ++part) load_part(part, h0, tid);
  asm volatile("" ::: "memory");
  // row block u of a head's y, from the staging tile (y_part) to global memory (y_flush), in
  // 16-byte row pieces, through a buffer resource bounded to the chunk's len rows: stores past
  // it are dropped by the hardware, so no store is conditional (live = false: every store is)
  constexpr int kYParts = (kGQ * P / 8) / kGThreads;
  typedef unsigned yu32x4 __attribute__((ext_vector_type(4)));
  auto y_rsrc = [&](int hn, bool live) {
    const __bf16* base = y + ((size_t)b * L + t0) * x_tok + (size_t)hn * P;
    const int nbytes = live ? (int)(((uint32_t)(len - 1) * (uint32_t)x_tok + P) * 2) : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nbytes, 0x00020000);
  };
  auto y_part = [&](int u, int t) {
    const int v = t + kGThreads * u;
    const int row = v / (P / 8), cv = (v % (P / 8)) * 8;
    return *reinterpret_cast<const uint4*>(&s_y[row * SL::YP + cv]);
  };
  auto y_flush = [&](int u, const uint4& val, __amdgpu_buffer_rsrc_t rs, int t) {
    const int v = t + kGThreads * u;
    const int row = v / (P / 8), cv = (v % (P / 8)) * 8;
    uint32_t yo = ((uint32_t)row * (uint32_t)x_tok + cv) * 2;
    asm volatile("" : "+v"(yo));
    __builtin_amdgcn_raw_buffer_store_b128((yu32x4){val.x, val.y, val.z, val.w}, rs, yo, 0, 0);
  };
#pragma unroll
  for (int u = 0; u < BPT; ++u) {
    const int v = tid + kGThreads * u;
    const int row = v / (N / 8), nv = (v % (N / 8)) * 8;
    *reinterpret_cast<uint4*>(&s_b[row * SL::BP + nv]) = row < len ? breg[u] : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&s_c[row * SL::BP + nv]) = creg[u];
  }
  __syncthreads();

  // ---- C B^T of this wavefront's 17 causal sub-tiles, kept for every head, in the order the
  // head loop takes them: slot 0 is strip s0's diagonal tile, slot k in 1..15 is (strip s0,
  // column tile k - 1) for k <= w and (strip s1, column tile k - w - 1) after, slot 16 is strip
  // s1's diagonal tile.  Lane (r, qd) holds CB[i = 16 s + r][j = 16 jt + 4 qd + e].
  f32x4 cb[kGSub];
  {
    typename ND::frag cf0, cf1;
    ND::load(cf0, &s_c[(16 * s0 + r) * SL::BP], qd);
    ND::load(cf1, &s_c[(16 * s1 + r) * SL::BP], qd);
#pragma unroll
    for (int k = 0; k < kGSub; ++k) {
      const bool first = k == 0 || (k < kGSub - 1 && k <= w);
      const int jt = k == 0 ? w : k == kGSub - 1 ? s1 : k <= w ? k - 1 : k - w - 1;
      typename ND::frag bfr;
      ND::load(bfr, &s_b[(16 * jt + r) * SL::BP], qd);
      if (first)
        cb[k] = ND::dot(bfr, cf0, zero4());
      else
        cb[k] = ND::dot(bfr, cf1, zero4());
    }
  }
  __syncthreads();                                           // s_b consumed: the head regions reuse it
  hr.template store<SL>(s_x, s_prev, s_da, s_dt, s_w, s_D, tid);
  __syncthreads();

  for (int hh = 0; hh < hs; ++hh) {
    const int h = h0 + hh;
    const bool more = hh + 1 < hs;

    // per-lane LDS offsets, opaque to the compiler at every head: otherwise it hoists the
    // head-independent operand addresses of the sub-tiles out of the head loop and spills them;
    // this way each read is a base register plus an offset.
    // Every lane-dependent quantity of the loop body is derived from a laundered copy of the
    // thread index for the same reason.
    int lt = tid, wl = w;
    asm volatile("" : "+v"(lt), "+s"(wl));
    const int r = lt & 15, qd = (lt >> 4) & 3;
    const int w = wl, s0 = wl, s1 = kGS - 1 - wl;   // (uniform conditions are recomputed per head)
    const int xo = 4 * (lt & 63), wo = 4 * qd;            // (xo: this lane's 8 bytes of an x tile)
    // likewise C B^T: nothing derived from it is hoisted out of the head loop
#pragma unroll
    for (int k = 0; k < kGSub; ++k) asm volatile("" : "+v"(cb[k]));

    // Every product is formed transposed, y^T = x^T L^T: lane (r, qd) of accumulator pt holds
    // y[i = 16 s + r][p = 16 pt + 4 qd + e], four consecutive headdims of one output row.
    // carried terms of both strips, exp(dAcs_i) Hprev C_i^T: each state tile is read once for both
    f32x4 acc[TP], acc1[TP];
    {
      typename ND::frag cf0, cf1;
      ND::load(cf0, &s_c[(16 * s0 + r) * SL::BP], qd);
      ND::load(cf1, &s_c[(16 * s1 + r) * SL::BP], qd);
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        typename ND::frag pf;
        ND::load(pf, &s_prev[(pt * 16 + r) * SL::BP], qd);
        acc[pt] = ND::dot(pf, cf0, zero4());
        acc1[pt] = ND::dot(pf, cf1, zero4());
      }
      const float f0 = __builtin_amdgcn_exp2f(s_da[16 * s0 + r]), f1 = __builtin_amdgcn_exp2f(s_da[16 * s1 + r]);
#pragma unroll
      for (int pt = 0; pt < TP; ++pt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[pt][e] *= f0;
          acc1[pt][e] *= f1;
        }
    }

    // the diagonal-block sub-tiles as one software pipeline over the 17 slots: the operands of
    // slot k + 1 (x tiles, transposed as they are read, and decay scalars) are read from LDS
    // before slot k's MFMAs, and every
    // slot accumulates into acc; when strip s0 is complete (after slot w) its results wait in
    // registers as bf16 and acc takes over strip s1's carried term.
    struct Ops {
      bf16x4 x[TP];
      float4 f0, f1;   // off the diagonal: the column weights; on it: the cumsums and dt'
      float dc;        // off the diagonal: the cumsum at the column tile's last position
    };
    auto read_ops = [&](int jt, bool diag, Ops& o) {
      const int xj = xo + jt * (P / 16) * SL::XT, wj = wo + 16 * jt;
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) o.x[pt] = lds_read_tr16(&s_x[xj + pt * SL::XT]);
      if (diag) {
        o.f0 = *reinterpret_cast<const float4*>(&s_da[wj]);
        o.f1 = *reinterpret_cast<const float4*>(&s_dt[wj]);
      } else {
        o.f0 = *reinterpret_cast<const float4*>(&s_w[wj]);
        o.dc = s_da[16 * jt + 15];
      }
    };
    const float dr0 = s_da[16 * s0 + r], dr1 = s_da[16 * s1 + r];
    // diagonal tile of strip s: one exponential per element and the causal mask; the skip term
    // D_p x[i][p] from the lane's own output elements of the tile (untransposed reads)
    auto diag_tile = [&](const f32x4& cbk, const Ops& o, float dr, int s) {
      const bf16x4 a = to_bf16x4((4 * qd + 0 <= r) ? cbk[0] * __builtin_amdgcn_exp2f(dr - o.f0.x) * o.f1.x : 0.f,
                                 (4 * qd + 1 <= r) ? cbk[1] * __builtin_amdgcn_exp2f(dr - o.f0.y) * o.f1.y : 0.f,
                                 (4 * qd + 2 <= r) ? cbk[2] * __builtin_amdgcn_exp2f(dr - o.f0.z) * o.f1.z : 0.f,
                                 (4 * qd + 3 <= r) ? cbk[3] * __builtin_amdgcn_exp2f(dr - o.f0.w) * o.f1.w : 0.f);
      const int xr = s * (P / 16) * SL::XT + r * 16 + 4 * qd;
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        const uint2 xv = *reinterpret_cast<const uint2*>(&s_x[xr + pt * SL::XT]);
        const float4 dv = *reinterpret_cast<const float4*>(&s_D[16 * pt + 4 * qd]);
        acc[pt] = mfma_16x16x16_bf16(o.x[pt], a, acc[pt]);
        acc[pt][0] += dv.x * unpack_lo(xv.x);
        acc[pt][1] += dv.y * unpack_hi(xv.x);
        acc[pt][2] += dv.z * unpack_lo(xv.y);
        acc[pt][3] += dv.w * unpack_hi(xv.y);
      }
    };
    // below the diagonal: a row factor times the column weights (both <= 1)
    auto off_tile = [&](const f32x4& cbk, const Ops& o, float dr) {
      const float ri = __builtin_amdgcn_exp2f(dr - o.dc);
      const bf16x4 a = to_bf16x4(cbk[0] * o.f0.x * ri, cbk[1] * o.f0.y * ri, cbk[2] * o.f0.z * ri, cbk[3] * o.f0.w * ri);
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) acc[pt] = mfma_16x16x16_bf16(o.x[pt], a, acc[pt]);
    };
    // output gate on the lane's elements of strip s (rows past the sequence read a clamped
    // address); z of both strips is loaded at the head's start, so that the gate waits for z
    // alone and not for the next head's inputs issued after it
    auto load_z = [&](int s, uint2 (&zv)[TP]) {
      const __bf16* zh = Z + ((size_t)b * L + t0) * x_tok + (size_t)h * P;
      const int i = 16 * s + r;
      uint32_t zo = (uint32_t)(i < len ? i : 0) * (uint32_t)x_tok + 4 * qd;
      asm volatile("" : "+v"(zo));
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) zv[pt] = *reinterpret_cast<const uint2*>(zh + zo + pt * 16);
    };
    uint2 zv0[TP], zv1[TP];
    if constexpr (GATE) {
      load_z(s0, zv0);
      load_z(s1, zv1);
    }
    auto gate = [&](const uint2 (&zv)[TP]) {
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        acc[pt][0] *= silu(unpack_lo(zv[pt].x));
        acc[pt][1] *= silu(unpack_hi(zv[pt].x));
        acc[pt][2] *= silu(unpack_lo(zv[pt].y));
        acc[pt][3] *= silu(unpack_hi(zv[pt].y));
      }
    };

    uint32_t ypk[TP][2];
    float dr = dr0;
    const __amdgpu_buffer_rsrc_t yrs = y_rsrc(h - 1, hh > 0);   // the previous head's y (none at the first)
    uint4 yv;
    Ops cur, nxt;
    read_ops(w, true, cur);                                  // slot 0: strip s0's diagonal tile
    read_ops(0, false, nxt);                                 // slot 1: column tile 0 of s0 or s1
    diag_tile(cb[0], cur, dr0, s0);
#pragma unroll
    for (int k = 1; k < kGSub - 1; ++k) {
      cur = nxt;
      // (each y row block read from LDS a slot before its store, ahead of the operand reads: the
      // store then waits for it alone)
      if (k % 2 == 1 && k / 2 < kYParts) yv = y_part(k / 2, lt);
      if (k + 1 < kGSub - 1)
        read_ops(k + 1 <= w ? k : k - w, false, nxt);
      else
        read_ops(s1, true, nxt);
      // the next head's inputs, a part every other slot, in flight for the rest of this head (the
      // last head reloads its own, unused); between them the previous head's y, a row block per
      // slot, from its staging tile (rewritten only after this head's first barrier)
      if (k % 2 == 1 && k / 2 < HR::kParts) load_part(k / 2, more ? h + 1 : h, lt);
      if (k % 2 == 0 && k / 2 - 1 < kYParts) y_flush(k / 2 - 1, yv, yrs, lt);
      if (k == w + 1) {                                      // strip s0 complete
        if constexpr (GATE) gate(zv0);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          ypk[pt][0] = pack_bf16(acc[pt][0], acc[pt][1]);
          ypk[pt][1] = pack_bf16(acc[pt][2], acc[pt][3]);
          acc[pt] = acc1[pt];
        }
        dr = dr1;
      }
      off_tile(cb[k], cur, dr);
    }
    diag_tile(cb[kGSub - 1], nxt, dr1, s1);                  // slot 16: strip s1's diagonal tile
    if constexpr (GATE) gate(zv1);
    __syncthreads();                                         // x, Hprev and scalars of head h consumed
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) {
      *reinterpret_cast<uint2*>(&s_y[(16 * s0 + r) * SL::YP + pt * 16 + 4 * qd]) = make_uint2(ypk[pt][0], ypk[pt][1]);
      *reinterpret_cast<uint2*>(&s_y[(16 * s1 + r) * SL::YP + pt * 16 + 4 * qd]) =
          make_uint2(pack_bf16(acc[pt][0], acc[pt][1]), pack_bf16(acc[pt][2], acc[pt][3]));
    }
    if (more) hr.template store<SL>(s_x, s_prev, s_da, s_dt, s_w, s_D, lt);
    __syncthreads();                                         // y staged; the next head's inputs in LDS
  }
  // the last head's y
  {
    int lt = tid;
    asm volatile("" : "+v"(lt));
    const __amdgpu_buffer_rsrc_t yrs = y_rsrc(h0 + hs - 1, true);
#pragma unroll
    for (int u = 0; u < kYParts; ++u) y_flush(u, y_part(u, lt), yrs, lt);
  }
}

bool chunk_scan_group_supported(int dtype, int P, int N, int Q) {
  return dtype == DT_BF16 && Q == kGQ && P == 64 && N == 128;
}

hipError_t launch_chunk_scan_group(const FwdArgs& a, int hs, hipStream_t s) {
  if (!chunk_scan_group_supported(a.dtype, a.P, a.N, a.Q) || !a.prev16) return hipErrorInvalidValue;
  const int hpg = a.H / a.G;
  if (hs < 1 || hpg % hs != 0) return hipErrorInvalidValue;
  const uint32_t nblocks = (uint32_t)a.B * a.nc * a.G * (hpg / hs);
  if (nblocks == 0) return hipSuccess;
  hipExtLaunchKernelGGL(a.z ? chunk_scan_group_kernel<64, 128, true> : chunk_scan_group_kernel<64, 128, false>,
                        dim3(nblocks), dim3(kGThreads), 0, s, a.ev0, a.ev1, 0,
                        static_cast<const __bf16*>(a.x), static_cast<const __bf16*>(a.Bm),
                        static_cast<const __bf16*>(a.Cm), a.dtp, a.dAcs, static_cast<const __bf16*>(a.prev16), a.D,
                        static_cast<const __bf16*>(a.z), static_cast<__bf16*>(a.y), a.L, a.H, a.G, a.nc, hs, nblocks,
                        static_cast<const __bf16*>(a.hin16), a.cdec, a.seg_len);
  return hipGetLastError();
}

}  // namespace ssd
