// Shared device helpers of the gfx950 SSD kernels: element conversion, softplus,
// MFMA wrappers, XCD-aware block order, 16-byte vector loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

namespace ssd {

// ---------------------------------------------------------------- element types
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// fp32 -> bf16 with round-to-nearest-even (the hardware conversion on gfx950)
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return static_cast<__bf16>(v); }

// 16 bytes of T: 4 fp32 or 8 bf16
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int n = 4;
  float v[4];
};
template <> struct Vec16<__bf16> {
  static constexpr int n = 8;
  __bf16 v[8];
};

template <typename T>
__device__ __forceinline__ Vec16<T> load16(const T* p) {
  Vec16<T> r;
  *reinterpret_cast<uint4*>(&r) = *reinterpret_cast<const uint4*>(p);
  return r;
}
template <typename T>
__device__ __forceinline__ Vec16<T> zero16() {
  Vec16<T> r;
  *reinterpret_cast<uint4*>(&r) = make_uint4(0, 0, 0, 0);
  return r;
}
// Zero a 16-byte vector unless ok (branch-free select).
template <typename T>
__device__ __forceinline__ Vec16<T> keep_if(const Vec16<T>& in, bool ok) {
  uint4 v = *reinterpret_cast<const uint4*>(&in);
  v.x = ok ? v.x : 0u;
  v.y = ok ? v.y : 0u;
  v.z = ok ? v.z : 0u;
  v.w = ok ? v.w : 0u;
  Vec16<T> r;
  *reinterpret_cast<uint4*>(&r) = v;
  return r;
}
// Branch-free guarded load: always reads `p` (the caller passes an in-bounds address,
// clamped when the element is not wanted) and returns zeros when !ok.  A conditional load
// would compile to a branch with an immediate wait for the data, serialising every load.
template <typename T>
__device__ __forceinline__ Vec16<T> load16_if(const T* p, bool ok) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  v.x = ok ? v.x : 0u;
  v.y = ok ? v.y : 0u;
  v.z = ok ? v.z : 0u;
  v.w = ok ? v.w : 0u;
  Vec16<T> r;
  *reinterpret_cast<uint4*>(&r) = v;
  return r;
}

// ---------------------------------------------------------------- scalar maths
// softplus(v) = log(1 + e^v).  Above 20 the correction log1p(e^-v) < 2.1e-9 is below
// fp32 resolution of v, so v itself is returned (and e^v never overflows).
__device__ __forceinline__ float softplus(float v) { return v > 20.f ? v : log1pf(expf(v)); }

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP lane moves (no LDS round
// trips): Hillis-Steele within each row of 16 lanes (row_shr 1, 2, 4, 8; lanes shifted in from
// before the row's start add 0), then each odd row adds the total of the row before it
// (row_bcast:15 into rows 1 and 3) and rows 2 and 3 the total of rows 0 and 1 (row_bcast:31).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
  const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false);
  return x + __builtin_bit_cast(float, t);
}
__device__ __forceinline__ float wave_incl_scan(float x) {
  x = dpp_add<0x111, 0xf>(x);   // row_shr:1
  x = dpp_add<0x112, 0xf>(x);   // row_shr:2
  x = dpp_add<0x114, 0xf>(x);   // row_shr:4
  x = dpp_add<0x118, 0xf>(x);   // row_shr:8
  x = dpp_add<0x142, 0xa>(x);   // row_bcast:15 into rows 1, 3
  x = dpp_add<0x143, 0xc>(x);   // row_bcast:31 into rows 2, 3
  return x;
}
// the value of the lane before (lane 0: 0), by a wave_shr:1 lane move
__device__ __forceinline__ float wave_shr1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x138, 0xf, 0xf, false));
}

// silu(u) = u / (1 + e^-u) with the hardware exp2 and reciprocal (each within ~1 ulp; the
// result is within a few ulp).  Saturates cleanly: u -> -inf gives -0, u -> +inf gives u.
__device__ __forceinline__ float silu(float u) {
  return u * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-u * 1.4426950408889634f));
}

// ---------------------------------------------------------------- block order
// Workgroups are dispatched round-robin over the 8 XCDs (id % 8), each with its own L2.
// Map the hardware id to a logical id so that consecutive logical ids run on the same
// XCD: blocks that share B/C tiles (heads of one group, one chunk) then share an L2.
__device__ __forceinline__ uint32_t xcd_swizzle(uint32_t id, uint32_t n) {
  const uint32_t q = n >> 3;
  const uint32_t full = q << 3;
  if (id >= full) return id;
  return (id & 7u) * q + (id >> 3);
}

// ---------------------------------------------------------------- MFMA
// 16x16 output tiles.  Lane l = 16*qd + r (r = l & 15, qd = l >> 4).
//   A operand: lane holds A[row r][k in the qd-th K slice]
//   B operand: lane holds B[k in the qd-th K slice][col r]
//   result   : lane holds D[4*qd + e][col r], e = 0..3
// Only the pairing of A and B items matters for the sum over k, so any assignment of
// k values to (qd, item) works as long as A and B use the same one.
__device__ __forceinline__ f32x4 mfma_16x16x4_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x16_bf16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Contraction over a dimension that is contiguous in LDS for both operands.
// K = k values per instruction, KPL = k values per lane (contiguous in memory).
template <typename T> struct KMma;
template <> struct KMma<float> {
  static constexpr int K = 4;
  static constexpr int KPL = 1;
  typedef float frag;
  __device__ static __forceinline__ frag load(const float* p) { return *p; }
  __device__ static __forceinline__ frag zero() { return 0.f; }
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) { return mfma_16x16x4_f32(a, b, c); }
};
template <> struct KMma<__bf16> {
  static constexpr int K = 32;
  static constexpr int KPL = 8;
  typedef bf16x8 frag;
  __device__ static __forceinline__ frag load(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  __device__ static __forceinline__ frag zero() {
    frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = static_cast<__bf16>(0.f);
    return z;
  }
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) { return mfma_16x16x32_bf16(a, b, c); }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace ssd
