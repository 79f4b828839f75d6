// Device helpers shared by the Atom, SNAC and MoE kernels of librrb.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace rrb {

// bf16 -> fp32 is exact: the bf16 pattern is the upper half of the binary32.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even, on the bit pattern: adding
// 0x7fff plus the lowest kept bit carries into bit 16 exactly when the
// dropped half is above the midpoint, or at the midpoint with an odd kept
// part.  Infinities stay infinite, finite overflow carries into the infinity
// pattern, subnormals and -0 are kept; every NaN becomes 0x7fc0.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_rne(lo)) |
         (static_cast<uint32_t>(f32_to_bf16_rne(hi)) << 16);
}

// Eight fp32 values to eight bf16 with gfx950's packed conversion
// (v_cvt_pk_bf16_f32: round to nearest even in the default rounding mode,
// subnormals kept, the same bits as f32_to_bf16_rne for every value that is
// not a NaN).  The hardware keeps a NaN's sign and payload, so a wave with a
// NaN in any lane's eight takes f32_to_bf16_rne instead (the same bits for
// every other value).  The test is four unordered compares into wave masks,
// ORed on the scalar unit (predicate 8 is LLVM's FCMP_UNO).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ uint4 pack_bf16x8(const float (&a)[8]) {
  uint4 o;
  const uint64_t nan = __builtin_amdgcn_fcmpf(a[0], a[1], 8) | __builtin_amdgcn_fcmpf(a[2], a[3], 8) |
                       __builtin_amdgcn_fcmpf(a[4], a[5], 8) | __builtin_amdgcn_fcmpf(a[6], a[7], 8);
  if (nan) {
    o.x = pack_bf16x2(a[0], a[1]);
    o.y = pack_bf16x2(a[2], a[3]);
    o.z = pack_bf16x2(a[4], a[5]);
    o.w = pack_bf16x2(a[6], a[7]);
  } else {
    o.x = cvt_pk_bf16(a[0], a[1]);
    o.y = cvt_pk_bf16(a[2], a[3]);
    o.z = cvt_pk_bf16(a[4], a[5]);
    o.w = cvt_pk_bf16(a[6], a[7]);
  }
  return o;
}

// Fixed rank-order fold of 8 bf16 lanes from R sources: fp32 accumulation,
// one rounding at the end.  The adds are written one per step so the
// compiler cannot reassociate them (no fast-math anywhere in this library).
template <int R>
__device__ __forceinline__ uint4 fold_bf16x8(const uint4 (&v)[R]) {
  float a[8];
  a[0] = bf16_lo(v[0].x); a[1] = bf16_hi(v[0].x);
  a[2] = bf16_lo(v[0].y); a[3] = bf16_hi(v[0].y);
  a[4] = bf16_lo(v[0].z); a[5] = bf16_hi(v[0].z);
  a[6] = bf16_lo(v[0].w); a[7] = bf16_hi(v[0].w);
#pragma unroll
  for (int r = 1; r < R; ++r) {
    a[0] = a[0] + bf16_lo(v[r].x); a[1] = a[1] + bf16_hi(v[r].x);
    a[2] = a[2] + bf16_lo(v[r].y); a[3] = a[3] + bf16_hi(v[r].y);
    a[4] = a[4] + bf16_lo(v[r].z); a[5] = a[5] + bf16_hi(v[r].z);
    a[6] = a[6] + bf16_lo(v[r].w); a[7] = a[7] + bf16_hi(v[r].w);
  }
  return pack_bf16x8(a);
}

// Tree-order sum of R fp32 terms held in t[] (overwritten): pairwise, level
// by level -- at stride s the partial sum at index i (a multiple of 2s) takes
// in the one at i + s when that exists -- so adjacent items pair up and an odd
// last item passes up unchanged; R = 8 gives ((0+1)+(2+3))+((4+5)+(6+7)).
// Every index is a compile-time constant after unrolling (registers only).
template <int R>
__device__ __forceinline__ float tree_sum(float (&t)[R]) {
#pragma unroll
  for (int s = 1; s < R; s *= 2) {
#pragma unroll
    for (int i = 0; i + s < R; i += 2 * s) t[i] = t[i] + t[i + s];
  }
  return t[0];
}

// The same tree for a run-time rank count n <= N (predicated, still in
// registers).
template <int N>
__device__ __forceinline__ float tree_sum_n(float (&t)[N], int n) {
#pragma unroll
  for (int s = 1; s < N; s *= 2) {
#pragma unroll
    for (int i = 0; i + s < N; i += 2 * s)
      if (i + s < n) t[i] = t[i] + t[i + s];
  }
  return t[0];
}

// Tree-order fold of 8 bf16 lanes from R sources, one rounding at the end.
template <int R>
__device__ __forceinline__ uint4 fold_tree_bf16x8(const uint4 (&v)[R]) {
  float s[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float t[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t w = k < 2 ? v[r].x : k < 4 ? v[r].y : k < 6 ? v[r].z : v[r].w;
      t[r] = (k & 1) ? bf16_hi(w) : bf16_lo(w);
    }
    s[k] = tree_sum<R>(t);
  }
  return pack_bf16x8(s);
}

template <int R>
__device__ __forceinline__ uint4 fold_tree_f32x4(const uint4 (&v)[R]) {
  float s[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float t[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      t[r] = __uint_as_float(k == 0 ? v[r].x : k == 1 ? v[r].y : k == 2 ? v[r].z : v[r].w);
    s[k] = tree_sum<R>(t);
  }
  uint4 o;
  o.x = __float_as_uint(s[0]);
  o.y = __float_as_uint(s[1]);
  o.z = __float_as_uint(s[2]);
  o.w = __float_as_uint(s[3]);
  return o;
}

template <int R>
__device__ __forceinline__ uint4 fold_f32x4(const uint4 (&v)[R]) {
  float a0 = __uint_as_float(v[0].x), a1 = __uint_as_float(v[0].y);
  float a2 = __uint_as_float(v[0].z), a3 = __uint_as_float(v[0].w);
#pragma unroll
  for (int r = 1; r < R; ++r) {
    a0 = a0 + __uint_as_float(v[r].x);
    a1 = a1 + __uint_as_float(v[r].y);
    a2 = a2 + __uint_as_float(v[r].z);
    a3 = a3 + __uint_as_float(v[r].w);
  }
  uint4 o;
  o.x = __float_as_uint(a0);
  o.y = __float_as_uint(a1);
  o.z = __float_as_uint(a2);
  o.w = __float_as_uint(a3);
  return o;
}

// One 16-byte vector of R sources in the fixed rank order or in tree order.
template <int R, bool BF16, bool TREE>
__device__ __forceinline__ uint4 fold_vec(const uint4 (&v)[R]) {
  if (TREE) return BF16 ? fold_tree_bf16x8<R>(v) : fold_tree_f32x4<R>(v);
  return BF16 ? fold_bf16x8<R>(v) : fold_f32x4<R>(v);
}

}  // namespace rrb
