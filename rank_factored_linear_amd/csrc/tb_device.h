// Device-side helpers shared by the gfx950 kernels of libtb.
//
// Fragments follow the CDNA matrix-core layout for 16x16 output tiles:
//   A operand (16 x K):  lane l holds row (l % 16), k = 8 * (l / 16) + 0..7
//   B operand (K x 16):  lane l holds col (l % 16), k = 8 * (l / 16) + 0..7
//   C / D (16 x 16):     lane l holds rows 4 * (l / 16) + 0..3, col (l % 16)
// A "k32 step" feeds 32 consecutive k to a 16x16 tile: one
// v_mfma_f32_16x16x32_bf16 for bf16, eight v_mfma_f32_16x16x4_f32 for fp32
// (the eight k of a lane are spread over the eight instructions; the sum over
// k does not depend on which instruction adds which k).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tb {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct bf16_t { uint16_t bits; };

// Eight consecutive elements of one row, as loaded by one lane.
template <typename E> struct Frag8;
template <> struct Frag8<bf16_t> { uint4 v; };
template <> struct Frag8<float> { float4 lo, hi; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  // Round to nearest, ties to even (the inputs here are finite).
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <typename E> __device__ __forceinline__ float to_f32(E v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v.bits); }

template <typename E> __device__ __forceinline__ E from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return bf16_t{f32_to_bf16(f)}; }

template <typename E> __device__ __forceinline__ Frag8<E> zero_frag() {
  Frag8<E> f;
  if constexpr (sizeof(E) == 2) f.v = make_uint4(0, 0, 0, 0);
  else { f.lo = make_float4(0.f, 0.f, 0.f, 0.f); f.hi = f.lo; }
  return f;
}

// 16-byte aligned vector load of 8 elements (p must be 16-byte aligned).
template <typename E> __device__ __forceinline__ Frag8<E> load_frag(const E* p) {
  Frag8<E> f;
  if constexpr (sizeof(E) == 2) f.v = *reinterpret_cast<const uint4*>(p);
  else { f.lo = reinterpret_cast<const float4*>(p)[0]; f.hi = reinterpret_cast<const float4*>(p)[1]; }
  return f;
}

template <typename E> __device__ __forceinline__ Frag8<E> load_frag_if(const E* p, bool ok) {
  return ok ? load_frag<E>(p) : zero_frag<E>();
}

// Element-wise load of up to 8 elements (n valid), for rows that are not
// 16-byte aligned or are cut short.
template <typename E> __device__ __forceinline__ Frag8<E> load_frag_partial(const E* p, int n) {
  Frag8<E> f = zero_frag<E>();
  if constexpr (sizeof(E) == 2) {
    uint16_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    for (int e = 0; e < 8; ++e) if (e < n) h[e] = q[e];
    f.v = make_uint4(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16),
                     h[4] | (uint32_t(h[5]) << 16), h[6] | (uint32_t(h[7]) << 16));
  } else {
    float t[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int e = 0; e < 8; ++e) if (e < n) t[e] = p[e];
    f.lo = make_float4(t[0], t[1], t[2], t[3]);
    f.hi = make_float4(t[4], t[5], t[6], t[7]);
  }
  return f;
}

// Eight fp32 values converted to the operand type of E (bf16 rounds).
template <typename E> __device__ __forceinline__ Frag8<E> frag_from_f32(const float* t8);
template <> __device__ __forceinline__ Frag8<float> frag_from_f32<float>(const float* t) {
  Frag8<float> f;
  f.lo = make_float4(t[0], t[1], t[2], t[3]);
  f.hi = make_float4(t[4], t[5], t[6], t[7]);
  return f;
}
template <> __device__ __forceinline__ Frag8<bf16_t> frag_from_f32<bf16_t>(const float* t) {
  Frag8<bf16_t> f;
  f.v = make_uint4(f32_to_bf16(t[0]) | (uint32_t(f32_to_bf16(t[1])) << 16),
                   f32_to_bf16(t[2]) | (uint32_t(f32_to_bf16(t[3])) << 16),
                   f32_to_bf16(t[4]) | (uint32_t(f32_to_bf16(t[5])) << 16),
                   f32_to_bf16(t[6]) | (uint32_t(f32_to_bf16(t[7])) << 16));
  return f;
}

// acc += A(16 x 32) * B(32 x 16) for one k32 step.
__device__ __forceinline__ f32x4 mma_k32(const Frag8<bf16_t>& a, const Frag8<bf16_t>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v), __builtin_bit_cast(bf16x8, b.v), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k32(const Frag8<float>& a, const Frag8<float>& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, c, 0, 0, 0);
  return c;
}

// Wait states after a group of matrix-core ops whose A/B registers the
// following code may rewrite at once: the write-after-read rule for
// matrix-core source operands (a VGPR that an issued op still reads must not
// be overwritten before the op has read it).  In a chain of 16x16x32 ops that
// accumulate into the same registers, an ALU write to the A or B register of
// an op right behind it gave wrong products on gfx950 (the compiler put no
// wait states there); 24 wait states after each group removed every error.
// 24 is empirical (the smallest count tried that did), with room for 16-pass
// ops.
__device__ __forceinline__ void mfma_operand_guard() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: ); }

// Agent-scope read-modify-write with acquire/release semantics.  On gfx950
// the release and acquire parts write back and invalidate the XCD's L2, so
// only a handful of workgroups per launch may use it.
__device__ __forceinline__ unsigned atomic_add_agent(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace tb
