// Deterministic grid-wide sum of (num, den) pairs, used by the relative
// Frobenius error kernels: each workgroup reduces its threads in a fixed tree
// order and publishes one partial pair; the last workgroup to count itself in
// sums the partials in workgroup order and writes the ratio
// sqrt(num) / sqrt(den) (0 when num is 0, +inf when only den is 0).
//
// Workspace: partial pairs first; its last kCounterBytes hold the arrival
// counters.  Workgroup b counts itself into group counter b % kGroups (256
// bytes apart); the last of a group bumps a top counter.  Thousands of
// increments of one word serialise at the memory side (~20 us), 16 groups do
// not.  Every counter is cleared by its last user, so the counter area must
// be zero before the first use and stays zero after every call.  Partials and
// counters move through device-scope (sc1) accesses, coherent across XCDs; a
// workgroup drains its partial before it counts itself in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tb.h"

namespace tb {
namespace reduce {

constexpr int kGroups = 16;
constexpr int kCounterBytes = 8192;
constexpr int kMaxPartials = (TB_FROBENIUS_WORKSPACE_BYTES - kCounterBytes) / 16;
static_assert(256 * (kGroups + 1) <= kCounterBytes, "counters fit their area");

__device__ __forceinline__ uint64_t load_coherent64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Fixed-order tree over the workgroup's NT threads (sa, sb: NT doubles of LDS each).
template <int NT>
__device__ __forceinline__ void block_reduce2(double& a, double& b, double* sa, double* sb) {
  const int tid = threadIdx.x;
  sa[tid] = a;
  sb[tid] = b;
  __syncthreads();
  for (int h = NT / 2; h > 0; h >>= 1) {
    if (tid < h) {
      sa[tid] += sa[tid + h];
      sb[tid] += sb[tid + h];
    }
    __syncthreads();
  }
  a = sa[0];
  b = sb[0];
  __syncthreads();
}

__host__ __device__ inline uint64_t* partials(void* workspace) { return static_cast<uint64_t*>(workspace); }
__host__ __device__ inline unsigned* counters(void* workspace) {
  return reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + TB_FROBENIUS_WORKSPACE_BYTES - kCounterBytes);
}

// Publishes this workgroup's (num, den) and, in the last workgroup to arrive,
// writes the ratio.  Every thread of the workgroup calls it with the same
// (already reduced) values.  s_last: one word of LDS for the arrival verdict.
template <int NT>
__device__ void finish_ratio(double num, double den, uint64_t* __restrict__ partial, unsigned* __restrict__ counters,
                             double* __restrict__ result, double* sa, double* sb, unsigned& s_last) {
  if (threadIdx.x == 0) {
    store_coherent64(&partial[2 * blockIdx.x], __double_as_longlong(num));
    store_coherent64(&partial[2 * blockIdx.x + 1], __double_as_longlong(den));
    __builtin_amdgcn_s_waitcnt(0);  // the partial is visible before the count
    const unsigned nb = gridDim.x, groups = nb < unsigned(kGroups) ? nb : unsigned(kGroups);
    const unsigned g = blockIdx.x % groups, members = (nb - g + groups - 1) / groups;
    unsigned* gc = counters + 64 * g;
    unsigned* top = counters + 64 * kGroups;
    bool last = false;
    if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
      __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == groups - 1) {
        __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = true;
      }
    }
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  double n = 0.0, d = 0.0;
  for (int i = threadIdx.x; i < int(gridDim.x); i += NT) {
    n += __longlong_as_double(load_coherent64(&partial[2 * i]));
    d += __longlong_as_double(load_coherent64(&partial[2 * i + 1]));
  }
  block_reduce2<NT>(n, d, sa, sb);
  if (threadIdx.x == 0) {
    double r;
    if (n == 0.0) r = 0.0;
    else if (d == 0.0) r = __builtin_inf();
    else r = sqrt(n) / sqrt(d);
    *result = r;
  }
}

template <int NT>
__device__ void finish_ratio(double num, double den, uint64_t* __restrict__ partial, unsigned* __restrict__ counters,
                             double* __restrict__ result, double* sa, double* sb) {
  __shared__ unsigned s_last;
  finish_ratio<NT>(num, den, partial, counters, result, sa, sb, s_last);
}

}  // namespace reduce
}  // namespace tb
