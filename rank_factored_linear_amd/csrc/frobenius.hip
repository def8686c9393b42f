// relative_frobenius_error(original, reconstructed) =
//     ||original - reconstructed||_F / ||original||_F
// ("Quality", section "Reconstruction error").
//
// One launch, no floating-point atomics, so the result is the same on every
// run: each workgroup walks a grid-stride set of 8-element chunks and sums
// (a - b)^2 and a^2 in fp64 (differences taken in fp64), reduces its threads
// in a fixed tree order into one partial pair and publishes it; the last
// workgroup to count itself in sums the partial pairs in workgroup order and
// writes the ratio (0 when the difference is zero, +inf when only the
// original is zero).  Counting in goes through 16 group counters (workgroup
// b into counter b % 16, 256 bytes apart) and one top counter that the last
// of each group bumps: thousands of increments of one word serialise at the
// memory side for ~20 us.  Every counter is cleared by its last user.
// Partials and the counter move through device-scope (sc1) accesses, coherent
// across XCDs; a workgroup drains its partial before it counts itself in.
// HBM-bound: every element of both matrices is read once.
#include "tb_device.h"
#include "tb_host.h"

namespace tb {

namespace {

constexpr int kThreads = 256;
// The workspace holds the partial pairs; its last 8 KB hold the counters
// (group g at byte 256 g, the top counter at byte 256 * kGroups).
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

template <typename E>
__device__ __forceinline__ void load8_f64(const E* p, double* out) {
  if constexpr (sizeof(E) == 2) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t u4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = double(bf16_to_f32(uint16_t(u4[e / 2] >> (16 * (e % 2)))));
  } else {
    const float4 lo = reinterpret_cast<const float4*>(p)[0];
    const float4 hi = reinterpret_cast<const float4*>(p)[1];
    out[0] = lo.x; out[1] = lo.y; out[2] = lo.z; out[3] = lo.w;
    out[4] = hi.x; out[5] = hi.y; out[6] = hi.z; out[7] = hi.w;
  }
}

__device__ __forceinline__ void block_reduce2(double& a, double& b, double* sa, double* sb) {
  const int tid = threadIdx.x;
  sa[tid] = a;
  sb[tid] = b;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if (tid < h) {
      sa[tid] += sa[tid + h];
      sb[tid] += sb[tid + h];
    }
    __syncthreads();
  }
  a = sa[0];
  b = sb[0];
}

template <typename E>
__global__ __launch_bounds__(kThreads) void frob_kernel(const E* __restrict__ a, const E* __restrict__ b, int64_t n8,
                                                        uint64_t* __restrict__ partial, unsigned* __restrict__ counters,
                                                        double* __restrict__ result) {
  __shared__ double sa[kThreads], sb[kThreads];
  __shared__ unsigned s_last;
  double num = 0.0, den = 0.0;
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t c = int64_t(blockIdx.x) * kThreads + threadIdx.x; c < n8; c += stride) {
    double va[8], vb[8];
    load8_f64<E>(a + c * 8, va);
    load8_f64<E>(b + c * 8, vb);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double d = va[e] - vb[e];
      num += d * d;
      den += va[e] * va[e];
    }
  }
  block_reduce2(num, den, sa, sb);
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
  num = 0.0;
  den = 0.0;
  for (int i = threadIdx.x; i < int(gridDim.x); i += kThreads) {
    num += __longlong_as_double(load_coherent64(&partial[2 * i]));
    den += __longlong_as_double(load_coherent64(&partial[2 * i + 1]));
  }
  block_reduce2(num, den, sa, sb);
  if (threadIdx.x == 0) {
    double r;
    if (num == 0.0) r = 0.0;
    else if (den == 0.0) r = __builtin_inf();
    else r = sqrt(num) / sqrt(den);
    *result = r;
  }
}

}  // namespace

hipError_t launch_frobenius(tb_dtype dtype, const void* a, const void* b, int64_t n, double* result, void* workspace,
                            int cus, hipStream_t stream) {
  const int64_t n8 = n / 8;
  int64_t blocks = (n8 + kThreads - 1) / kThreads;
  const int64_t cap = int64_t(cus) * 8 < kMaxPartials ? int64_t(cus) * 8 : kMaxPartials;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  uint64_t* partial = static_cast<uint64_t*>(workspace);
  unsigned* counters =
      reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + TB_FROBENIUS_WORKSPACE_BYTES - kCounterBytes);
  if (dtype == TB_BF16)
    hipLaunchKernelGGL(frob_kernel<bf16_t>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(b), n8, partial, counters, result);
  else
    hipLaunchKernelGGL(frob_kernel<float>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       static_cast<const float*>(a), static_cast<const float*>(b), n8, partial, counters, result);
  return hipGetLastError();
}

}  // namespace tb
