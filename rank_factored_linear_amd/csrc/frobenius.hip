// relative_frobenius_error(original, reconstructed) =
//     ||original - reconstructed||_F / ||original||_F
// ("Quality", section "Reconstruction error").
//
// One launch, no floating-point atomics, so the result is the same on every
// run: each workgroup walks a grid-stride set of 8-element chunks and sums
// (a - b)^2 and a^2 in fp64 (differences taken in fp64), then the grid-wide
// fixed-order sum of tb_reduce.h writes the ratio.
// HBM-bound: every element of both matrices is read once.
#include "tb_device.h"
#include "tb_host.h"
#include "tb_reduce.h"

namespace tb {

namespace {

constexpr int kThreads = 256;

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

template <typename E>
__global__ __launch_bounds__(kThreads) void frob_kernel(const E* __restrict__ a, const E* __restrict__ b, int64_t n8,
                                                        uint64_t* __restrict__ partial, unsigned* __restrict__ counters,
                                                        double* __restrict__ result) {
  __shared__ double sa[kThreads], sb[kThreads];
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
  reduce::block_reduce2<kThreads>(num, den, sa, sb);
  reduce::finish_ratio<kThreads>(num, den, partial, counters, result, sa, sb);
}

}  // namespace

hipError_t launch_frobenius(tb_dtype dtype, const void* a, const void* b, int64_t n, double* result, void* workspace,
                            int cus, hipStream_t stream) {
  const int64_t n8 = n / 8;
  int64_t blocks = (n8 + kThreads - 1) / kThreads;
  const int64_t cap = int64_t(cus) * 8 < reduce::kMaxPartials ? int64_t(cus) * 8 : reduce::kMaxPartials;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  uint64_t* partial = reduce::partials(workspace);
  unsigned* counters = reduce::counters(workspace);
  if (dtype == TB_BF16)
    hipLaunchKernelGGL(frob_kernel<bf16_t>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(b), n8, partial, counters, result);
  else
    hipLaunchKernelGGL(frob_kernel<float>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       static_cast<const float*>(a), static_cast<const float*>(b), n8, partial, counters, result);
  return hipGetLastError();
}

}  // namespace tb
