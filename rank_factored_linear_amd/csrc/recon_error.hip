// relative_frobenius_error(original, reconstruct_weight(s, W0, U, V)) without
// writing the rebuilt weight ("The theta bundle", reconstruction formula;
// "Quality", section "Reconstruction error").
//
// Each rebuilt entry is formed in fp32 exactly as the reconstruct kernels
// form it (the rank-r product accumulated in fp32 on the matrix cores, plus
// s[o] * W0[o][i]), then compared with the original in fp64: differences,
// squares and sums in fp64, and the grid-wide fixed-order sum of tb_reduce.h.
// Reading W0, U, V, s and the original once, it moves 6 bytes per element
// (bf16 bundle, fp32 original) where rebuilding W and then comparing moves 14.
#include "tb_device.h"
#include "tb_host.h"
#include "tb_rebuild.h"
#include "tb_reduce.h"

namespace tb {

namespace {

constexpr int kThreads = rebuild::kThreads;

template <typename EO>
__device__ __forceinline__ void load4(const EO* p, float (&o)[4]) {
  if constexpr (sizeof(EO) == 4) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    o[0] = q.x; o[1] = q.y; o[2] = q.z; o[3] = q.w;
  } else {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    o[0] = bf16_to_f32(uint16_t(q.x)); o[1] = bf16_to_f32(uint16_t(q.x >> 16));
    o[2] = bf16_to_f32(uint16_t(q.y)); o[3] = bf16_to_f32(uint16_t(q.y >> 16));
  }
}

__device__ __forceinline__ void add_err(double orig, float rebuilt, double& num, double& den) {
  const double d = orig - double(rebuilt);
  num += d * d;
  den += orig * orig;
}

// bf16 bundles, rank % 8 == 0: 128 x 128 tiles (tb_rebuild.h), grid-stride.
template <typename EO>
__global__ __launch_bounds__(kThreads, 2) void rerr_t128_kernel(const bf16_t* __restrict__ s,
                                                                 const bf16_t* __restrict__ w0,
                                                                 const bf16_t* __restrict__ u,
                                                                 const bf16_t* __restrict__ v,
                                                                 const EO* __restrict__ orig, int O, int I, int R,
                                                                 int tiles_i, int tiles, uint64_t* partial,
                                                                 unsigned* counters, double* result) {
  namespace t = rebuild::t128;
  __shared__ __attribute__((aligned(16))) unsigned char lds[t::kLdsBytes];
  __shared__ double sa[kThreads], sb[kThreads];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int wi = w & 1, wo = w >> 1, h = l >> 5, lr = l & 31;
  double num = 0.0, den = 0.0;
  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int bo = tile / tiles_i, o0 = bo * t::BT, i0 = (tile - bo * tiles_i) * t::BT;
    t::f32x16 acc[2][2];
    t::product(u, v, O, I, R, o0, i0, lds, acc);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int o = o0 + wo * 64 + cb * 32 + lr;
      if (o >= O) continue;
      const float so = bf16_to_f32(s[o].bits);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = i0 + wi * 64 + rb * 32 + 8 * b + 4 * h;   // I % 8 == 0: i < I covers i .. i+3
          if (i >= I) continue;
          const uint2 wv = *reinterpret_cast<const uint2*>(w0 + size_t(o) * I + i);
          float ov[4];
          load4<EO>(orig + size_t(o) * I + i, ov);
          const t::f32x16& c = acc[rb][cb];
          add_err(ov[0], c[4 * b + 0] + so * bf16_to_f32(uint16_t(wv.x)), num, den);
          add_err(ov[1], c[4 * b + 1] + so * bf16_to_f32(uint16_t(wv.x >> 16)), num, den);
          add_err(ov[2], c[4 * b + 2] + so * bf16_to_f32(uint16_t(wv.y)), num, den);
          add_err(ov[3], c[4 * b + 3] + so * bf16_to_f32(uint16_t(wv.y >> 16)), num, den);
        }
    }
  }
  reduce::block_reduce2<kThreads>(num, den, sa, sb);
  reduce::finish_ratio<kThreads>(num, den, partial, counters, result, sa, sb);
}

// Any element type and rank: 64 x 64 tiles with fragments from global memory.
template <typename EI, typename EO>
__global__ __launch_bounds__(kThreads) void rerr_t64_kernel(const EI* __restrict__ s, const EI* __restrict__ w0,
                                                            const EI* __restrict__ u, const EI* __restrict__ v,
                                                            const EO* __restrict__ orig, int O, int I, int R,
                                                            int tiles_i, int tiles, uint64_t* partial,
                                                            unsigned* counters, double* result) {
  namespace t = rebuild::t64;
  __shared__ double sa[kThreads], sb[kThreads];
  const int l = threadIdx.x % kWave, w = threadIdx.x / kWave;
  double num = 0.0, den = 0.0;
  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int bo = tile / tiles_i, o0 = bo * t::BT, i0 = (tile - bo * tiles_i) * t::BT;
    f32x4 acc[4];
    t::product<EI>(u, v, O, I, R, o0, i0, acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int o = o0 + w * 16 + (l >> 4) * 4 + e;
      if (o >= O) continue;
      const float sc = to_f32<EI>(s[o]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int i = i0 + ct * 16 + (l & 15);
        if (i < I)
          add_err(double(to_f32<EO>(orig[size_t(o) * I + i])), acc[ct][e] + sc * to_f32<EI>(w0[size_t(o) * I + i]), num,
                  den);
      }
    }
  }
  reduce::block_reduce2<kThreads>(num, den, sa, sb);
  reduce::finish_ratio<kThreads>(num, den, partial, counters, result, sa, sb);
}

// Rank 0: the rebuilt weight is s[o] * W0[o][i]; each wave covers 256
// consecutive elements per step (lane l: 4 l .. 4 l + 3), grid-stride.
template <typename EI, typename EO>
__global__ __launch_bounds__(kThreads) void rerr_rank0_kernel(const EI* __restrict__ s, const EI* __restrict__ w0,
                                                              const EO* __restrict__ orig, int64_t n, int I,
                                                              uint64_t* partial, unsigned* counters, double* result) {
  __shared__ double sa[kThreads], sb[kThreads];
  const int l = threadIdx.x & 63;
  const int64_t waves = int64_t(gridDim.x) * (kThreads / kWave);
  double num = 0.0, den = 0.0;
  for (int64_t wv = int64_t(blockIdx.x) * (kThreads / kWave) + (threadIdx.x >> 6); wv * 256 < n; wv += waves) {
    const int64_t base = wv * 256 + l * 4;   // I % 8 == 0: the four share a row
    if (base >= n) continue;
    const float sc = to_f32<EI>(s[base / I]);
    float wv4[4], ov[4];
    if constexpr (sizeof(EI) == 2) {
      const uint2 q = *reinterpret_cast<const uint2*>(w0 + base);
      wv4[0] = bf16_to_f32(uint16_t(q.x)); wv4[1] = bf16_to_f32(uint16_t(q.x >> 16));
      wv4[2] = bf16_to_f32(uint16_t(q.y)); wv4[3] = bf16_to_f32(uint16_t(q.y >> 16));
    } else {
      const float4 q = *reinterpret_cast<const float4*>(w0 + base);
      wv4[0] = q.x; wv4[1] = q.y; wv4[2] = q.z; wv4[3] = q.w;
    }
    load4<EO>(orig + base, ov);
#pragma unroll
    for (int e = 0; e < 4; ++e) add_err(ov[e], sc * wv4[e], num, den);
  }
  reduce::block_reduce2<kThreads>(num, den, sa, sb);
  reduce::finish_ratio<kThreads>(num, den, partial, counters, result, sa, sb);
}

int64_t cap_grid(int64_t want, int64_t per_cu, int cus) {
  int64_t g = want;
  if (g > per_cu * cus) g = per_cu * cus;
  if (g > reduce::kMaxPartials) g = reduce::kMaxPartials;
  return g < 1 ? 1 : g;
}

template <typename EI, typename EO>
hipError_t launch_typed(const void* s, const void* w0, const void* u, const void* v, const void* orig, int64_t O,
                        int64_t I, int64_t R, double* result, void* workspace, int cus, hipStream_t stream) {
  uint64_t* partial = reduce::partials(workspace);
  unsigned* counters = reduce::counters(workspace);
  const EI* s_ = static_cast<const EI*>(s);
  const EI* w_ = static_cast<const EI*>(w0);
  const EO* o_ = static_cast<const EO*>(orig);
  if (R == 0) {
    const int64_t grid = cap_grid((O * I + 1023) / 1024, 8, cus);
    hipLaunchKernelGGL((rerr_rank0_kernel<EI, EO>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, s_, w_, o_, O * I,
                       int(I), partial, counters, result);
  } else if (sizeof(EI) == 2 && R % 8 == 0) {
    const int tiles_i = int((I + 127) / 128), tiles = tiles_i * int((O + 127) / 128);
    const int64_t grid = cap_grid(tiles, 2, cus);
    hipLaunchKernelGGL((rerr_t128_kernel<EO>), dim3(unsigned(grid)), dim3(kThreads), 0, stream,
                       reinterpret_cast<const bf16_t*>(s), reinterpret_cast<const bf16_t*>(w0),
                       static_cast<const bf16_t*>(u), static_cast<const bf16_t*>(v), o_, int(O), int(I), int(R), tiles_i,
                       tiles, partial, counters, result);
  } else {
    const int tiles_i = int((I + 63) / 64), tiles = tiles_i * int((O + 63) / 64);
    const int64_t grid = cap_grid(tiles, 4, cus);
    hipLaunchKernelGGL((rerr_t64_kernel<EI, EO>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, s_, w_,
                       static_cast<const EI*>(u), static_cast<const EI*>(v), o_, int(O), int(I), int(R), tiles_i, tiles,
                       partial, counters, result);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reconstruction_error(tb_dtype bundle_dtype, tb_dtype orig_dtype, const void* s, const void* w0,
                                       const void* u, const void* v, const void* orig, int64_t out_dim, int64_t in_dim,
                                       int64_t rank, double* result, void* workspace, int cus, hipStream_t stream) {
  if (bundle_dtype == TB_BF16) {
    if (orig_dtype == TB_F32 && persistent_error_supported(out_dim, in_dim, rank))
      return launch_reconstruction_error_persistent(s, w0, u, v, static_cast<const float*>(orig), out_dim, in_dim, rank,
                                                    result, workspace, cus, stream);
    if (orig_dtype == TB_F32)
      return launch_typed<bf16_t, float>(s, w0, u, v, orig, out_dim, in_dim, rank, result, workspace, cus, stream);
    return launch_typed<bf16_t, bf16_t>(s, w0, u, v, orig, out_dim, in_dim, rank, result, workspace, cus, stream);
  }
  if (orig_dtype == TB_F32)
    return launch_typed<float, float>(s, w0, u, v, orig, out_dim, in_dim, rank, result, workspace, cus, stream);
  return launch_typed<float, bf16_t>(s, w0, u, v, orig, out_dim, in_dim, rank, result, workspace, cus, stream);
}

}  // namespace tb
