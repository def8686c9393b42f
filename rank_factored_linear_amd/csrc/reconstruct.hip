// reconstruct_weight: w_out = diag(s) . W0 + U . V^T  ("The theta bundle",
// component table and reconstruction formula).
//
// rank 0 is a pure scaled copy, bound by HBM: each thread rebuilds 8
// consecutive elements of one row (16-byte loads, 16/32-byte stores).
// rank > 0 is a K = rank GEMM (U rows and V rows are both contiguous along
// the rank dimension) on the matrix cores with the scaled copy fused into the
// epilogue; at rank 256 it is still HBM-bound but needs far more than the
// fp32 vector rate to keep up with HBM.
#include "tb_device.h"
#include "tb_host.h"

namespace tb {

namespace {

constexpr int kThreads = 256;

template <typename EI, typename EO>
__global__ __launch_bounds__(kThreads) void reconstruct_rank0_kernel(const EI* __restrict__ s, const EI* __restrict__ w0,
                                                                     EO* __restrict__ out, int64_t n8, int I) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t c = int64_t(blockIdx.x) * kThreads + threadIdx.x; c < n8; c += stride) {
    const int64_t base = c * 8;
    const int64_t o = base / I;
    const float sc = to_f32<EI>(s[o]);
    float v[8];
    if constexpr (sizeof(EI) == 2) {
      const uint4 q = *reinterpret_cast<const uint4*>(w0 + base);
      const uint32_t u4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = sc * bf16_to_f32(uint16_t(u4[e / 2] >> (16 * (e % 2))));
    } else {
      const float4 lo = reinterpret_cast<const float4*>(w0 + base)[0];
      const float4 hi = reinterpret_cast<const float4*>(w0 + base)[1];
      v[0] = sc * lo.x; v[1] = sc * lo.y; v[2] = sc * lo.z; v[3] = sc * lo.w;
      v[4] = sc * hi.x; v[5] = sc * hi.y; v[6] = sc * hi.z; v[7] = sc * hi.w;
    }
    if constexpr (sizeof(EO) == 4) {
      float4* dst = reinterpret_cast<float4*>(out + base);
      dst[0] = make_float4(v[0], v[1], v[2], v[3]);
      dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      *reinterpret_cast<uint4*>(out + base) =
          make_uint4(f32_to_bf16(v[0]) | (uint32_t(f32_to_bf16(v[1])) << 16), f32_to_bf16(v[2]) | (uint32_t(f32_to_bf16(v[3])) << 16),
                     f32_to_bf16(v[4]) | (uint32_t(f32_to_bf16(v[5])) << 16), f32_to_bf16(v[6]) | (uint32_t(f32_to_bf16(v[7])) << 16));
    }
  }
}

// Workgroup tile: 64 rows x 64 columns; wave w owns rows 16w..16w+15.
template <typename EI, typename EO>
__global__ __launch_bounds__(kThreads) void reconstruct_lowrank_kernel(const EI* __restrict__ s, const EI* __restrict__ w0,
                                                                       const EI* __restrict__ u, const EI* __restrict__ v,
                                                                       EO* __restrict__ out, int O, int I, int R) {
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int lr = l & 15, kq = (l >> 4) * 8;
  const int i0 = blockIdx.x * 64, o0 = blockIdx.y * 64 + w * 16;
  const bool aligned = (R % 8) == 0;
  f32x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int urow = o0 + lr;
  for (int kk = 0; kk < R; kk += 32) {
    const int j = kk + kq;
    Frag8<EI> fa = zero_frag<EI>();
    if (urow < O && j < R)
      fa = aligned ? load_frag<EI>(u + size_t(urow) * R + j) : load_frag_partial<EI>(u + size_t(urow) * R + j, min(8, R - j));
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int vrow = i0 + ct * 16 + lr;
      Frag8<EI> fb = zero_frag<EI>();
      if (vrow < I && j < R)
        fb = aligned ? load_frag<EI>(v + size_t(vrow) * R + j) : load_frag_partial<EI>(v + size_t(vrow) * R + j, min(8, R - j));
      acc[ct] = mma_k32(fa, fb, acc[ct]);
      __builtin_amdgcn_sched_barrier(0);
      mfma_operand_guard();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int o = o0 + (l >> 4) * 4 + e;
    if (o >= O) continue;
    const float sc = to_f32<EI>(s[o]);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int i = i0 + ct * 16 + lr;
      if (i < I) out[size_t(o) * I + i] = from_f32<EO>(acc[ct][e] + sc * to_f32<EI>(w0[size_t(o) * I + i]));
    }
  }
}

template <typename EI, typename EO>
hipError_t launch_typed(const void* s, const void* w0, const void* u, const void* v, void* w_out, int64_t O, int64_t I,
                        int64_t R, hipStream_t stream) {
  if (R == 0) {
    const int64_t n8 = O * I / 8;
    int64_t blocks = (n8 + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL((reconstruct_rank0_kernel<EI, EO>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       static_cast<const EI*>(s), static_cast<const EI*>(w0), static_cast<EO*>(w_out), n8, int(I));
  } else {
    dim3 grid(unsigned((I + 63) / 64), unsigned((O + 63) / 64));
    hipLaunchKernelGGL((reconstruct_lowrank_kernel<EI, EO>), grid, dim3(kThreads), 0, stream, static_cast<const EI*>(s),
                       static_cast<const EI*>(w0), static_cast<const EI*>(u), static_cast<const EI*>(v),
                       static_cast<EO*>(w_out), int(O), int(I), int(R));
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reconstruct(tb_dtype in_dtype, tb_dtype out_dtype, const void* s, const void* w0, const void* u,
                              const void* v, void* w_out, int64_t out_dim, int64_t in_dim, int64_t rank,
                              hipStream_t stream) {
  if (in_dtype == TB_BF16) {
    if (out_dtype == TB_F32) return launch_typed<bf16_t, float>(s, w0, u, v, w_out, out_dim, in_dim, rank, stream);
    return launch_typed<bf16_t, bf16_t>(s, w0, u, v, w_out, out_dim, in_dim, rank, stream);
  }
  if (out_dtype == TB_F32) return launch_typed<float, float>(s, w0, u, v, w_out, out_dim, in_dim, rank, stream);
  return launch_typed<float, bf16_t>(s, w0, u, v, w_out, out_dim, in_dim, rank, stream);
}

}  // namespace tb
