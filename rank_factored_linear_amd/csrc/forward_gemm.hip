// Theta-bundle projection for many tokens (bf16, m > 64): two launches.
//
//   1. T = x . V                    [m, r], rounded to bf16 into the workspace
//   2. y = s (.) (x . W0^T) + T . U^T
//
// ("The theta bundle": the transpose of weight = diag(s) W0 + U V^T applied
// to x.)  Step 2 is a matrix-core GEMM whose operands are both contiguous
// along the reduction dimension (x rows over in_dim, W0 rows over in_dim).
// Tiles of x and W0 are staged through LDS with double buffering: the global
// loads for step k+1 are in flight while the matrix cores work on step k.
// The epilogue scales each output column by s in fp32 and then continues the
// same accumulators over the rank dimension with T and U (both contiguous
// along r), so the rank-r delta costs r/in_dim extra reduction steps and no
// extra pass over y.
#include "tb_device.h"
#include "tb_host.h"

namespace tb {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// T = x . V.  V is [in_dim, r] with r contiguous, so a 32 x 64 tile of V is
// staged in LDS transposed (each lane then reads 8 consecutive in_dim values
// of one column as its B fragment).  Workgroup tile: 64 tokens x 64 columns.
// ---------------------------------------------------------------------------
constexpr int kTM = 64, kTN = 64, kTPitch = 40;  // LDS pitch in elements (80 B)

__global__ __launch_bounds__(kThreads) void xv_gemm_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ v,
                                                           bf16_t* __restrict__ t, int M, int I, int R) {
  __shared__ uint16_t vt[kTN * kTPitch];
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int lr = l & 15, kq = (l >> 4) * 8;
  const int m0 = blockIdx.x * kTM, j0 = blockIdx.y * kTN;
  const int kr = tid / 8, jc = (tid % 8) * 8;  // V staging: row kr of the tile, columns jc..jc+7
  const bool aligned = (R % 8) == 0;
  const int arow = m0 + w * 16 + lr;
  f32x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < I; k0 += 32) {
    Frag8<bf16_t> fv = zero_frag<bf16_t>();
    const int vi = k0 + kr, vj = j0 + jc;
    if (vi < I && vj < R)
      fv = aligned ? load_frag<bf16_t>(v + size_t(vi) * R + vj) : load_frag_partial<bf16_t>(v + size_t(vi) * R + vj, min(8, R - vj));
    const Frag8<bf16_t> fx = load_frag_if<bf16_t>(x + size_t(arow) * I + k0 + kq, arow < M && k0 + kq < I);
    __syncthreads();  // previous step's reads of vt are done
    const uint32_t wv[4] = {fv.v.x, fv.v.y, fv.v.z, fv.v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[(jc + e) * kTPitch + kr] = uint16_t(wv[e / 2] >> (16 * (e % 2)));
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      Frag8<bf16_t> fb;
      fb.v = *reinterpret_cast<const uint4*>(&vt[(ct * 16 + lr) * kTPitch + kq]);
      acc[ct] = mma_k32(fx, fb, acc[ct]);
    }
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int j = j0 + ct * 16 + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + w * 16 + (l >> 4) * 4 + e;
      if (m < M && j < R) t[size_t(m) * R + j] = bf16_t{f32_to_bf16(acc[ct][e])};
    }
  }
}

// ---------------------------------------------------------------------------
// Main GEMM.  Workgroup tile 128 tokens x 128 outputs x 64 in_dim per stage;
// four waves in a 2 x 2 arrangement, each owning 64 x 64 (4 x 4 tiles).
// ---------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, BK = 64, PITCH = BK + 8;  // 144-byte LDS rows

struct GemmArgs {
  const bf16_t* x;
  const bf16_t* s;
  const bf16_t* w0;
  const bf16_t* u;
  const bf16_t* t;
  bf16_t* y;
  int M, O, I, R;
  int tiles_m, tiles_n;
};

__device__ __forceinline__ void gemm_load_stage(const GemmArgs& a, int m0, int n0, int k0, Frag8<bf16_t> (&ra)[4],
                                                Frag8<bf16_t> (&rb)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = tid + kThreads * q;
    const int row = c / 8, kc = k0 + (c % 8) * 8;
    const int am = m0 + row, bn = n0 + row;
    ra[q] = load_frag_if<bf16_t>(a.x + size_t(am) * a.I + kc, am < a.M && kc < a.I);
    rb[q] = load_frag_if<bf16_t>(a.w0 + size_t(bn) * a.I + kc, bn < a.O && kc < a.I);
  }
}

__device__ __forceinline__ void gemm_store_stage(uint16_t* as, uint16_t* bs, const Frag8<bf16_t> (&ra)[4],
                                                 const Frag8<bf16_t> (&rb)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = tid + kThreads * q;
    const int row = c / 8, kc = (c % 8) * 8;
    *reinterpret_cast<uint4*>(&as[row * PITCH + kc]) = ra[q].v;
    *reinterpret_cast<uint4*>(&bs[row * PITCH + kc]) = rb[q].v;
  }
}

__global__ __launch_bounds__(kThreads) void forward_gemm_kernel(GemmArgs a) {
  __shared__ uint16_t lds[2][2][BM * PITCH];  // [buffer][A or B][tile]
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int lr = l & 15, kq = (l >> 4) * 8;
  const int wm = w / 2, wn = w % 2;

  // Tiles are walked in column-major groups of 8 token tiles so that the
  // workgroups running together share W0 and x tiles in L2.
  const int bid = blockIdx.x;
  const int group = 8;
  const int per_group = group * a.tiles_n;
  const int gid = bid / per_group, first_m = gid * group;
  const int gsize = min(a.tiles_m - first_m, group);
  const int tm = first_m + (bid % per_group) % gsize;
  const int tn = (bid % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  Frag8<bf16_t> ra[4], rb[4];
  gemm_load_stage(a, m0, n0, 0, ra, rb);
  gemm_store_stage(lds[0][0], lds[0][1], ra, rb);
  __syncthreads();
  const int KT = (a.I + BK - 1) / BK;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gemm_load_stage(a, m0, n0, (kt + 1) * BK, ra, rb);
    const uint16_t* as = lds[cur][0];
    const uint16_t* bs = lds[cur][1];
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      Frag8<bf16_t> fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i].v = *reinterpret_cast<const uint4*>(&as[(wm * 64 + i * 16 + lr) * PITCH + kk + kq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j].v = *reinterpret_cast<const uint4*>(&bs[(wn * 64 + j * 16 + lr) * PITCH + kk + kq]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma_k32(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < KT) gemm_store_stage(lds[cur ^ 1][0], lds[cur ^ 1][1], ra, rb);
    __syncthreads();
  }

  // Epilogue: scale output column o by s[o], add T . U^T, round once.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int o = n0 + wn * 64 + j * 16 + lr;
    const float sc = o < a.O ? bf16_to_f32(a.s[o].bits) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][j] *= sc;
  }
  if (a.R > 0) {
    const bool aligned = (a.R % 8) == 0;
    for (int kk = 0; kk < a.R; kk += 32) {
      const int jr = kk + kq;
      Frag8<bf16_t> fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 64 + i * 16 + lr;
        fa[i] = zero_frag<bf16_t>();
        if (m < a.M && jr < a.R)
          fa[i] = aligned ? load_frag<bf16_t>(a.t + size_t(m) * a.R + jr) : load_frag_partial<bf16_t>(a.t + size_t(m) * a.R + jr, min(8, a.R - jr));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int o = n0 + wn * 64 + j * 16 + lr;
        fb[j] = zero_frag<bf16_t>();
        if (o < a.O && jr < a.R)
          fb[j] = aligned ? load_frag<bf16_t>(a.u + size_t(o) * a.R + jr) : load_frag_partial<bf16_t>(a.u + size_t(o) * a.R + jr, min(8, a.R - jr));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma_k32(fa[i], fb[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int o = n0 + wn * 64 + j * 16 + lr;
      if (o >= a.O) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 64 + i * 16 + (l >> 4) * 4 + e;
        if (m < a.M) a.y[size_t(m) * a.O + o] = bf16_t{f32_to_bf16(acc[i][j][e])};
      }
    }
  }
}

}  // namespace

GemmPlan plan_gemm(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank) {
  (void)out_dim;
  (void)in_dim;
  GemmPlan p{};
  p.off_t = kControlBytes;
  p.bytes = align_up(p.off_t + size_t(m) * size_t(rank) * 2, 256);
  return p;
}

hipError_t launch_forward_gemm(const GemmPlan& p, const void* x, const void* s, const void* w0, const void* u,
                               const void* v, void* y, int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank,
                               void* workspace, hipStream_t stream) {
  bf16_t* t = reinterpret_cast<bf16_t*>(static_cast<char*>(workspace) + p.off_t);
  if (rank > 0) {
    dim3 grid(unsigned((m + kTM - 1) / kTM), unsigned((rank + kTN - 1) / kTN));
    hipLaunchKernelGGL(xv_gemm_kernel, grid, dim3(kThreads), 0, stream, static_cast<const bf16_t*>(x),
                       static_cast<const bf16_t*>(v), t, int(m), int(in_dim), int(rank));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  GemmArgs a;
  a.x = static_cast<const bf16_t*>(x);
  a.s = static_cast<const bf16_t*>(s);
  a.w0 = static_cast<const bf16_t*>(w0);
  a.u = static_cast<const bf16_t*>(u);
  a.t = t;
  a.y = static_cast<bf16_t*>(y);
  a.M = int(m); a.O = int(out_dim); a.I = int(in_dim); a.R = int(rank);
  a.tiles_m = int((m + BM - 1) / BM);
  a.tiles_n = int((out_dim + BN - 1) / BN);
  hipLaunchKernelGGL(forward_gemm_kernel, dim3(unsigned(a.tiles_m * a.tiles_n)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tb
