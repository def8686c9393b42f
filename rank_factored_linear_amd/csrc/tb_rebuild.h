// Tiles of U . V^T on the matrix cores, shared by the kernels that rebuild
// W = diag(s) . W0 + U . V^T (reconstruct) and those that compare the rebuilt
// W with an original without writing it (reconstruction error).
// U [O, R] and V [I, R] are both contiguous along the rank R.
#pragma once

#include "tb_device.h"

namespace tb {
namespace rebuild {

constexpr int kThreads = 256;

// ---- 128 x 128 tiles, bf16, R % 8 == 0 ------------------------------------
// Four waves of 64 x 64; k-tiles of 64 staged in LDS (16-byte chunks XOR-
// swizzled by row) from registers.  The product is taken as V . U^T, so
// acc[rb][cb] element 4 b + e is C[i][o] for
//   i = i0 + 64 (w % 2) + 32 rb + 8 b + 4 (lane / 32) + e,
//   o = o0 + 64 (w / 2) + 32 cb + lane % 32:
// each lane holds four consecutive columns of one output row.
namespace t128 {

constexpr int BT = 128;
constexpr int BK = 64;
constexpr int kRowBytes = BK * 2;
constexpr int kTileBytes = BT * kRowBytes;
constexpr int kLdsBytes = 2 * kTileBytes;   // [U tile][V tile]

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                 0);
}

// Byte offset of chunk c of row r inside a tile: the chunk index is XORed
// with r % 8, so eight consecutive rows read at one chunk hit all 32 banks.
__device__ __forceinline__ int chunk_off(int r, int c) { return r * kRowBytes + ((c ^ (r & 7)) << 4); }

// acc = (V . U^T) of the tile at (o0, i0).  Uses lds[kLdsBytes]; begins with
// a barrier, so it may follow another tile's use of the same LDS.
__device__ __forceinline__ void product(const bf16_t* __restrict__ u, const bf16_t* __restrict__ v, int O, int I,
                                        int R, int o0, int i0, unsigned char* lds, f32x16 (&acc)[2][2]) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wi = w & 1, wo = w >> 1, h = l >> 5, lr = l & 31;
  // Staging: thread t moves chunk t % 8 of rows t / 8 + 32 q (q = 0..3) of both tiles.
  const int sc = tid & 7, sr = tid >> 3;
  uint4 su[4], sv[4];
  auto fetch = [&](int kt) {
    const int k = kt * BK + sc * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ro = o0 + sr + 32 * q, ri = i0 + sr + 32 * q;
      su[q] = (ro < O && k < R) ? *reinterpret_cast<const uint4*>(u + size_t(ro) * R + k) : make_uint4(0, 0, 0, 0);
      sv[q] = (ri < I && k < R) ? *reinterpret_cast<const uint4*>(v + size_t(ri) * R + k) : make_uint4(0, 0, 0, 0);
    }
  };
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  const int KT = (R + BK - 1) / BK;
  fetch(0);
  for (int kt = 0; kt < KT; ++kt) {
    __syncthreads();  // every wave has read the previous k-tile (or the previous user's data)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int off = chunk_off(sr + 32 * q, sc);
      *reinterpret_cast<uint4*>(lds + off) = su[q];
      *reinterpret_cast<uint4*>(lds + kTileBytes + off) = sv[q];
    }
    __syncthreads();
    if (kt + 1 < KT) fetch(kt + 1);  // lands while this k-tile multiplies
    uint4 fa[2][4], fb[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int ri = wi * 64 + rb * 32 + lr, ro = wo * 64 + rb * 32 + lr;
        fa[rb][ks] = *reinterpret_cast<const uint4*>(lds + kTileBytes + chunk_off(ri, ks * 2 + h));
        fb[rb][ks] = *reinterpret_cast<const uint4*>(lds + chunk_off(ro, ks * 2 + h));
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mma32(fa[rb][ks], fb[cb][ks], acc[rb][cb]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_operand_guard();
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace t128

// ---- 64 x 64 tiles, any element type and rank -----------------------------
// Wave w owns output rows o0 + 16 w .. +15; fragments come straight from
// global memory.  acc[ct] element e is C[o][i] for o = o0 + 16 w + 4 (lane / 16) + e,
// i = i0 + 16 ct + lane % 16.
namespace t64 {

constexpr int BT = 64;

template <typename EI>
__device__ __forceinline__ void product(const EI* __restrict__ u, const EI* __restrict__ v, int O, int I, int R,
                                        int o0, int i0, f32x4 (&acc)[4]) {
  const int l = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int lr = l & 15, kq = (l >> 4) * 8;
  const bool aligned = (R % 8) == 0;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int urow = o0 + w * 16 + lr;
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
}

}  // namespace t64
}  // namespace rebuild
}  // namespace tb
