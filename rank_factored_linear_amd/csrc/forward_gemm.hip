// Theta-bundle projection for many tokens (bf16, m > 64): two launches.
//
//   1. T = x . V                    [m, r], rounded to bf16 into the workspace
//   2. y = s (.) (x . W0^T) + T . U^T
//
// ("The theta bundle": the transpose of weight = diag(s) W0 + U V^T applied
// to x.)  Step 2 is a matrix-core GEMM whose operands are both contiguous
// along the reduction dimension (x rows over in_dim, W0 rows over in_dim).
// The scale by s is applied in fp32 to the finished sums of x . W0^T, and the
// same accumulators then continue over the rank dimension with T and U (both
// contiguous along r), so the rank-r delta costs r/in_dim extra reduction
// steps and no extra pass over y.  Rows that are 16-byte aligned (in_dim and
// rank multiples of 8) take the 256 x 256 stream-K kernel; other shapes take
// a general 128 x 128 kernel.
#include "tb_device.h"
#include "tb_host.h"

#include <algorithm>

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
// General GEMM (any in_dim and rank).  Workgroup tile 128 tokens x 128
// outputs x 64 in_dim per stage; four waves in a 2 x 2 arrangement, each
// owning 64 x 64 (4 x 4 tiles).
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

  // Epilogue: scale output column o by s[o] (no s: unit scale), add T . U^T, round once.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int o = n0 + wn * 64 + j * 16 + lr;
    const float sc = o < a.O ? (a.s ? bf16_to_f32(a.s[o].bits) : 1.f) : 0.f;
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

// ---------------------------------------------------------------------------
// Shared by the two matrix-core kernels below.
// ---------------------------------------------------------------------------
constexpr int kCounterBase = 64;              // control words from here count arrivals
constexpr unsigned kRsrcFlags = 0x00020000u;  // buffer descriptor word 3: 32-bit data format
constexpr int kCoherent = 16;                 // sc1: device-scope access, coherent across XCDs

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_byte;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Lane addresses in an LDS ring are passed through an empty asm statement so
// the compiler keeps each as one register and folds every per-step,
// per-buffer displacement (all below 64 KB) into the instruction's immediate
// offset instead of materialising one register per displacement.
__device__ __forceinline__ lds_byte* opaque(lds_byte* p) {
  asm volatile("" : "+v"(p));
  return p;
}

// ---------------------------------------------------------------------------
// Main GEMM for 16-byte aligned rows (in_dim and rank multiples of 8).
//
// Output tiles of 256 tokens x 256 outputs; eight waves, each owning 128 x 64
// as 4 x 2 accumulator tiles of v_mfma_f32_32x32x16_bf16.  The reduction runs
// in k-tiles of 64 through a two-buffer LDS ring filled by direct-to-LDS
// buffer loads (no staging through registers, no LDS store instructions: the
// LDS instruction queue carries only the fragment reads); rows past the
// matrix and chunks past the reduction length read as zero.
//
// The rank tail runs through the same pipeline: after the last k-tile of
// x . W0^T the accumulators are scaled by s and the reduction continues over
// the rank dimension with T = x . V (from the workspace) and U, both
// contiguous along r.
//
// Workgroups are persistent, one per compute unit, and take whole tiles in
// rounds.  When the tile count leaves a last, partly filled round, those
// remainder tiles are each split into S equal k-slices and the slices are
// handed out slice-major, so the workgroups running together hold the same
// k-range of neighbouring tiles and share their x and W0 k-tiles in L2.  A
// slice stores its fp32 partial; the last of a tile's slices to arrive sums
// all S partials in slice order (so the result does not depend on arrival
// order) and finishes the tile.
// ---------------------------------------------------------------------------
namespace big {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kWaves = 8, kThreads = kWaves * kWave;
constexpr int WN = kWaves / 2;            // waves along the output columns (two along the tokens)
constexpr int TJ = BN / WN / 32;          // 32-column accumulator tiles per wave
constexpr int kTileBytes = BM * BK * 2;   // one operand's k-tile in LDS: 256 rows of 128 bytes
// LDS ring [A0][A1][B0][B1]: buffer 1 sits 32 KB after buffer 0, within the
// immediate offset of every lane address.
constexpr int kBOffset = 2 * kTileBytes;
constexpr int kRingBytes = 4 * kTileBytes;
constexpr int kPartFloats = BM * BN;      // fp32 partial of one output tile
constexpr unsigned kOutOfRange = 0x80000000u;  // lane offset past every buffer: the load returns zeros

struct Args {
  const bf16_t* x;
  const bf16_t* s;
  const bf16_t* w0;
  const bf16_t* u;
  const bf16_t* t;
  bf16_t* y;
  int M, O, I, R;
  int tiles_m, tiles_n;
  int KT, KR;        // k-tiles of in_dim and of rank
  int split_tiles;   // tiles [0, split_tiles) are split into S k-slices ...
  int S, kps;        // ... of kps k-tiles each (the last may be shorter)
  int xcd_major;     // 1: workgroup g takes position (g % 8) * (grid / 8) + g / 8
  unsigned* ctrl;
  float* part;       // [S * split_tiles][kPartFloats] partials, slice-major
};

// A k-tile of each operand goes from HBM straight into LDS: each wave issues
// four 1 KB direct-to-LDS loads per operand (rows (4w + j) * 8 .. +7), lane l
// of a load landing at M0 + 16 l.  Within a row the 16-byte chunks are stored
// XOR-swizzled by (row >> 1) & 7, so the fragment reads of 16 consecutive
// rows hit distinct banks; the swizzle is applied by choosing which global
// chunk each lane fetches.  The loads are written as inline assembly: the
// compiler does not see them write LDS, so it does not drain every load
// before each LDS read, and the waits are explicit (vmcnt before the
// barrier that publishes a k-tile).
struct Operands {
  __amdgpu_buffer_rsrc_t ra, rb;
  int ve, vo;      // lane offsets (row, swizzled chunk) for the even and odd loads j
  int ce, co;      // the global chunk index each of them fetches
  int rowstep8;    // bytes of 8 rows (soffset step between the loads j)
  int kel;         // reduction length in elements
};

__device__ __forceinline__ Operands make_operands(const bf16_t* a, int arows, const bf16_t* b, int brows, int m0,
                                                  int n0, int k) {
  Operands o;
  const int ar = min(arows - m0, BM), br = min(brows - n0, BN);
  o.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a + size_t(m0) * k), 0, ar * k * 2, kRsrcFlags);
  o.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(b + size_t(n0) * k), 0, br * k * 2, kRsrcFlags);
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave), l = int(threadIdx.x) % kWave;
  // Load j covers rows w*32 + 8j + l/8; rows of even and of odd j share the swizzle.
  const int row_e = w * 32 + (l >> 3), row_o = row_e + 8, pos = l & 7;
  o.ce = pos ^ ((row_e >> 1) & 7);
  o.co = pos ^ ((row_o >> 1) & 7);
  o.ve = row_e * k * 2 + (o.ce << 4);
  o.vo = row_e * k * 2 + (o.co << 4);  // the soffset of load j adds its 8j rows
  o.rowstep8 = 8 * k * 2;
  o.kel = k;
  return o;
}

// Lane addresses in the LDS ring, built once per workgroup.
struct Lanes {
  unsigned dma_a, dma_b;  // this wave's first 1 KB of A and of B in buffer 0 (uniform)
  lds_byte* a_rd[4];      // A fragment of k16 step st: row wm*128 + lane%32, swizzled chunk 2st + lane/32
  lds_byte* b_rd[4];      // B fragment of k16 step st: row wn*(BN/WN) + lane%32
};

__device__ __forceinline__ Lanes make_lanes(uint8_t* ring) {
  lds_byte* base = (lds_byte*)ring;
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave), l = int(threadIdx.x) % kWave;
  const int lr = l & 31, hi = l >> 5, wm = w / WN, wn = w % WN, x = (lr >> 1) & 7;
  Lanes ln;
  const unsigned b0 = unsigned(uintptr_t(base));
  ln.dma_a = __builtin_amdgcn_readfirstlane(b0 + unsigned(w) * 4096u);
  ln.dma_b = __builtin_amdgcn_readfirstlane(b0 + unsigned(kBOffset) + unsigned(w) * 4096u);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int chunk = ((2 * st + hi) ^ x) << 4;
    ln.a_rd[st] = opaque(base + (wm * 128 + lr) * 128 + chunk);
    ln.b_rd[st] = opaque(base + kBOffset + (wn * (BN / WN) + lr) * 128 + chunk);
  }
  return ln;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Four direct-to-LDS loads of one operand: load j writes 1 KB at dst + j KB
// from the global rows at soffset soff + j * rowstep8.  M0 takes one wait
// state before a load that reads it.
__device__ __forceinline__ void dma4(unsigned dst, __amdgpu_buffer_rsrc_t r, int ve, int vo, int soff, int rowstep8) {
  asm volatile(
      "s_mov_b32 m0, %[d0]\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[ve], %[r], %[s0] offen lds\n\t"
      "s_mov_b32 m0, %[d1]\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[vo], %[r], %[s1] offen lds\n\t"
      "s_mov_b32 m0, %[d2]\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[ve], %[r], %[s2] offen lds\n\t"
      "s_mov_b32 m0, %[d3]\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[vo], %[r], %[s3] offen lds"
      :
      : [d0] "s"(dst), [d1] "s"(dst + 1024u), [d2] "s"(dst + 2048u), [d3] "s"(dst + 3072u), [ve] "v"(ve), [vo] "v"(vo),
        [r] "s"(r), [s0] "s"(soff), [s1] "s"(soff + rowstep8), [s2] "s"(soff + 2 * rowstep8),
        [s3] "s"(soff + 3 * rowstep8)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Every direct-to-LDS load of this wave has landed.
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// k-tile kt of both operands into LDS buffer BUF (eight loads per wave).  In
// a k-tile that runs past the reduction length, lanes whose chunk starts at or
// beyond it fetch from past the buffer and so write zeros.
template <int BUF>
__device__ __forceinline__ void issue(const Operands& o, const Lanes& ln, int kt) {
  int ve = o.ve, vo = o.vo;
  const int left = o.kel - kt * BK;
  if (left < BK) {
    ve = o.ce * 8 < left ? ve : int(kOutOfRange);
    vo = o.co * 8 < left ? vo : int(kOutOfRange);
  }
  dma4(ln.dma_a + BUF * kTileBytes, o.ra, ve, vo, kt * BK * 2, o.rowstep8);
  dma4(ln.dma_b + BUF * kTileBytes, o.rb, ve, vo, kt * BK * 2, o.rowstep8);
}

// Operand fragments of k16 step st from buffer BUF: A rows wm*128 + 32i +
// lane%32, B rows wn*(BN/WN) + 32j + lane%32, k = 16 st + 8 (lane / 32) + 0..7.
template <int BUF>
__device__ __forceinline__ void read_frags(const Lanes& ln, int st, u32x4 (&fa)[4], u32x4 (&fb)[TJ]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    fa[i] = *reinterpret_cast<const lds_u32x4*>(ln.a_rd[st] + BUF * kTileBytes + i * 32 * 128);
#pragma unroll
  for (int j = 0; j < TJ; ++j)
    fb[j] = *reinterpret_cast<const lds_u32x4*>(ln.b_rd[st] + BUF * kTileBytes + j * 32 * 128);
}

__device__ __forceinline__ void mma_step(const u32x4 (&fa)[4], const u32x4 (&fb)[TJ], f32x16 (&acc)[4][TJ]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[i]),
                                                          __builtin_bit_cast(bf16x8, fb[j]), acc[i][j], 0, 0, 0);
}

// One k-tile in software-pipelined form.  On entry tile k sits in LDS buffer
// BUF and its k16 steps 0 and 1 are in (fa0, fb0) and (fa1, fb1); the loads
// of tile k+1 into the other buffer are in flight.  Steps 2 and 3 are read
// while steps 0 and 1 multiply; the barrier falls between steps 2 and 3, once
// tile k+1 has landed; then tile k2 is issued into BUF (free: every wave has
// read its steps) while step 3's products cover the first reads of tile k+1.
// On exit the invariant holds for tile k+1.
template <int BUF>
__device__ __forceinline__ void k_step(const Operands& o, const Lanes& ln, int k2, u32x4 (&fa0)[4], u32x4 (&fb0)[TJ],
                                       u32x4 (&fa1)[4], u32x4 (&fb1)[TJ], f32x16 (&acc)[4][TJ]) {
  mma_step(fa0, fb0, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<BUF>(ln, 2, fa0, fb0);
  __builtin_amdgcn_sched_barrier(0);
  mma_step(fa1, fb1, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<BUF>(ln, 3, fa1, fb1);
  __builtin_amdgcn_sched_barrier(0);
  mma_step(fa0, fb0, acc);
  __builtin_amdgcn_sched_barrier(0);
  wait_dma();
  __syncthreads();
  read_frags<1 - BUF>(ln, 0, fa0, fb0);
  __builtin_amdgcn_sched_barrier(0);
  issue<BUF>(o, ln, k2);
  __builtin_amdgcn_sched_barrier(0);
  mma_step(fa1, fb1, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<1 - BUF>(ln, 1, fa1, fb1);
}

// acc += A[rows, kb*64 : ke*64] . B[rows, same]^T.  Leaves the LDS ring free
// and no load in flight.
__device__ __forceinline__ void k_loop(const Operands& o, int kb, int ke, f32x16 (&acc)[4][TJ], const Lanes& ln) {
  const int n = ke - kb;
  u32x4 fa0[4], fb0[TJ], fa1[4], fb1[TJ];
  issue<0>(o, ln, kb);
  issue<1>(o, ln, min(kb + 1, ke - 1));
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // tile kb has landed (the next tile's eight loads may not)
  __syncthreads();
  read_frags<0>(ln, 0, fa0, fb0);
  read_frags<0>(ln, 1, fa1, fb1);
  for (int k = 0; k < n; k += 2) {
    // Tiles past the end are loaded again as the last tile (clamped) and
    // never multiplied.
    k_step<0>(o, ln, min(kb + k + 2, ke - 1), fa0, fb0, fa1, fb1, acc);
    if (k + 1 < n) k_step<1>(o, ln, min(kb + k + 3, ke - 1), fa0, fb0, fa1, fb1, acc);
  }
  wait_dma();
  __syncthreads();
}

// Tile u of the processing order -> (token tile, output tile): groups of
// eight token tiles are walked column by column, so workgroups that run
// together share x and W0 rows in L2.
__device__ __forceinline__ void tile_coords(const Args& a, int u, int& tm, int& tn) {
  const int per_group = 8 * a.tiles_n;
  const int first = (u / per_group) * 8, gsize = min(a.tiles_m - first, 8), r = u % per_group;
  tm = first + r % gsize;
  tn = r / gsize;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const Args& a, int slot) {
  return __builtin_amdgcn_make_buffer_rsrc(a.part + size_t(slot) * kPartFloats, 0, kPartFloats * 4, kRsrcFlags);
}

// Partials are laid out as the accumulators sit in registers: 16-byte piece
// q = (TJ i + j) * 4 + c of every lane, lanes contiguous.
__device__ __forceinline__ void store_partial(const Args& a, int slot, const f32x16 (&acc)[4][TJ]) {
  const __amdgpu_buffer_rsrc_t rs = part_rsrc(a, slot);
  const int lane_off = int(threadIdx.x) * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 v = {__float_as_uint(acc[i][j][4 * c]), __float_as_uint(acc[i][j][4 * c + 1]),
                         __float_as_uint(acc[i][j][4 * c + 2]), __float_as_uint(acc[i][j][4 * c + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, lane_off, ((i * TJ + j) * 4 + c) * kThreads * 16, kCoherent);
      }
}

// acc = partial (first) or acc += partial.
__device__ __forceinline__ void add_partial(const Args& a, int slot, bool first, f32x16 (&acc)[4][TJ]) {
  const __amdgpu_buffer_rsrc_t rs = part_rsrc(a, slot);
  const int lane_off = int(threadIdx.x) * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off, ((i * TJ + j) * 4 + c) * kThreads * 16,
                                                              kCoherent);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[i][j][4 * c + e] = first ? __uint_as_float(v[e]) : acc[i][j][4 * c + e] + __uint_as_float(v[e]);
      }
}

// Scale by s, add T . U^T, round to bf16 and store.
__device__ __forceinline__ void finish_tile(const Args& a, int m0, int n0, f32x16 (&acc)[4][TJ], const Lanes& ln) {
  const int w = int(threadIdx.x) / kWave, l = int(threadIdx.x) % kWave, lr = l & 31, hi = l >> 5;
  const int wm = w / WN, wn = w % WN;
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int n = n0 + wn * (BN / WN) + j * 32 + lr;
    const float sc = n < a.O ? (a.s ? bf16_to_f32(a.s[n].bits) : 1.f) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][j] *= sc;
  }
  if (a.R > 0) {
    const Operands r = make_operands(a.t, a.M, a.u, a.O, m0, n0, a.R);
    k_loop(r, 0, a.KR, acc, ln);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int n = n0 + wn * (BN / WN) + j * 32 + lr;
      if (n >= a.O) continue;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + wm * 128 + i * 32 + 8 * b + 4 * hi + e;
          if (m < a.M) a.y[size_t(m) * a.O + n] = bf16_t{f32_to_bf16(acc[i][j][4 * b + e])};
        }
    }
}

// k-tiles [kb, ke) of tile u; finishes the tile if it holds the whole
// reduction or arrives last among the tile's workgroups.
// k-tiles [kb, ke) of tile u: the whole reduction (slice < 0) or k-slice
// `slice`; finishes the tile if it holds the whole reduction or is the last
// of the tile's slices to arrive.
__device__ __forceinline__ void do_tile(const Args& a, int u, int kb, int ke, int slice, const Lanes& ln,
                                        unsigned* s_last) {
  int tm, tn;
  tile_coords(a, u, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  f32x16 acc[4][TJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};
  k_loop(make_operands(a.x, a.M, a.w0, a.O, m0, n0, a.I), kb, ke, acc, ln);
  if (slice >= 0) {
    store_partial(a, slice * a.split_tiles + u, acc);
    __builtin_amdgcn_s_waitcnt(0);  // partial written through before counting in
    __syncthreads();
    if (threadIdx.x == 0)
      *s_last = __hip_atomic_fetch_add(&a.ctrl[kCounterBase + u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                unsigned(a.S - 1);
    __syncthreads();
    if (!*s_last) return;
    for (int q = 0; q < a.S; ++q) add_partial(a, q * a.split_tiles + u, q == 0, acc);
    if (threadIdx.x == 0)
      __hip_atomic_store(&a.ctrl[kCounterBase + u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  finish_tile(a, m0, n0, acc, ln);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4))) void gemm_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRingBytes];
  __shared__ unsigned s_last;
  const int g = int(blockIdx.x), G = int(gridDim.x);
  const int pos = a.xcd_major ? (g % 8) * (G / 8) + g / 8 : g;
  const Lanes ln = make_lanes(ring);
  for (int v = pos; v < a.split_tiles * a.S; v += G) {
    const int u = v % a.split_tiles, slice = v / a.split_tiles;
    do_tile(a, u, slice * a.kps, min(a.KT, (slice + 1) * a.kps), slice, ln, &s_last);
  }
  const int tiles = a.tiles_m * a.tiles_n;
  for (int u = a.split_tiles + pos; u < tiles; u += G) do_tile(a, u, 0, a.KT, -1, ln, &s_last);
}

}  // namespace big

// ---------------------------------------------------------------------------
// T = x . V for many tokens.  V is [in_dim, r] with r contiguous, so its
// k-tiles are staged in LDS as they sit in memory (rows of k) and the matrix
// core's B fragments (eight consecutive k of one column per lane) are read
// with the transposing LDS read: within each group of 16 lanes, lane i
// receives element i % 4 of the 8-byte chunks addressed by lanes 4e + i / 4
// (e = 0..3), so lanes that point at rows kb + j / 4, columns nb + 4 (j % 4)
// each receive four consecutive k of column nb + i.
//
// Workgroup tile: 64 tokens x 256 columns of T, four waves of 64 x 64 (2 x 2
// tiles of v_mfma_f32_32x32x16_bf16), k-tiles of 64 double-buffered in LDS
// from two register sets of buffer loads.  The reduction over in_dim is split
// into KS slices so the grid fills the chip; with KS > 1 each slice stores its
// fp32 partial and the last of a tile's slices to arrive sums them in slice
// order and stores T rounded to bf16.
// ---------------------------------------------------------------------------
namespace xv {

constexpr int BM = 64, BN = 256, BK = 64, kThreads = 256;
constexpr int kXPitch = BK * 2 + 16;   // 144-byte rows of the x tile
constexpr int kVPitch = BN * 2 + 64;   // 576-byte rows of the V tile: 16 banks of skew per row
constexpr int kXTile = BM * kXPitch;   // 9 KB
constexpr int kVTile = BK * kVPitch;   // 36 KB
constexpr int kRingBytes = 2 * kVTile + 2 * kXTile;  // [V0][V1][X0][X1]
constexpr int kPartFloats = BM * BN;
// x tiles are read by one column block of T only (rank <= 256), while every
// row block re-reads the V tiles: x is loaded non-temporal (the NT bit of the
// buffer load's cache policy) so that it does not push V out of L2.
constexpr int kXPolicy = 2;

struct Args {
  const bf16_t* x;
  const bf16_t* v;
  bf16_t* t;
  int M, I, R;
  int RB, CB, KT;  // row blocks, column blocks, k-tiles of in_dim
  int KS, kps;     // k-slices and k-tiles per slice
  unsigned* ctrl;
  float* part;     // [RB * CB][KS][kPartFloats]
};

struct Lanes {
  lds_byte* x_rd;   // A fragment: row lane%32, k half lane/32
  lds_byte* v_rd0;  // transposing B reads, buffer 0 / 1
  lds_byte* v_rd1;
  lds_byte* x_wr;   // x staging: row tid/8, chunk tid%8
  lds_byte* v_wr0;  // V staging: k-row tid/32, chunk tid%32, buffer 0 / 1
  lds_byte* v_wr1;
};

__device__ __forceinline__ Lanes make_lanes(uint8_t* ring) {
  lds_byte* base = (lds_byte*)ring;
  const int tid = int(threadIdx.x), w = tid / kWave, l = tid % kWave, lr = l & 31, hi = l >> 5;
  const int g = l >> 4, j16 = l & 15;
  const int vrow = 8 * (g >> 1) + (j16 >> 2), vcol = 64 * w + 16 * (g & 1) + 4 * (j16 & 3);
  Lanes ln;
  ln.x_rd = opaque(base + 2 * kVTile + lr * kXPitch + hi * 16);
  ln.v_rd0 = opaque(base + vrow * kVPitch + vcol * 2);
  ln.v_rd1 = opaque(base + kVTile + vrow * kVPitch + vcol * 2);
  ln.x_wr = opaque(base + 2 * kVTile + (tid >> 3) * kXPitch + (tid & 7) * 16);
  ln.v_wr0 = opaque(base + (tid >> 5) * kVPitch + (tid & 31) * 16);
  ln.v_wr1 = opaque(base + kVTile + (tid >> 5) * kVPitch + (tid & 31) * 16);
  return ln;
}

struct Src {
  __amdgpu_buffer_rsrc_t rx, rv;
  int xoff, voff;     // lane byte offsets: x row tid/8 chunk tid%8; V k-row tid/32 chunk tid%32
  int xstep, vstep;   // bytes of 32 x rows / 8 V rows
  int I, ncols;       // reduction length; valid columns of this column block
};

__device__ __forceinline__ void fetch(const Src& s, int kt, u32x4 (&px)[2], u32x4 (&pv)[8]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) px[q] = __builtin_amdgcn_raw_buffer_load_b128(s.rx, s.xoff, kt * BK * 2 + q * s.xstep, kXPolicy);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    pv[q] = __builtin_amdgcn_raw_buffer_load_b128(s.rv, s.voff, kt * 8 * s.vstep + q * s.vstep, 0);
}

template <int BUF>
__device__ __forceinline__ void stage(const Lanes& ln, const Src& s, int kt, u32x4 (&px)[2], u32x4 (&pv)[8]) {
  // x chunks at or past in_dim would read the next row: zero them.  V rows
  // past in_dim read as zero from the buffer bound; V columns past r of this
  // block would read the next row: zero them.
  if (s.I - kt * BK < BK) {
    const bool keep = int(threadIdx.x & 7) * 8 < s.I - kt * BK;
#pragma unroll
    for (int q = 0; q < 2; ++q) px[q] = keep ? px[q] : u32x4{0u, 0u, 0u, 0u};
  }
  if (s.ncols < BN) {
    const bool keep = int(threadIdx.x & 31) * 8 < s.ncols;
#pragma unroll
    for (int q = 0; q < 8; ++q) pv[q] = keep ? pv[q] : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) *reinterpret_cast<lds_u32x4*>(ln.x_wr + BUF * kXTile + q * 32 * kXPitch) = px[q];
#pragma unroll
  for (int q = 0; q < 8; ++q) *reinterpret_cast<lds_u32x4*>((BUF ? ln.v_wr1 : ln.v_wr0) + q * 8 * kVPitch) = pv[q];
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int BUF>
__device__ __forceinline__ void read_frags(const Lanes& ln, int st, u32x4 (&fa)[2], u32x4 (&fb)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
    fa[i] = *reinterpret_cast<const lds_u32x4*>(ln.x_rd + BUF * kXTile + i * 32 * kXPitch + st * 32);
  lds_byte* vr = BUF ? ln.v_rd1 : ln.v_rd0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vr + (16 * st) * kVPitch + 64 * j));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vr + (16 * st + 4) * kVPitch + 64 * j));
    fb[j] = u32x4{uint32_t(uint16_t(lo[0])) | (uint32_t(uint16_t(lo[1])) << 16),
                  uint32_t(uint16_t(lo[2])) | (uint32_t(uint16_t(lo[3])) << 16),
                  uint32_t(uint16_t(hi[0])) | (uint32_t(uint16_t(hi[1])) << 16),
                  uint32_t(uint16_t(hi[2])) | (uint32_t(uint16_t(hi[3])) << 16)};
  }
}

__device__ __forceinline__ void mma_step(const u32x4 (&fa)[2], const u32x4 (&fb)[2], f32x16 (&acc)[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[i]),
                                                          __builtin_bit_cast(bf16x8, fb[j]), acc[i][j], 0, 0, 0);
}

template <int BUF>
__device__ __forceinline__ void multiply_tile(const Lanes& ln, f32x16 (&acc)[2][2]) {
  u32x4 fa0[2], fb0[2], fa1[2], fb1[2];
  read_frags<BUF>(ln, 0, fa0, fb0);
  read_frags<BUF>(ln, 1, fa1, fb1);
  __builtin_amdgcn_sched_barrier(0);
  mma_step(fa0, fb0, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<BUF>(ln, 2, fa0, fb0);
  __builtin_amdgcn_sched_barrier(0);
  mma_step(fa1, fb1, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<BUF>(ln, 3, fa1, fb1);
  __builtin_amdgcn_sched_barrier(0);
  mma_step(fa0, fb0, acc);
  __builtin_amdgcn_sched_barrier(0);
  mma_step(fa1, fb1, acc);
}

__global__ __launch_bounds__(kThreads) void xv_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRingBytes];
  __shared__ unsigned s_last;
  const int tid = int(threadIdx.x);
  const int b = int(blockIdx.x), ks = b % a.KS, tile = b / a.KS;
  const int rb = tile / a.CB, cb = tile % a.CB;
  const int m0 = rb * BM, n0 = cb * BN;
  const int kb = ks * a.kps, ke = min(a.KT, kb + a.kps);
  const Lanes ln = make_lanes(ring);
  Src s;
  s.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a.x + size_t(m0) * a.I), 0,
                                          min(a.M - m0, BM) * a.I * 2, kRsrcFlags);
  s.rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a.v + n0), 0, (a.I * a.R - n0) * 2, kRsrcFlags);
  s.xoff = (tid >> 3) * a.I * 2 + (tid & 7) * 16;
  s.voff = (tid >> 5) * a.R * 2 + (tid & 31) * 16;
  s.xstep = 32 * a.I * 2;
  s.vstep = 8 * a.R * 2;
  s.I = a.I;
  s.ncols = min(BN, a.R - n0);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  if (kb < ke) {
    const int n = ke - kb;
    u32x4 px0[2], pv0[8], px1[2], pv1[8];
    fetch(s, kb, px0, pv0);
    fetch(s, min(kb + 1, ke - 1), px1, pv1);
    stage<0>(ln, s, kb, px0, pv0);
    __syncthreads();
    for (int k = 0; k < n; k += 2) {
      const int k1 = min(kb + k + 1, ke - 1), k2 = min(kb + k + 2, ke - 1), k3 = min(kb + k + 3, ke - 1);
      fetch(s, k2, px0, pv0);
      __builtin_amdgcn_sched_barrier(0);
      multiply_tile<0>(ln, acc);
      __builtin_amdgcn_sched_barrier(0);
      stage<1>(ln, s, k1, px1, pv1);
      __syncthreads();
      if (k + 1 < n) {
        fetch(s, k3, px1, pv1);
        __builtin_amdgcn_sched_barrier(0);
        multiply_tile<1>(ln, acc);
        __builtin_amdgcn_sched_barrier(0);
        stage<0>(ln, s, k2, px0, pv0);
        __syncthreads();
      }
    }
  }

  if (a.KS > 1) {
    // Partial in register order: 16-byte piece q = (2i + j) * 4 + c of every lane.
    float* blk = a.part + size_t(tile) * a.KS * kPartFloats;
    const __amdgpu_buffer_rsrc_t mine =
        __builtin_amdgcn_make_buffer_rsrc(blk + size_t(ks) * kPartFloats, 0, kPartFloats * 4, kRsrcFlags);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 val = {__float_as_uint(acc[i][j][4 * c]), __float_as_uint(acc[i][j][4 * c + 1]),
                             __float_as_uint(acc[i][j][4 * c + 2]), __float_as_uint(acc[i][j][4 * c + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(val, mine, tid * 16, ((i * 2 + j) * 4 + c) * kThreads * 16,
                                                 kCoherent);
        }
    __builtin_amdgcn_s_waitcnt(0);  // partial written through before counting in
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(&a.ctrl[kCounterBase + tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               unsigned(a.KS - 1);
    __syncthreads();
    if (!s_last) return;
    for (int q = 0; q < a.KS; ++q) {
      const __amdgpu_buffer_rsrc_t src =
          __builtin_amdgcn_make_buffer_rsrc(blk + size_t(q) * kPartFloats, 0, kPartFloats * 4, kRsrcFlags);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const u32x4 val = __builtin_amdgcn_raw_buffer_load_b128(
                src, tid * 16, ((i * 2 + j) * 4 + c) * kThreads * 16, kCoherent);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[i][j][4 * c + e] = q == 0 ? __uint_as_float(val[e]) : acc[i][j][4 * c + e] + __uint_as_float(val[e]);
          }
    }
    if (tid == 0) __hip_atomic_store(&a.ctrl[kCounterBase + tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int w = tid / kWave, l = tid % kWave, lr = l & 31, hi = l >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 64 * w + 32 * j + lr;
      if (n >= a.R) continue;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + 32 * i + 8 * bb + 4 * hi + e;
          if (m < a.M) a.t[size_t(m) * a.R + n] = bf16_t{f32_to_bf16(acc[i][j][4 * bb + e])};
        }
    }
}

}  // namespace xv

}  // namespace

namespace {

// Cost model of the split remainder round, in k-tiles of one workgroup:
// storing a 256 x 256 fp32 partial and reading one back each cost about as
// much as a few k-tiles of multiplication; slices shorter than kMinSlice
// k-tiles are not worth their partials.
constexpr int kStoreCost = 6, kLoadCost = 4, kMinSlice = 4;

}  // namespace

GemmPlan plan_gemm(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, int cus) {
  GemmPlan p{};
  p.off_t = 0;
  const size_t off = align_up(p.off_t + size_t(m) * size_t(rank) * 2, 256);
  p.bytes = off;
  // The matrix-core kernels for 16-byte aligned rows address one tile's rows
  // (and all of V) with 32-bit byte offsets.
  p.aligned = in_dim % 8 == 0 && rank % 8 == 0 && in_dim < (int64_t(1) << 22) && rank < (int64_t(1) << 22) &&
              in_dim * rank < (int64_t(1) << 30);
  p.big = p.aligned;
  if (!p.aligned) return p;
  // x . V: enough k-slices to give every compute unit a workgroup, each at
  // least two k-tiles long and at most 16 partials per tile.
  size_t o2 = off;
  if (rank > 0) {
    p.xv_rb = int((m + xv::BM - 1) / xv::BM);
    p.xv_cb = int((rank + xv::BN - 1) / xv::BN);
    p.xv_kt = int((in_dim + xv::BK - 1) / xv::BK);
    const int64_t tiles = int64_t(p.xv_rb) * p.xv_cb;
    int64_t ks = tiles >= cus ? 1 : cus / tiles;
    ks = std::min<int64_t>(ks, std::min<int64_t>(16, std::max<int64_t>(1, p.xv_kt / 2)));
    if (tiles > kMaxGroupCounters) ks = 1;
    p.xv_kps = int((p.xv_kt + ks - 1) / ks);
    p.xv_ks = int((p.xv_kt + p.xv_kps - 1) / p.xv_kps);
    p.off_xvpart = o2;
    if (p.xv_ks > 1) o2 = align_up(o2 + size_t(tiles) * p.xv_ks * xv::kPartFloats * 4, 256);
  }
  const size_t off_big = o2;
  p.bytes = o2;
  p.tiles_m = int((m + big::BM - 1) / big::BM);
  p.tiles_n = int((out_dim + big::BN - 1) / big::BN);
  p.KT = int((in_dim + big::BK - 1) / big::BK);
  p.KR = int((rank + big::BK - 1) / big::BK);
  const int64_t tiles = int64_t(p.tiles_m) * p.tiles_n, KT = p.KT;
  const int G = cus >= 8 ? cus / 8 * 8 : cus;
  const auto round8 = [&](int64_t g) { return int(cus >= 8 ? std::min<int64_t>(G, (g + 7) / 8 * 8) : std::min<int64_t>(G, g)); };

  // Whole tiles in ceil(tiles / G) rounds ...
  int64_t best = (tiles + G - 1) / G * KT;
  p.grid = round8(tiles);
  p.split_tiles = 0;
  p.S = 1;
  p.kps = p.KT;
  // ... or the whole rounds plus the remainder tiles split into S k-slices,
  // all slices in one extra round.
  const int64_t rounds = tiles / G, rem = tiles % G;
  for (int64_t S = 2; rem != 0 && S <= 16 && rem * S <= G; ++S) {
    const int64_t kps = (KT + S - 1) / S, slices = (KT + kps - 1) / kps;
    if (kps < kMinSlice) break;
    const int64_t cost = rounds * KT + kps + kStoreCost + kLoadCost * slices;
    if (cost < best && rem <= kMaxGroupCounters) {
      best = cost;
      p.split_tiles = int(rem);
      p.S = int(slices);
      p.kps = int(kps);
      p.grid = rounds > 0 ? G : round8(rem * slices);
    }
  }
  // Fewer workgroups than half the compute units even with the k-slices:
  // the 128 x 128 kernel's four times as many tiles finish sooner.
  if (p.grid < G / 2) {
    p.big = 0;
    p.split_tiles = 0;
  }
  p.xcd_major = p.grid % 8 == 0 ? 1 : 0;
  p.off_part = off_big;
  if (p.split_tiles > 0) p.bytes = off_big + size_t(p.split_tiles) * p.S * big::kPartFloats * 4;
  return p;
}

hipError_t launch_forward_gemm(const GemmPlan& p, const void* x, const void* s, const void* w0, const void* u,
                               const void* v, void* y, int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank,
                               unsigned* ctrl, char* data, hipStream_t stream) {
  char* ws = data;
  bf16_t* t = reinterpret_cast<bf16_t*>(ws + p.off_t);
  if (rank > 0 && p.aligned) {
    xv::Args a;
    a.x = static_cast<const bf16_t*>(x);
    a.v = static_cast<const bf16_t*>(v);
    a.t = t;
    a.M = int(m); a.I = int(in_dim); a.R = int(rank);
    a.RB = p.xv_rb; a.CB = p.xv_cb; a.KT = p.xv_kt;
    a.KS = p.xv_ks; a.kps = p.xv_kps;
    a.ctrl = ctrl;
    a.part = reinterpret_cast<float*>(ws + p.off_xvpart);
    hipLaunchKernelGGL(xv::xv_kernel, dim3(unsigned(p.xv_rb * p.xv_cb * p.xv_ks)), dim3(xv::kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (rank > 0) {
    dim3 grid(unsigned((m + kTM - 1) / kTM), unsigned((rank + kTN - 1) / kTN));
    hipLaunchKernelGGL(xv_gemm_kernel, grid, dim3(kThreads), 0, stream, static_cast<const bf16_t*>(x),
                       static_cast<const bf16_t*>(v), t, int(m), int(in_dim), int(rank));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.big) {
    big::Args a;
    a.x = static_cast<const bf16_t*>(x);
    a.s = static_cast<const bf16_t*>(s);
    a.w0 = static_cast<const bf16_t*>(w0);
    a.u = static_cast<const bf16_t*>(u);
    a.t = t;
    a.y = static_cast<bf16_t*>(y);
    a.M = int(m); a.O = int(out_dim); a.I = int(in_dim); a.R = int(rank);
    a.tiles_m = p.tiles_m; a.tiles_n = p.tiles_n;
    a.KT = p.KT; a.KR = p.KR;
    a.split_tiles = p.split_tiles; a.S = p.S; a.kps = p.kps; a.xcd_major = p.xcd_major;
    a.ctrl = ctrl;
    a.part = reinterpret_cast<float*>(ws + p.off_part);
    hipLaunchKernelGGL(big::gemm_kernel, dim3(unsigned(p.grid)), dim3(big::kThreads), 0, stream, a);
    return hipGetLastError();
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
