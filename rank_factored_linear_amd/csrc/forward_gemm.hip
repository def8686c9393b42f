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

// One projection of a launch (its output tiles are workgroups start[j] ..
// start[j+1] - 1 of the grid).
struct GemmMember {
  const bf16_t* x;
  const bf16_t* s;
  const bf16_t* w0;
  const bf16_t* u;
  const bf16_t* t;
  bf16_t* y;
  int O, tiles_n;
};

// The projections of one launch share the token count, in_dim and rank.
struct GemmArgs {
  int n;
  int start[kMaxProjections + 1];
  GemmMember mem[kMaxProjections];
  int M, I, R;
  int tiles_m;
  const unsigned* err;  // sticky error word: while set, y is written as NaN
};

// The workspace's sticky error word, read once at kernel entry (relaxed,
// device scope).  A set word means an earlier call on this workspace timed
// out and may have left stale counts behind.
__device__ __forceinline__ uint32_t load_error_word(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void gemm_load_stage(const GemmArgs& a, const GemmMember& mb, int m0, int n0, int k0,
                                                Frag8<bf16_t> (&ra)[4], Frag8<bf16_t> (&rb)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = tid + kThreads * q;
    const int row = c / 8, kc = k0 + (c % 8) * 8;
    const int am = m0 + row, bn = n0 + row;
    ra[q] = load_frag_if<bf16_t>(mb.x + size_t(am) * a.I + kc, am < a.M && kc < a.I);
    rb[q] = load_frag_if<bf16_t>(mb.w0 + size_t(bn) * a.I + kc, bn < mb.O && kc < a.I);
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

  // The workgroup's member; within it tiles are walked in column-major groups
  // of 8 token tiles so that the workgroups running together share W0 and x
  // tiles in L2.
  int mj = 0;
  while (mj + 1 < a.n && int(blockIdx.x) >= a.start[mj + 1]) ++mj;
  const GemmMember& mb = a.mem[mj];
  const int bid = int(blockIdx.x) - a.start[mj];
  const int group = 8;
  const int per_group = group * mb.tiles_n;
  const int gid = bid / per_group, first_m = gid * group;
  const int gsize = min(a.tiles_m - first_m, group);
  const int tm = first_m + (bid % per_group) % gsize;
  const int tn = (bid % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;
  const uint32_t err_at_entry = load_error_word(a.err);

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  Frag8<bf16_t> ra[4], rb[4];
  gemm_load_stage(a, mb, m0, n0, 0, ra, rb);
  gemm_store_stage(lds[0][0], lds[0][1], ra, rb);
  __syncthreads();
  const int KT = (a.I + BK - 1) / BK;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gemm_load_stage(a, mb, m0, n0, (kt + 1) * BK, ra, rb);
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
    const float sc = o < mb.O ? (mb.s ? bf16_to_f32(mb.s[o].bits) : 1.f) : 0.f;
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
          fa[i] = aligned ? load_frag<bf16_t>(mb.t + size_t(m) * a.R + jr) : load_frag_partial<bf16_t>(mb.t + size_t(m) * a.R + jr, min(8, a.R - jr));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int o = n0 + wn * 64 + j * 16 + lr;
        fb[j] = zero_frag<bf16_t>();
        if (o < mb.O && jr < a.R)
          fb[j] = aligned ? load_frag<bf16_t>(mb.u + size_t(o) * a.R + jr) : load_frag_partial<bf16_t>(mb.u + size_t(o) * a.R + jr, min(8, a.R - jr));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma_k32(fa[i], fb[j], acc[i][j]);
    }
  }
  const bool poisoned = err_at_entry != 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int o = n0 + wn * 64 + j * 16 + lr;
      if (o >= mb.O) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 64 + i * 16 + (l >> 4) * 4 + e;
        if (m < a.M) mb.y[size_t(m) * mb.O + o] = bf16_t{f32_to_bf16(poisoned ? __builtin_nanf("") : acc[i][j][e])};
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
typedef __attribute__((address_space(3))) uint16_t lds_u16;

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
// The finished tile leaves through LDS: each wave stages 16 of its 128 rows at
// a time (64 columns of bf16, rows 144 bytes apart so that the two row groups
// of one LDS write, 4 rows apart, fall in different banks), in an area of its
// own beside the ring.
constexpr int kStagePitch = 144, kStageBytes = 16 * kStagePitch;
static_assert(kRingBytes + kWaves * kStageBytes + 4 * BN + 16 <= 160 * 1024, "ring, staging and scales fit the LDS");

// One projection of a launch: its operands and output tiles.
struct Member {
  const bf16_t* x;
  const bf16_t* s;
  const bf16_t* w0;
  const bf16_t* u;
  const bf16_t* t;
  bf16_t* y;
  int O;
  int tiles_n;
  int wide;  // y 16-byte aligned and O a multiple of 8: rows leave in 16-byte pieces
};

// A launch covers the output tiles of n projections that share the token
// count, in_dim and rank (the members of a group, or one projection): member
// j owns tiles [start[j], start[j+1]) of the processing order.
struct Args {
  int n;
  int start[kMaxProjections + 1];
  Member mem[kMaxProjections];
  int M, I, R;
  int tiles_m;
  int KT, KR;        // k-tiles of in_dim and of rank
  int split_tiles;   // tiles [0, split_tiles) are split into S k-slices ...
  int S, kps;        // ... of kps k-tiles each (the last may be shorter)
  int xcd_major;     // 1: workgroup g takes position (g % 8) * (grid / 8) + g / 8
  unsigned* ctrl;
  const unsigned* err;  // sticky error word: while set, tiles are written as NaN and no counter is touched
  float* part;       // [S * split_tiles][kPartFloats] partials, slice-major
  int polls;         // bound of a slice's wait for the other slices of its tile
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
// The tile bases and strides of one pair of operands (all uniform; the
// buffer descriptors are built from them where the loads are issued, so that
// choosing between two pairs is a choice between scalars); the per-lane parts
// of the addresses are in Lanes.
struct Operands {
  const bf16_t* a;
  const bf16_t* b;
  int abytes, bbytes;  // bytes of the tile's rows of each operand (loads past them return zeros)
  int row_bytes;   // bytes of one row (k elements)
  int rowstep8;    // bytes of 8 rows (soffset step between the loads j)
  int kel;         // reduction length in elements
};

__device__ __forceinline__ Operands make_operands(const bf16_t* a, int arows, const bf16_t* b, int brows, int m0,
                                                  int n0, int k) {
  Operands o;
  const int ar = min(arows - m0, BM), br = min(brows - n0, BN);
  o.a = a + size_t(m0) * k;
  o.b = b + size_t(n0) * k;
  o.abytes = ar * k * 2;
  o.bbytes = br * k * 2;
  o.row_bytes = k * 2;
  o.rowstep8 = 8 * k * 2;
  o.kel = k;
  return o;
}

// Lane addresses in the LDS ring, built once per workgroup.
struct Lanes {
  unsigned dma_a, dma_b;  // this wave's first 1 KB of A and of B in buffer 0 (uniform)
  // Global side of the direct-to-LDS loads: load j of the wave covers rows
  // w*32 + 8j + lane/8 (the even and the odd j share the swizzle), the lane
  // fetching chunk ce (even j) or co (odd j) of its row.
  int row_e, ce, co;
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
  ln.row_e = w * 32 + (l >> 3);
  ln.ce = (l & 7) ^ ((ln.row_e >> 1) & 7);
  ln.co = (l & 7) ^ (((ln.row_e + 8) >> 1) & 7);
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
__device__ __forceinline__ bf16_t* uniform_ptr(const bf16_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v)), hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<bf16_t*>((uint64_t(hi) << 32) | lo);
}

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
  int ve = ln.row_e * o.row_bytes + (ln.ce << 4), vo = ln.row_e * o.row_bytes + (ln.co << 4);
  const int left = o.kel - kt * BK;
  if (left < BK) {
    ve = ln.ce * 8 < left ? ve : int(kOutOfRange);
    vo = ln.co * 8 < left ? vo : int(kOutOfRange);
  }
  // Every operand here is uniform; readfirstlane says so to the compiler,
  // which cannot always prove it for a choice between two operand pairs.
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(o.a), 0, __builtin_amdgcn_readfirstlane(o.abytes), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(o.b), 0, __builtin_amdgcn_readfirstlane(o.bbytes), kRsrcFlags);
  const int soff = __builtin_amdgcn_readfirstlane(kt * BK * 2), step = __builtin_amdgcn_readfirstlane(o.rowstep8);
  dma4(ln.dma_a + BUF * kTileBytes, ra, ve, vo, soff, step);
  dma4(ln.dma_b + BUF * kTileBytes, rb, ve, vo, soff, step);
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

// The k-tiles of one work item: nmain k-tiles of x . W0^T from kb, then
// (for the workgroup that adds the rank term) KR k-tiles of T . U^T.  The
// accumulators are scaled by s after the last k-tile of x . W0^T.
struct KSeq {
  Operands main, rank;
  int kb, nmain, n;
};

template <int BUF>
__device__ __forceinline__ void issue_seq(const KSeq& q, const Lanes& ln, int t) {
  const bool m = t < q.nmain;
  Operands o;
  o.a = m ? q.main.a : q.rank.a;
  o.b = m ? q.main.b : q.rank.b;
  o.abytes = m ? q.main.abytes : q.rank.abytes;
  o.bbytes = m ? q.main.bbytes : q.rank.bbytes;
  o.row_bytes = m ? q.main.row_bytes : q.rank.row_bytes;
  o.rowstep8 = m ? q.main.rowstep8 : q.rank.rowstep8;
  o.kel = m ? q.main.kel : q.rank.kel;
  issue<BUF>(o, ln, m ? q.kb + t : t - q.nmain);
}

// The first two k-tiles of a sequence into buffers 0 and 1 (the ring must be
// free).
__device__ __forceinline__ void prefetch(const KSeq& q, const Lanes& ln) {
  issue_seq<0>(q, ln, 0);
  if (q.n > 1) issue_seq<1>(q, ln, 1);
}

// One k-tile in software-pipelined form.  On entry k-tile t sits in LDS
// buffer BUF and its k16 steps 0 and 1 are in (fa0, fb0) and (fa1, fb1); the
// loads of k-tile t+1 into the other buffer are in flight.  Steps 2 and 3 are
// read while steps 0 and 1 multiply; the barrier falls between steps 2 and 3,
// once k-tile t+1 has landed; then k-tile t+2 (if any) is issued into BUF
// (free: every wave has read its steps) while step 3's products cover the
// first reads of k-tile t+1.  On exit the invariant holds for k-tile t+1.
template <int BUF>
__device__ __forceinline__ void k_step(const KSeq& q, const Lanes& ln, int t, u32x4 (&fa0)[4], u32x4 (&fb0)[TJ],
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
  if (t + 2 < q.n) issue_seq<BUF>(q, ln, t + 2);
  __builtin_amdgcn_sched_barrier(0);
  mma_step(fa1, fb1, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<1 - BUF>(ln, 1, fa1, fb1);
}

__device__ __forceinline__ void scale_cols(f32x16 (&acc)[4][TJ], const float (&sc)[TJ]) {
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][j] *= sc[j];
}

// k-tiles t .. te-1 of a sequence (k-tile t sits in buffer t & 1).
__device__ __forceinline__ void k_range(const KSeq& q, const Lanes& ln, int t, int te, u32x4 (&fa0)[4],
                                        u32x4 (&fb0)[TJ], u32x4 (&fa1)[4], u32x4 (&fb1)[TJ], f32x16 (&acc)[4][TJ]) {
  if (t < te && (t & 1)) {
    k_step<1>(q, ln, t, fa0, fb0, fa1, fb1, acc);
    ++t;
  }
  for (; t + 1 < te; t += 2) {
    k_step<0>(q, ln, t, fa0, fb0, fa1, fb1, acc);
    k_step<1>(q, ln, t + 1, fa0, fb0, fa1, fb1, acc);
  }
  if (t < te) k_step<0>(q, ln, t, fa0, fb0, fa1, fb1, acc);
}

// acc = the sequence's reduction (x . W0^T over its k-tiles, scaled by sc,
// plus T . U^T when it has rank k-tiles).  Its first two k-tiles were issued
// by prefetch(); every vector memory operation of the wave issued before
// (stores of the previous item included) is waited for.  Leaves the LDS ring
// free and no load in flight.  s_own: the scale of column threadIdx.x of the
// tile (threads below BN), passed on to every wave through s_tile in LDS.
__device__ __forceinline__ void k_run(const KSeq& q, float s_own, float* s_tile, f32x16 (&acc)[4][TJ],
                                      const Lanes& ln) {
  u32x4 fa0[4], fb0[TJ], fa1[4], fb1[TJ];
  wait_dma();
  if (threadIdx.x < BN) s_tile[threadIdx.x] = s_own;
  __syncthreads();
  read_frags<0>(ln, 0, fa0, fb0);
  read_frags<0>(ln, 1, fa1, fb1);
  k_range(q, ln, 0, q.nmain, fa0, fb0, fa1, fb1, acc);
  float sc[TJ];
  const int wn = int(threadIdx.x) / kWave % WN, lr = int(threadIdx.x) & 31;
#pragma unroll
  for (int j = 0; j < TJ; ++j) sc[j] = s_tile[wn * (BN / WN) + j * 32 + lr];
  scale_cols(acc, sc);
  k_range(q, ln, q.nmain, q.n, fa0, fb0, fa1, fb1, acc);
  wait_dma();
  __syncthreads();
}

// Tile u of the processing order -> (member, token tile, output tile).
// Within a member, groups of eight token tiles are walked column by column,
// so workgroups that run together share x and W0 rows in L2.
__device__ __forceinline__ int tile_coords(const Args& a, int u, int& tm, int& tn) {
  int j = 0;
  while (j + 1 < a.n && u >= a.start[j + 1]) ++j;
  u -= a.start[j];
  const int tiles_n = a.mem[j].tiles_n;
  const int per_group = 8 * tiles_n;
  const int first = (u / per_group) * 8, gsize = min(a.tiles_m - first, 8), r = u % per_group;
  tm = first + r % gsize;
  tn = r / gsize;
  return j;
}

// Work item v of the launch: the k-slices of the split tiles first
// (slice-major), then the whole tiles.
struct Item {
  int u, slice;    // tile of the processing order; k-slice, or -1 for a whole tile
  int mj, m0, n0;  // member, first token and first output column
  int kb, ke;      // k-tiles of x . W0^T
  int rank;        // whether the item adds the rank term
};

__device__ __forceinline__ Item make_item(const Args& a, int v) {
  Item it;
  const int nsplit = a.split_tiles * a.S;
  it.kb = 0;
  it.ke = a.KT;
  if (v < nsplit) {
    it.u = v % a.split_tiles;
    it.slice = v / a.split_tiles;
    it.kb = it.slice * a.kps;
    it.ke = min(a.KT, it.kb + a.kps);
  } else {
    it.u = a.split_tiles + (v - nsplit);
    it.slice = -1;
  }
  int tm, tn;
  it.mj = tile_coords(a, it.u, tm, tn);
  it.m0 = tm * BM;
  it.n0 = tn * BN;
  // The rank term goes to the whole tile or to the last k-slice (the one
  // ending at the last k-tile).
  it.rank = a.R > 0 && (it.slice < 0 || it.ke == a.KT) ? 1 : 0;
  return it;
}

__device__ __forceinline__ KSeq make_seq(const Args& a, const Item& it) {
  const Member& mb = a.mem[it.mj];
  KSeq q;
  q.main = make_operands(mb.x, a.M, mb.w0, mb.O, it.m0, it.n0, a.I);
  q.rank = make_operands(mb.t, a.M, mb.u, mb.O, it.m0, it.n0, a.R);  // unused without rank k-tiles
  q.kb = it.kb;
  q.nmain = it.ke - it.kb;
  q.n = q.nmain + (it.rank ? a.KR : 0);
  return q;
}

// Round the wave's 128 x 64 block to bf16 and store it, 16 rows at a time
// through the wave's LDS staging area (outside the ring, so the next item's
// first k-tiles can land meanwhile): the accumulator layout gives a lane one
// column of four rows, the staging turns that into eight columns of one row,
// so each lane stores 16 contiguous bytes.
__device__ __forceinline__ void store_tile(const Args& a, const Member& mb, int m0, int n0, const f32x16 (&acc)[4][TJ],
                                           lds_byte* stage) {
  const int w = int(threadIdx.x) / kWave, l = int(threadIdx.x) % kWave, lr = l & 31, hi = l >> 5;
  const int wm = w / WN, wn = w % WN;
  lds_byte* const base = stage + w * kStageBytes;
  lds_byte* const wr = base + 4 * hi * kStagePitch + lr * 2;            // row 4 hi (+ 8b' + e), column lr (+ 32j)
  lds_byte* const rd = base + (l >> 3) * kStagePitch + (l & 7) * 16;    // row l/8 (+ 8r), columns 8 (l%8) .. +7
  const int n = n0 + wn * (BN / WN) + (l & 7) * 8;
  const bool wide = mb.wide && n + 8 <= mb.O;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      // Rows 32i + 16p + (8b' + 4hi + e) of the wave's block, b = 2p + b'.
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<lds_u16*>(wr + (8 * bb + e) * kStagePitch + j * 64) =
                f32_to_bf16(acc[i][j][4 * (2 * p + bb) + e]);
      // The wave reads back only what it wrote, and a wave's LDS operations
      // complete in order: no barrier, only no compiler reordering.
      asm volatile("" ::: "memory");
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const u32x4 v = *reinterpret_cast<const lds_u32x4*>(rd + r * 8 * kStagePitch);
        const int m = m0 + wm * 128 + i * 32 + p * 16 + r * 8 + (l >> 3);
        if (m >= a.M) continue;
        bf16_t* dst = mb.y + size_t(m) * mb.O + n;
        if (wide) {
          *reinterpret_cast<u32x4*>(dst) = v;
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if (n + t < mb.O) dst[t] = bf16_t{uint16_t(v[t / 2] >> (16 * (t % 2)))};
        }
      }
      asm volatile("" ::: "memory");
    }
}

// NaN over the whole tile (a poisoned workspace).
__device__ __forceinline__ void nan_tile(const Args& a, const Member& mb, int m0, int n0) {
  for (int e = int(threadIdx.x); e < BM * BN; e += kThreads) {
    const int m = m0 + e / BN, n = n0 + e % BN;
    if (m < a.M && n < mb.O) mb.y[size_t(m) * mb.O + n] = bf16_t{f32_to_bf16(__builtin_nanf(""))};
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const Args& a, int slot) {
  return __builtin_amdgcn_make_buffer_rsrc(a.part + size_t(slot) * kPartFloats, 0, kPartFloats * 4, kRsrcFlags);
}

// Partials are laid out as the accumulators sit in registers: 16-byte piece
// q = (TJ i + j) * 4 + c of every lane, lanes contiguous.
constexpr int kPieces = 4 * TJ * 4;

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

// The tile of a slice that has stored its partial: every slice of the tile
// sums its share of the pieces over all S partials, in slice order (so the
// result does not depend on which slice arrives when), rounds and stores it.
// Each partial already carries the scale by s, and the last slice's the rank
// term.  False if the wait for the other slices timed out (nothing stored).
// Needs S >= 2 (a slice's share is then at most half of the pieces).
__device__ __forceinline__ bool reduce_share(const Args& a, const Member& mb, int u, int slice, int m0, int n0,
                                             unsigned* s_flag) {
  unsigned* counter = &a.ctrl[kCounterBase + u];
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = false;
    for (int it = 0; it < a.polls && !ok; ++it) {
      ok = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= unsigned(a.S);
      if (!ok) __builtin_amdgcn_s_sleep(1);
    }
    *s_flag = ok ? 1u : 0u;
  }
  __syncthreads();
  const bool ok = *s_flag != 0u;
  __syncthreads();  // every wave has read *s_flag before it is reused
  if (!ok) return false;
  const int w = int(threadIdx.x) / kWave, l = int(threadIdx.x) % kWave, lr = l & 31, hi = l >> 5;
  const int wm = w / WN, wn = w % WN;
  // This slice's pieces [p0, p0 + np) (np <= kPieces / 2 = 16), in batches
  // of eight: a batch's loads of one partial are in flight together (past
  // the share, a batch re-reads its last piece and drops it).
  const int p0 = slice * kPieces / a.S, np = (slice + 1) * kPieces / a.S - p0;
  const int lane_off = int(threadIdx.x) * 16;
  for (int k0 = 0; k0 < np; k0 += 8) {
    f32x4 sum[8];
    for (int q = 0; q < a.S; ++q) {
      const __amdgpu_buffer_rsrc_t rs = part_rsrc(a, q * a.split_tiles + u);
      u32x4 d[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        d[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off, (p0 + min(k0 + k, np - 1)) * kThreads * 16,
                                                     kCoherent);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const f32x4 f = {__uint_as_float(d[k][0]), __uint_as_float(d[k][1]), __uint_as_float(d[k][2]),
                         __uint_as_float(d[k][3])};
        sum[k] = q == 0 ? f : sum[k] + f;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int pc = p0 + k0 + k;
      if (k0 + k >= np) break;
      const int i = pc / (TJ * 4), j = (pc / 4) % TJ, c = pc % 4;
      const int n = n0 + wn * (BN / WN) + j * 32 + lr;
      if (n >= mb.O) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 128 + i * 32 + 8 * c + 4 * hi + e;
        if (m < a.M) mb.y[size_t(m) * mb.O + n] = bf16_t{f32_to_bf16(sum[k][e])};
      }
    }
  }
  // Count out: the last of the tile's 2S arrivals resets the counter for the
  // next launch (every slice has passed its wait by then).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == unsigned(2 * a.S - 1))
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Persistent workgroups: workgroup g takes items pos, pos + G, ... where pos
// spreads the grid XCD-major.  Each item's first two k-tiles are loaded while
// the previous item stores its results.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4))) void gemm_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRingBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves * kStageBytes];
  __shared__ float s_tile[BN];
  __shared__ unsigned s_flag;
  const int g = int(blockIdx.x), G = int(gridDim.x);
  const int pos = a.xcd_major ? (g % 8) * (G / 8) + g / 8 : g;
  const int total = a.split_tiles * a.S + (a.start[a.n] - a.split_tiles);
  const Lanes ln = make_lanes(ring);
  // Poisoned workspace (thread 0's copy of the error word decides for the
  // workgroup): every item writes NaN over its tile and touches no counter.
  if (threadIdx.x == 0) s_flag = load_error_word(a.err);
  __syncthreads();
  const bool poisoned = s_flag != 0u;
  __syncthreads();
  if (pos >= total) return;
  Item it = make_item(a, pos);
  prefetch(make_seq(a, it), ln);
  for (int v = pos; v < total; v += G) {
    const Member& mb = a.mem[it.mj];
    float s_own = 0.f;
    if (threadIdx.x < BN) {
      const int n = it.n0 + int(threadIdx.x);
      s_own = n < mb.O ? (mb.s ? bf16_to_f32(mb.s[n].bits) : 1.f) : 0.f;
    }
    f32x16 acc[4][TJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};
    k_run(make_seq(a, it), s_own, s_tile, acc, ln);
    const Item cur = it;
    if (v + G < total) {
      it = make_item(a, v + G);
      prefetch(make_seq(a, it), ln);
    }
    if (poisoned) {
      nan_tile(a, mb, cur.m0, cur.n0);
    } else if (cur.slice < 0) {
      store_tile(a, mb, cur.m0, cur.n0, acc, (lds_byte*)stage);
    } else {
      store_partial(a, cur.slice * a.split_tiles + cur.u, acc);
      __builtin_amdgcn_s_waitcnt(0);  // partial written through before counting in
      __syncthreads();
      if (!reduce_share(a, mb, cur.u, cur.slice, cur.m0, cur.n0, &s_flag)) {
        if (threadIdx.x == 0) atomicOr(const_cast<unsigned*>(a.err), 1u);
        nan_tile(a, mb, cur.m0, cur.n0);
      }
    }
  }
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

// T tiles are BM tokens x BN columns.  Four waves: with BN = 256 each takes
// 64 columns of all BM rows, with BN = 128 a (BM/2)-row x 64-column quarter;
// products of 32 x 32.
constexpr int BK = 64, kThreads = 256;
constexpr int kXPitch = BK * 2 + 16;   // 144-byte rows of the x tile
// x tiles are read by one column block of T only (rank <= 256), while every
// row block re-reads the V tiles: x is loaded non-temporal (the NT bit of the
// buffer load's cache policy) so that it does not push V out of L2.
constexpr int kXPolicy = 2;

template <int BM, int BN>
struct Geo {
  static constexpr int kXTile = BM * kXPitch;     // 9 or 18 KB
  static constexpr int XQ = BM / 32;              // x loads per lane and k-tile (32 rows per pass)
  static constexpr int kVPitch = BN * 2 + 64;     // bytes per row of the V tile: 16 banks of skew per row
  static constexpr int kVTile = BK * kVPitch;     // 36 or 20 KB
  static constexpr int kRingBytes = 2 * kVTile + 2 * kXTile;  // [V0][V1][X0][X1]
  static constexpr int kPartFloats = BM * BN;
  static constexpr int VL = BN / 8;               // lanes per V row (16-byte chunks)
  static constexpr int VR = kThreads / VL;        // V rows per staging pass
  static constexpr int VQ = BK / VR;              // V loads per lane and k-tile
  static constexpr int WR = BN == 256 ? BM : BM / 2;  // rows of a wave
  static constexpr int AI = WR / 32;              // 32-row products per wave
  static constexpr int AJ = 2;                    // 32-column products per wave
  static constexpr int kPieces = AI * AJ * 4;     // 16-byte pieces of a lane's accumulators
  __device__ static int row0(int w) { return BN == 256 ? 0 : WR * (w >> 1); }
  __device__ static int col0(int w) { return BN == 256 ? 64 * w : 64 * (w & 1); }
  static_assert(VQ * VR == BK, "V staging covers a k-tile");
  static_assert(kPartFloats * 4 == kPieces * kThreads * 16, "partial = every lane's pieces");
  static_assert(AI >= 1 && AI <= 2, "one or two row products per wave");
};

// One projection of a launch: its x, V and T.
struct Member {
  const bf16_t* x;
  const bf16_t* v;
  bf16_t* t;
};

// The n projections of one launch share the token count, in_dim and rank;
// member j owns workgroups [j, j+1) x RB * CB * KS of the grid, and its tiles
// are numbered j * RB * CB + (local tile) for the arrival counters and the
// partials.
struct Args {
  int n;
  Member mem[kMaxProjections];
  int M, I, R;
  int RB, CB, KT;  // row blocks, column blocks, k-tiles of in_dim
  int KS, kps;     // k-slices and k-tiles per slice
  unsigned* ctrl;
  const unsigned* err;  // sticky error word: while set, nothing is published and no counter is touched
  float* part;     // [RB * CB][KS][BM * BN]
  int polls;       // bound of a slice's wait for the other slices of its tile
};

struct Lanes {
  lds_byte* x_rd;   // A fragment: row row0(w) + lane%32, k half lane/32
  lds_byte* v_rd0;  // transposing B reads, buffer 0 / 1
  lds_byte* v_rd1;
  lds_byte* x_wr;   // x staging: row tid/8, chunk tid%8
  lds_byte* v_wr0;  // V staging: k-row tid/VL, chunk tid%VL, buffer 0 / 1
  lds_byte* v_wr1;
};

template <int BM, int BN>
__device__ __forceinline__ Lanes make_lanes(uint8_t* ring) {
  using G = Geo<BM, BN>;
  lds_byte* base = (lds_byte*)ring;
  const int tid = int(threadIdx.x), w = tid / kWave, l = tid % kWave, lr = l & 31, hi = l >> 5;
  const int g = l >> 4, j16 = l & 15;
  const int vrow = 8 * (g >> 1) + (j16 >> 2), vcol = G::col0(w) + 16 * (g & 1) + 4 * (j16 & 3);
  Lanes ln;
  ln.x_rd = opaque(base + 2 * G::kVTile + (G::row0(w) + lr) * kXPitch + hi * 16);
  ln.v_rd0 = opaque(base + vrow * G::kVPitch + vcol * 2);
  ln.v_rd1 = opaque(base + G::kVTile + vrow * G::kVPitch + vcol * 2);
  ln.x_wr = opaque(base + 2 * G::kVTile + (tid >> 3) * kXPitch + (tid & 7) * 16);
  ln.v_wr0 = opaque(base + (tid / G::VL) * G::kVPitch + (tid % G::VL) * 16);
  ln.v_wr1 = opaque(base + G::kVTile + (tid / G::VL) * G::kVPitch + (tid % G::VL) * 16);
  return ln;
}

struct Src {
  __amdgpu_buffer_rsrc_t rx, rv;
  int xoff, voff;     // lane byte offsets: x row tid/8 chunk tid%8; V k-row tid/VL chunk tid%VL
  int xstep, vstep;   // bytes of 32 x rows / VR V rows
  int I, ncols;       // reduction length; valid columns of this column block
};

template <int BM, int BN>
__device__ __forceinline__ void fetch(const Src& s, int kt, u32x4 (&px)[Geo<BM, BN>::XQ],
                                      u32x4 (&pv)[Geo<BM, BN>::VQ]) {
  using G = Geo<BM, BN>;
#pragma unroll
  for (int q = 0; q < G::XQ; ++q)
    px[q] = __builtin_amdgcn_raw_buffer_load_b128(s.rx, s.xoff, kt * BK * 2 + q * s.xstep, kXPolicy);
#pragma unroll
  for (int q = 0; q < G::VQ; ++q)
    pv[q] = __builtin_amdgcn_raw_buffer_load_b128(s.rv, s.voff, kt * G::VQ * s.vstep + q * s.vstep, 0);
}

template <int BM, int BN, int BUF>
__device__ __forceinline__ void stage(const Lanes& ln, const Src& s, int kt, u32x4 (&px)[Geo<BM, BN>::XQ],
                                      u32x4 (&pv)[Geo<BM, BN>::VQ]) {
  using G = Geo<BM, BN>;
  // x chunks at or past in_dim would read the next row: zero them.  V rows
  // past in_dim read as zero from the buffer bound; V columns past r of this
  // block would read the next row: zero them.
  if (s.I - kt * BK < BK) {
    const bool keep = int(threadIdx.x & 7) * 8 < s.I - kt * BK;
#pragma unroll
    for (int q = 0; q < G::XQ; ++q) px[q] = keep ? px[q] : u32x4{0u, 0u, 0u, 0u};
  }
  if (s.ncols < BN) {
    const bool keep = int(threadIdx.x % G::VL) * 8 < s.ncols;
#pragma unroll
    for (int q = 0; q < G::VQ; ++q) pv[q] = keep ? pv[q] : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int q = 0; q < G::XQ; ++q) *reinterpret_cast<lds_u32x4*>(ln.x_wr + BUF * G::kXTile + q * 32 * kXPitch) = px[q];
#pragma unroll
  for (int q = 0; q < G::VQ; ++q)
    *reinterpret_cast<lds_u32x4*>((BUF ? ln.v_wr1 : ln.v_wr0) + q * G::VR * G::kVPitch) = pv[q];
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int BM, int BN, int BUF>
__device__ __forceinline__ void read_frags(const Lanes& ln, int st, u32x4 (&fa)[Geo<BM, BN>::AI], u32x4 (&fb)[2]) {
  using G = Geo<BM, BN>;
#pragma unroll
  for (int i = 0; i < G::AI; ++i)
    fa[i] = *reinterpret_cast<const lds_u32x4*>(ln.x_rd + BUF * G::kXTile + i * 32 * kXPitch + st * 32);
  lds_byte* vr = BUF ? ln.v_rd1 : ln.v_rd0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vr + (16 * st) * G::kVPitch + 64 * j));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vr + (16 * st + 4) * G::kVPitch + 64 * j));
    fb[j] = u32x4{uint32_t(uint16_t(lo[0])) | (uint32_t(uint16_t(lo[1])) << 16),
                  uint32_t(uint16_t(lo[2])) | (uint32_t(uint16_t(lo[3])) << 16),
                  uint32_t(uint16_t(hi[0])) | (uint32_t(uint16_t(hi[1])) << 16),
                  uint32_t(uint16_t(hi[2])) | (uint32_t(uint16_t(hi[3])) << 16)};
  }
}

template <int AI>
__device__ __forceinline__ void mma_step(const u32x4 (&fa)[AI], const u32x4 (&fb)[2], f32x16 (&acc)[AI][2]) {
#pragma unroll
  for (int i = 0; i < AI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[i]),
                                                          __builtin_bit_cast(bf16x8, fb[j]), acc[i][j], 0, 0, 0);
}

template <int BM, int BN, int BUF>
__device__ __forceinline__ void multiply_tile(const Lanes& ln, f32x16 (&acc)[Geo<BM, BN>::AI][2]) {
  constexpr int AI = Geo<BM, BN>::AI;
  u32x4 fa0[AI], fb0[2], fa1[AI], fb1[2];
  read_frags<BM, BN, BUF>(ln, 0, fa0, fb0);
  read_frags<BM, BN, BUF>(ln, 1, fa1, fb1);
  __builtin_amdgcn_sched_barrier(0);
  mma_step<AI>(fa0, fb0, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<BM, BN, BUF>(ln, 2, fa0, fb0);
  __builtin_amdgcn_sched_barrier(0);
  mma_step<AI>(fa1, fb1, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_frags<BM, BN, BUF>(ln, 3, fa1, fb1);
  __builtin_amdgcn_sched_barrier(0);
  mma_step<AI>(fa0, fb0, acc);
  __builtin_amdgcn_sched_barrier(0);
  mma_step<AI>(fa1, fb1, acc);
}

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void xv_kernel(Args a) {
  using G = Geo<BM, BN>;
  constexpr int AI = G::AI, VQ = G::VQ, XQ = G::XQ;
  __shared__ __attribute__((aligned(16))) uint8_t ring[G::kRingBytes];
  __shared__ unsigned s_last;
  const int tid = int(threadIdx.x);
  const int per_member = a.RB * a.CB * a.KS;
  const int mj = int(blockIdx.x) / per_member, b = int(blockIdx.x) % per_member;
  const Member& mb = a.mem[mj];
  const int ks = b % a.KS, ltile = b / a.KS, tile = mj * a.RB * a.CB + ltile;
  const int rb = ltile / a.CB, cb = ltile % a.CB;
  const int m0 = rb * BM, n0 = cb * BN;
  const int kb = ks * a.kps, ke = min(a.KT, kb + a.kps);
  const Lanes ln = make_lanes<BM, BN>(ring);
  const uint32_t err_at_entry = load_error_word(a.err);
  Src s;
  s.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(mb.x + size_t(m0) * a.I), 0,
                                          min(a.M - m0, BM) * a.I * 2, kRsrcFlags);
  s.rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(mb.v + n0), 0, (a.I * a.R - n0) * 2, kRsrcFlags);
  s.xoff = (tid >> 3) * a.I * 2 + (tid & 7) * 16;
  s.voff = (tid / G::VL) * a.R * 2 + (tid % G::VL) * 16;
  s.xstep = 32 * a.I * 2;
  s.vstep = G::VR * a.R * 2;
  s.I = a.I;
  s.ncols = min(BN, a.R - n0);

  f32x16 acc[AI][2];
#pragma unroll
  for (int i = 0; i < AI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  if (kb < ke) {
    const int n = ke - kb;
    u32x4 px0[XQ], pv0[VQ], px1[XQ], pv1[VQ];
    fetch<BM, BN>(s, kb, px0, pv0);
    fetch<BM, BN>(s, min(kb + 1, ke - 1), px1, pv1);
    stage<BM, BN, 0>(ln, s, kb, px0, pv0);
    __syncthreads();
    for (int k = 0; k < n; k += 2) {
      const int k1 = min(kb + k + 1, ke - 1), k2 = min(kb + k + 2, ke - 1), k3 = min(kb + k + 3, ke - 1);
      fetch<BM, BN>(s, k2, px0, pv0);
      __builtin_amdgcn_sched_barrier(0);
      multiply_tile<BM, BN, 0>(ln, acc);
      __builtin_amdgcn_sched_barrier(0);
      stage<BM, BN, 1>(ln, s, k1, px1, pv1);
      __syncthreads();
      if (k + 1 < n) {
        fetch<BM, BN>(s, k3, px1, pv1);
        __builtin_amdgcn_sched_barrier(0);
        multiply_tile<BM, BN, 1>(ln, acc);
        __builtin_amdgcn_sched_barrier(0);
        stage<BM, BN, 0>(ln, s, k2, px0, pv0);
        __syncthreads();
      }
    }
  }

  // Poisoned workspace: the projection's y is written as NaN, so T is not needed.
  if (tid == 0) s_last = err_at_entry;
  __syncthreads();
  if (s_last != 0u) return;
  __syncthreads();
  const int w = tid / kWave, l = tid % kWave, lr = l & 31, hi = l >> 5;
  const int wr = G::row0(w), wc = G::col0(w);
  if (a.KS > 1) {
    // Partial in register order: 16-byte piece q = (2i + j) * 4 + c of every
    // lane.  Every slice of the tile then waits (bounded) for the others and
    // sums its share of the pieces over all KS partials in slice order, so
    // the result does not depend on arrival order.
    float* blk = a.part + size_t(tile) * a.KS * G::kPartFloats;
    const __amdgpu_buffer_rsrc_t mine =
        __builtin_amdgcn_make_buffer_rsrc(blk + size_t(ks) * G::kPartFloats, 0, G::kPartFloats * 4, kRsrcFlags);
#pragma unroll
    for (int i = 0; i < AI; ++i)
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
    unsigned* counter = &a.ctrl[kCounterBase + tile];
    if (tid == 0) {
      __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bool ok = false;
      for (int it = 0; it < a.polls && !ok; ++it) {
        ok = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= unsigned(a.KS);
        if (!ok) __builtin_amdgcn_s_sleep(1);
      }
      s_last = ok ? 1u : 0u;
      if (!ok) atomicOr(const_cast<unsigned*>(a.err), 1u);
    }
    __syncthreads();
    if (s_last == 0u) return;  // timed out: the sticky error word makes the projection's y NaN
    constexpr int kPieces = G::kPieces;
    const int p0 = ks * kPieces / a.KS, np = (ks + 1) * kPieces / a.KS - p0;
    f32x4 sum[kPieces / 2];
    for (int k0 = 0; k0 < np; k0 += kPieces / 2) {
      for (int q = 0; q < a.KS; ++q) {
        const __amdgpu_buffer_rsrc_t src =
            __builtin_amdgcn_make_buffer_rsrc(blk + size_t(q) * G::kPartFloats, 0, G::kPartFloats * 4, kRsrcFlags);
        u32x4 d[kPieces / 2];
#pragma unroll
        for (int k = 0; k < kPieces / 2; ++k)
          d[k] = __builtin_amdgcn_raw_buffer_load_b128(src, tid * 16, (p0 + min(k0 + k, np - 1)) * kThreads * 16,
                                                       kCoherent);
#pragma unroll
        for (int k = 0; k < kPieces / 2; ++k) {
          const f32x4 f = {__uint_as_float(d[k][0]), __uint_as_float(d[k][1]), __uint_as_float(d[k][2]),
                           __uint_as_float(d[k][3])};
          sum[k] = q == 0 ? f : sum[k] + f;
        }
      }
#pragma unroll
      for (int k = 0; k < kPieces / 2; ++k) {
        if (k0 + k >= np) break;
        const int pc = p0 + k0 + k, i = pc / 8, j = (pc / 4) % 2, bb = pc % 4;
        const int n = n0 + wc + 32 * j + lr;
        if (n >= a.R) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + wr + 32 * i + 8 * bb + 4 * hi + e;
          if (m < a.M) mb.t[size_t(m) * a.R + n] = bf16_t{f32_to_bf16(sum[k][e])};
        }
      }
    }
    // Count out: the last of the tile's 2 KS arrivals resets the counter for
    // the next launch (every slice has passed its wait by then).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0 &&
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == unsigned(2 * a.KS - 1))
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
#pragma unroll
  for (int i = 0; i < AI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wc + 32 * j + lr;
      if (n >= a.R) continue;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + wr + 32 * i + 8 * bb + 4 * hi + e;
          if (m < a.M) mb.t[size_t(m) * a.R + n] = bf16_t{f32_to_bf16(acc[i][j][4 * bb + e])};
        }
    }
}

// Tile shape of T for a rank: 64 x 128 up to rank 128 (a 256-column tile
// would load and multiply a dead half of V), else 64 x 256.  (128 x 128 at
// rank 256, two workgroups per compute unit and a fifth fewer bytes per flop,
// ran the 60-layer stack at 4096 tokens no faster.)
inline int block_rows(int64_t) { return 64; }
inline int block_cols(int64_t rank) { return rank <= 128 ? 128 : 256; }

}  // namespace xv

}  // namespace

namespace {

// Cost model of the split remainder round, in k-tiles of one workgroup:
// storing a 256 x 256 fp32 partial and reading one back each cost about as
// much as a few k-tiles of multiplication; slices shorter than kMinSlice
// k-tiles are not worth their partials.
constexpr int kStoreCost = 6, kLoadCost = 4, kMinSlice = 4;

}  // namespace

GemmPlan plan_gemm(int n, const int64_t* out_dims, int64_t m, int64_t in_dim, int64_t rank, int cus) {
  GemmPlan p{};
  p.n = n;
  // Each member's T, then the launch's x . V partials, then the split tiles'
  // partials.
  size_t off = 0;
  for (int j = 0; j < n; ++j) {
    p.off_t[j] = off;
    off = align_up(off + size_t(m) * size_t(rank) * 2, 256);
  }
  p.bytes = off;
  // The matrix-core kernels for 16-byte aligned rows address one tile's rows
  // (and all of V) with 32-bit byte offsets.
  p.aligned = in_dim % 8 == 0 && rank % 8 == 0 && in_dim < (int64_t(1) << 22) && rank < (int64_t(1) << 22) &&
              in_dim * rank < (int64_t(1) << 30);
  p.tiles_m = int((m + big::BM - 1) / big::BM);
  p.KT = int((in_dim + big::BK - 1) / big::BK);
  p.KR = int((rank + big::BK - 1) / big::BK);
  const auto general = [&] {
    p.big = 0;
    p.split_tiles = 0;
    p.tiles_m = int((m + BM - 1) / BM);
    p.start[0] = 0;
    for (int j = 0; j < n; ++j) {
      p.tiles_n[j] = int((out_dims[j] + BN - 1) / BN);
      p.start[j + 1] = p.start[j] + p.tiles_m * p.tiles_n[j];
    }
    p.grid = p.start[n];
  };
  if (!p.aligned) {
    general();
    return p;
  }
  // x . V: enough k-slices to give every compute unit a workgroup, each at
  // least two k-tiles long and at most 16 partials per tile.
  if (rank > 0) {
    p.xv_bm = xv::block_rows(rank);
    p.xv_bn = xv::block_cols(rank);
    p.xv_rb = int((m + p.xv_bm - 1) / p.xv_bm);
    p.xv_cb = int((rank + p.xv_bn - 1) / p.xv_bn);
    p.xv_kt = int((in_dim + xv::BK - 1) / xv::BK);
    const int64_t tiles = int64_t(n) * p.xv_rb * p.xv_cb;
    int64_t ks = tiles >= cus ? 1 : cus / tiles;
    ks = std::min<int64_t>(ks, std::min<int64_t>(16, std::max<int64_t>(1, p.xv_kt / 2)));
    if (tiles > kMaxGroupCounters) ks = 1;
    p.xv_kps = int((p.xv_kt + ks - 1) / ks);
    p.xv_ks = int((p.xv_kt + p.xv_kps - 1) / p.xv_kps);
    p.off_xvpart = off;
    if (p.xv_ks > 1) off = align_up(off + size_t(tiles) * p.xv_ks * p.xv_bm * p.xv_bn * 4, 256);
  }
  p.bytes = off;
  p.start[0] = 0;
  for (int j = 0; j < n; ++j) {
    p.tiles_n[j] = int((out_dims[j] + big::BN - 1) / big::BN);
    p.start[j + 1] = p.start[j] + p.tiles_m * p.tiles_n[j];
  }
  const int64_t tiles = p.start[n], KT = p.KT;
  const int G = cus >= 8 ? cus / 8 * 8 : cus;
  const auto round8 = [&](int64_t g) { return int(cus >= 8 ? std::min<int64_t>(G, (g + 7) / 8 * 8) : std::min<int64_t>(G, g)); };

  // Whole tiles in ceil(tiles / G) rounds ...
  int64_t best = (tiles + G - 1) / G * KT;
  p.big = 1;
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
    general();
    return p;
  }
  p.xcd_major = p.grid % 8 == 0 ? 1 : 0;
  p.off_part = off;
  if (p.split_tiles > 0) p.bytes = off + size_t(p.split_tiles) * p.S * big::kPartFloats * 4;
  return p;
}

hipError_t launch_forward_gemm(const GemmPlan& p, const Projection* projs, int64_t m, int64_t in_dim,
                               int64_t rank, unsigned* ctrl, char* data, const unsigned* err_word, hipStream_t stream) {
  const int n = p.n;
  const auto t_of = [&](int j) { return reinterpret_cast<bf16_t*>(data + p.off_t[j]); };
  if (rank > 0 && p.aligned) {
    xv::Args a;
    a.n = n;
    for (int j = 0; j < n; ++j)
      a.mem[j] = xv::Member{static_cast<const bf16_t*>(projs[j].x), static_cast<const bf16_t*>(projs[j].v), t_of(j)};
    a.M = int(m); a.I = int(in_dim); a.R = int(rank);
    a.RB = p.xv_rb; a.CB = p.xv_cb; a.KT = p.xv_kt;
    a.KS = p.xv_ks; a.kps = p.xv_kps;
    a.ctrl = ctrl;
    a.err = err_word;
    a.part = reinterpret_cast<float*>(data + p.off_xvpart);
    a.polls = decode_wait_polls();
    const dim3 grid(unsigned(n * p.xv_rb * p.xv_cb * p.xv_ks));
    if (p.xv_bm != 64) return hipErrorInvalidValue;
    if (p.xv_bn == 256) hipLaunchKernelGGL((xv::xv_kernel<64, 256>), grid, dim3(xv::kThreads), 0, stream, a);
    else hipLaunchKernelGGL((xv::xv_kernel<64, 128>), grid, dim3(xv::kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (rank > 0) {
    dim3 grid(unsigned((m + kTM - 1) / kTM), unsigned((rank + kTN - 1) / kTN));
    for (int j = 0; j < n; ++j) {
      hipLaunchKernelGGL(xv_gemm_kernel, grid, dim3(kThreads), 0, stream, static_cast<const bf16_t*>(projs[j].x),
                         static_cast<const bf16_t*>(projs[j].v), t_of(j), int(m), int(in_dim), int(rank));
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (p.big) {
    big::Args a;
    a.n = n;
    for (int j = 0; j <= n; ++j) a.start[j] = p.start[j];
    for (int j = 0; j < n; ++j)
      a.mem[j] = big::Member{static_cast<const bf16_t*>(projs[j].x), static_cast<const bf16_t*>(projs[j].s),
                             static_cast<const bf16_t*>(projs[j].w0), static_cast<const bf16_t*>(projs[j].u), t_of(j),
                             static_cast<bf16_t*>(projs[j].y), int(projs[j].out_dim), p.tiles_n[j],
                             int(uintptr_t(projs[j].y) % 16 == 0 && projs[j].out_dim % 8 == 0)};
    a.M = int(m); a.I = int(in_dim); a.R = int(rank);
    a.tiles_m = p.tiles_m;
    a.KT = p.KT; a.KR = p.KR;
    a.split_tiles = p.split_tiles; a.S = p.S; a.kps = p.kps; a.xcd_major = p.xcd_major;
    a.ctrl = ctrl;
    a.err = err_word;
    a.part = reinterpret_cast<float*>(data + p.off_part);
    a.polls = decode_wait_polls();
    hipLaunchKernelGGL(big::gemm_kernel, dim3(unsigned(p.grid)), dim3(big::kThreads), 0, stream, a);
    return hipGetLastError();
  }
  GemmArgs a;
  a.n = n;
  for (int j = 0; j <= n; ++j) a.start[j] = p.start[j];
  for (int j = 0; j < n; ++j)
    a.mem[j] = GemmMember{static_cast<const bf16_t*>(projs[j].x), static_cast<const bf16_t*>(projs[j].s),
                          static_cast<const bf16_t*>(projs[j].w0), static_cast<const bf16_t*>(projs[j].u), t_of(j),
                          static_cast<bf16_t*>(projs[j].y), int(projs[j].out_dim), p.tiles_n[j]};
  a.M = int(m); a.I = int(in_dim); a.R = int(rank);
  a.tiles_m = p.tiles_m;
  a.err = err_word;
  hipLaunchKernelGGL(forward_gemm_kernel, dim3(unsigned(p.grid)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tb
