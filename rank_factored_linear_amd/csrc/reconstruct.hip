// reconstruct_weight: w_out = diag(s) . W0 + U . V^T  ("The theta bundle",
// component table and reconstruction formula).
//
// rank 0 is a pure scaled copy, bound by HBM (wave-contiguous spans, fp32
// output streamed out non-temporal).
// rank > 0 is a K = rank GEMM (U rows and V rows are both contiguous along
// the rank dimension) on the matrix cores with the scaled copy fused into the
// epilogue; at rank 256 it is still HBM-bound (6 bytes of W0 and fp32 output
// per 512 flops) but needs far more than the fp32 vector rate to keep up.
//
// bf16 bundles with rank % 8 == 0 take 128 x 128 output tiles on
// v_mfma_f32_32x32x16_bf16, four waves of 64 x 64: up to rank 256 the
// persistent kernel below (rp), beyond it reconstruct_mfma_kernel (one tile
// per workgroup, k-tiles of 64 staged in LDS with 16-byte chunks XOR-swizzled
// by row).  The product is taken as V . U^T, so that each lane ends up
// holding four consecutive columns of one output row.
#include "tb_device.h"
#include "tb_host.h"
#include "tb_rebuild.h"
#include "tb_reduce.h"

namespace tb {

namespace {

constexpr int kThreads = 256;

// Each wave handles 512 consecutive elements per step as two halves of 256:
// lane l takes elements 4 l .. 4 l + 3 of each half, so every load and store
// instruction covers one contiguous span (512 or 1024 bytes) and the fp32
// stores fill whole cache lines; they are streamed out non-temporal.
template <typename EI, typename EO>
__global__ __launch_bounds__(kThreads) void reconstruct_rank0_kernel(const EI* __restrict__ s, const EI* __restrict__ w0,
                                                                     EO* __restrict__ out, int64_t n, int I) {
  const int l = int(threadIdx.x) & 63;
  const int64_t waves = int64_t(gridDim.x) * (kThreads / kWave);
  for (int64_t wv = int64_t(blockIdx.x) * (kThreads / kWave) + (threadIdx.x >> 6); wv * 512 < n; wv += waves) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int64_t base = wv * 512 + half * 256 + l * 4;   // I % 8 == 0: the four share a row
      if (base >= n) continue;
      const float sc = to_f32<EI>(s[base / I]);
      float v[4];
      if constexpr (sizeof(EI) == 2) {
        const uint2 q = *reinterpret_cast<const uint2*>(w0 + base);
        v[0] = sc * bf16_to_f32(uint16_t(q.x));
        v[1] = sc * bf16_to_f32(uint16_t(q.x >> 16));
        v[2] = sc * bf16_to_f32(uint16_t(q.y));
        v[3] = sc * bf16_to_f32(uint16_t(q.y >> 16));
      } else {
        const float4 q = *reinterpret_cast<const float4*>(w0 + base);
        v[0] = sc * q.x; v[1] = sc * q.y; v[2] = sc * q.z; v[3] = sc * q.w;
      }
      if constexpr (sizeof(EO) == 4) {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(out + base));
      } else {
        *reinterpret_cast<uint2*>(out + base) = make_uint2(f32_to_bf16(v[0]) | (uint32_t(f32_to_bf16(v[1])) << 16),
                                                           f32_to_bf16(v[2]) | (uint32_t(f32_to_bf16(v[3])) << 16));
      }
    }
  }
}

// 64 x 64 tiles (any element type and rank); wave w owns rows 16 w .. +15.
template <typename EI, typename EO>
__global__ __launch_bounds__(kThreads) void reconstruct_lowrank_kernel(const EI* __restrict__ s, const EI* __restrict__ w0,
                                                                       const EI* __restrict__ u, const EI* __restrict__ v,
                                                                       EO* __restrict__ out, int O, int I, int R) {
  const int l = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int i0 = blockIdx.x * rebuild::t64::BT, o0 = blockIdx.y * rebuild::t64::BT;
  f32x4 acc[4];
  rebuild::t64::product<EI>(u, v, O, I, R, o0, i0, acc);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int o = o0 + w * 16 + (l >> 4) * 4 + e;
    if (o >= O) continue;
    const float sc = to_f32<EI>(s[o]);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int i = i0 + ct * 16 + (l & 15);
      if (i < I) out[size_t(o) * I + i] = from_f32<EO>(acc[ct][e] + sc * to_f32<EI>(w0[size_t(o) * I + i]));
    }
  }
}

// ---- bf16 bundles, rank % 8 == 0 --------------------------------------------
namespace mm {

template <typename EO>
__device__ __forceinline__ void store4(EO* p, float a, float b, float c, float d) {
  if constexpr (sizeof(EO) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  } else {
    *reinterpret_cast<uint2*>(p) = make_uint2(f32_to_bf16(a) | (uint32_t(f32_to_bf16(b)) << 16),
                                              f32_to_bf16(c) | (uint32_t(f32_to_bf16(d)) << 16));
  }
}

// blockIdx.x: 128-column block of the output (rows of V); blockIdx.y: 128-row
// block (rows of U).
template <typename EO>
__global__ __launch_bounds__(kThreads, 2) void reconstruct_mfma_kernel(const bf16_t* __restrict__ s,
                                                                        const bf16_t* __restrict__ w0,
                                                                        const bf16_t* __restrict__ u,
                                                                        const bf16_t* __restrict__ v,
                                                                        EO* __restrict__ out, int O, int I, int R) {
  namespace t = rebuild::t128;
  __shared__ __attribute__((aligned(16))) unsigned char lds[t::kLdsBytes];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int i0 = blockIdx.x * t::BT, o0 = blockIdx.y * t::BT;
  const int wi = w & 1, wo = w >> 1, h = l >> 5, lr = l & 31;
  t::f32x16 acc[2][2];
  t::product(u, v, O, I, R, o0, i0, lds, acc);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int o = o0 + wo * 64 + cb * 32 + lr;
    if (o >= O) continue;
    const float so = bf16_to_f32(s[o].bits);
    const bf16_t* wrow = w0 + size_t(o) * I;
    EO* orow = out + size_t(o) * I;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int i = i0 + wi * 64 + rb * 32 + 8 * b + 4 * h;   // I % 8 == 0: i < I covers i .. i+3
        if (i >= I) continue;
        const uint2 wv = *reinterpret_cast<const uint2*>(wrow + i);
        const t::f32x16& c = acc[rb][cb];
        store4<EO>(orow + i, c[4 * b + 0] + so * bf16_to_f32(uint16_t(wv.x)),
                   c[4 * b + 1] + so * bf16_to_f32(uint16_t(wv.x >> 16)),
                   c[4 * b + 2] + so * bf16_to_f32(uint16_t(wv.y)),
                   c[4 * b + 3] + so * bf16_to_f32(uint16_t(wv.y >> 16)));
      }
  }
}

}  // namespace mm

// ---- bf16 bundles, 192 < rank <= 256: persistent, direct-to-LDS ----------------
//
// Two workgroups per compute unit walk their output tiles (128 x 128) in
// turn, so that one workgroup's matrix-core and LDS work overlaps the other's
// waits.  U and V come in k-tiles of 32 through a four-slot LDS ring (16 KB a
// slot) by direct-to-LDS buffer loads; each slot is refilled, three k-tiles
// ahead and across tile boundaries, as soon as every wave has read it.  The
// W0 and s values of the next tile are loaded into registers at the end of a
// tile's epilogue, ahead of its stores, and so have the whole next k-loop to
// arrive.  The epilogue moves
// each wave's 64 x 64 accumulators through LDS (the slot of the last k-tile
// for waves 0 and 1, a 16 KB staging area for waves 2 and 3) so that 16 lanes
// cover 64 consecutive outputs of one row: 128-byte W0 reads and 256-byte
// non-temporal fp32 writes per row.  80 KB of LDS per workgroup.
//
// Memory instructions complete in issue order, so the wait for a k-tile is a
// count of the loads and stores issued after it: every load and store here
// is issued unconditionally (lanes outside the matrix get an offset past the
// buffer: loads return zero, stores are dropped), tiles past a workgroup's
// last one are loaded as zeros, and the counts below are exact.
namespace rp {

constexpr int BT = 128, BK = 32, kSlots = 4;
constexpr int kOpBytes = BT * BK * 2;             // one operand's k-tile: 128 rows of 64 bytes
constexpr int kSlotBytes = 2 * kOpBytes;          // [U k-tile][V k-tile], 16 KB
constexpr int kRingBytes = kSlots * kSlotBytes;   // 64 KB
constexpr int kWaveStage = 8192;                  // one wave's epilogue rows: 32 x 64 fp32
constexpr int kLdsBytes = kRingBytes + 2 * kWaveStage;
constexpr int kStageRow = 256;
constexpr unsigned kRsrcFlags = 0x00020000u;  // buffer descriptor word 3: 32-bit data format
constexpr int kPast = int(0x80000000u);       // lane offset past every buffer
constexpr int kNT = 2;                        // non-temporal cache policy
static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per compute unit");

// k-tiles per output tile for a rank: ceil(rank / 32) rounded up to 2, 4 or 8
// (the k-tiles past the rank load zeros), which covers every rank up to 256.
inline int ktiles(int64_t R) {
  const int k = int((R + BK - 1) / BK);
  return k <= 2 ? 2 : k <= 4 ? 4 : 8;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds_byte;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

__device__ __forceinline__ lds_byte* opaque(lds_byte* p) {
  asm volatile("" : "+v"(p));
  return p;
}

// Buffer views of one output tile (uniform: scalar registers).
struct Tile {
  int o0, i0, orows, irows;
  __amdgpu_buffer_rsrc_t ru, rv, rw, rs, ro;
};

template <typename EO>
__device__ __forceinline__ Tile tile_at(int t, int tiles_i, const bf16_t* s, const bf16_t* w0, const bf16_t* u,
                                        const bf16_t* v, EO* out, int O, int I, int R) {
  Tile g;
  const int bo = t / tiles_i, bi = t - bo * tiles_i;
  g.o0 = bo * BT;
  g.i0 = bi * BT;
  g.orows = min(O - g.o0, BT);
  g.irows = min(I - g.i0, BT);
  g.ru = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(u + size_t(g.o0) * R), 0, g.orows * R * 2, kRsrcFlags);
  g.rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(v + size_t(g.i0) * R), 0, g.irows * R * 2, kRsrcFlags);
  g.rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(w0 + size_t(g.o0) * I), 0, g.orows * I * 2, kRsrcFlags);
  g.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(s + g.o0), 0, g.orows * 2, kRsrcFlags);
  g.ro = __builtin_amdgcn_make_buffer_rsrc(out + size_t(g.o0) * I, 0, g.orows * I * int(sizeof(EO)), kRsrcFlags);
  return g;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Two direct-to-LDS loads: load j writes 1 KB at dst + j KB (lane l at
// +16 l) from lane offset v[j] + soff.  The buffer's range check covers the
// lane offset only, so every lane offset carries its row and chunk (or lies
// past the buffer: the lane then writes zeros).  M0 takes one wait state
// before a load that reads it.
__device__ __forceinline__ void dma2(unsigned dst, __amdgpu_buffer_rsrc_t r, const int (&v)[2], int soff) {
  asm volatile(
      "s_mov_b32 m0, %[d0]\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[v0], %[r], %[so] offen lds\n\t"
      "s_mov_b32 m0, %[d1]\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[v1], %[r], %[so] offen lds"
      :
      : [d0] "s"(dst), [d1] "s"(dst + 1024u), [v0] "v"(v[0]), [v1] "v"(v[1]), [r] "s"(r), [so] "s"(soff)
      : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Per-lane constants of the direct-to-LDS loads.  A k-tile row is 64 bytes,
// four 16-byte chunks; chunk c of row r is stored at position
// c ^ ((r >> 2) & 3), so that the fragment reads of 16 consecutive rows (one
// chunk each) hit 16 distinct 16-byte bank groups.  Wave w fills rows
// 32 w + 16 j + l / 4 (j = 0, 1) of each operand's k-tile: lane l lands at
// position l % 4 of its row and fetches the global chunk that the swizzle
// stores there, (l % 4) ^ ((l >> 4) & 3) for both j.
struct Dma {
  unsigned dst;  // this wave's first KB of slot 0, U operand
  int row, c;    // row of load 0; global chunk
};

// k-tile kt of tile g into ring slot SLOT.  Rows past the tile's, chunks past
// the rank and every lane of a dummy tile (past the workgroup's last) write
// zeros.
template <int SLOT>
__device__ __forceinline__ void issue(const Dma& d, const Tile& g, int kt, bool dummy, int R) {
  const bool ok = !dummy && d.c * 8 < R - kt * BK;
  int vu[2], vv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = d.row + 16 * j, off = row * R * 2 + (d.c << 4);
    vu[j] = (ok && row < g.orows) ? off : kPast;
    vv[j] = (ok && row < g.irows) ? off : kPast;
  }
  dma2(d.dst + SLOT * kSlotBytes, g.ru, vu, kt * BK * 2);
  dma2(d.dst + SLOT * kSlotBytes + kOpBytes, g.rv, vv, kt * BK * 2);
}

// Epilogue layout: in round cb (0, 1) lane l of wave w handles output row
// 64 (w / 2) + 32 cb + 4 p + l / 16 (p = 0..7) and columns 64 (w % 2) + 4 (l % 16) .. +3
// of the tile.  The W0 values are held in that layout; of s, lane l holds
// row 64 (w / 2) + 32 cb + l % 32 and the epilogue fetches the row it needs
// from that lane.
struct Pre {
  u32x2 w[2][8];
  uint32_t s[2];
};

template <typename EO>
__device__ __forceinline__ int out_off(const Tile& g, int I, int wo, int wi, int cb, int p, int l) {
  const int orel = wo * 64 + cb * 32 + 4 * p + (l >> 4), i = g.i0 + wi * 64 + (l & 15) * 4;
  return (orel < g.orows && i < I) ? (orel * I + i) * int(sizeof(EO)) : kPast;
}

// 18 loads: 2 of s, 16 of W0.
__device__ __forceinline__ void prefetch(Pre& q, const Tile& g, bool dummy, int I, int wo, int wi, int l) {
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int srow = wo * 64 + cb * 32 + (l & 31);
    q.s[cb] = __builtin_amdgcn_raw_buffer_load_b16(g.rs, (!dummy && srow < g.orows) ? srow * 2 : kPast, 0, 0);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int orel = wo * 64 + cb * 32 + 4 * p + (l >> 4), i = g.i0 + wi * 64 + (l & 15) * 4;
      const bool ok = !dummy && orel < g.orows && i < I;
      q.w[cb][p] = __builtin_amdgcn_raw_buffer_load_b64(g.rw, ok ? (orel * I + i) * 2 : kPast, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // issue in order of use
    }
  }
}

// s of epilogue row 4 p + l / 16 of round cb, from the lane that holds it.
__device__ __forceinline__ float row_scale(const Pre& q, int cb, int p, int l) {
  return bf16_to_f32(uint16_t(__builtin_amdgcn_ds_bpermute((4 * p + (l >> 4)) << 2, int(q.s[cb]))));
}

// The four outputs of one epilogue position: product + s W0.
__device__ __forceinline__ f32x4 add_scaled(f32x4 c, u32x2 wv, float so) {
  return f32x4{c[0] + so * bf16_to_f32(uint16_t(wv[0])), c[1] + so * bf16_to_f32(uint16_t(wv[0] >> 16)),
               c[2] + so * bf16_to_f32(uint16_t(wv[1])), c[3] + so * bf16_to_f32(uint16_t(wv[1] >> 16))};
}

// Measuring the error against an fp32 original: the original's values of
// epilogue round cb, loaded as the round starts (the registers of a whole
// tile ahead would not fit two workgroups per compute unit).
__device__ __forceinline__ void load_orig(u32x4 (&o)[8], const Tile& g, int cb, int I, int wo, int wi, int l) {
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int orel = wo * 64 + cb * 32 + 4 * p + (l >> 4), i = g.i0 + wi * 64 + (l & 15) * 4;
    const bool ok = orel < g.orows && i < I;
    o[p] = __builtin_amdgcn_raw_buffer_load_b128(g.ro, ok ? (orel * I + i) * 4 : kPast, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ __forceinline__ f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                 0);
}

// Fragments of k16 steps 0, 1 of the k-tile in ring slot SLOT (A from V rows
// 64 wi + 32 rb + lane % 32, B from U rows 64 wo + 32 cb + lane % 32, chunk
// ks * 2 + lane / 32, swizzled), then the 8 products.
template <int SLOT>
__device__ __forceinline__ void multiply_step(lds_byte* const (&rdU)[2], lds_byte* const (&rdV)[2],
                                              f32x16 (&acc)[2][2]) {
  constexpr int off = SLOT * kSlotBytes;
  u32x4 fa[2][2], fb[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      fa[r][ks] = *reinterpret_cast<const lds_u32x4*>(rdV[ks] + off + kOpBytes + r * 32 * 64);
      fb[r][ks] = *reinterpret_cast<const lds_u32x4*>(rdU[ks] + off + r * 32 * 64);
    }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mma32(fa[rb][ks], fb[cb][ks], acc[rb][cb]);
  __builtin_amdgcn_sched_barrier(0);
  mfma_operand_guard();
  __builtin_amdgcn_sched_barrier(0);
}

// Four outputs in the stored form: fp32, or bf16 pairs packed into words.
template <typename EO> struct Packed { typedef u32x4 type; };
template <> struct Packed<bf16_t> { typedef u32x2 type; };

template <typename EO>
__device__ __forceinline__ typename Packed<EO>::type pack_out(f32x4 r) {
  if constexpr (sizeof(EO) == 4) {
    return u32x4{__float_as_uint(r[0]), __float_as_uint(r[1]), __float_as_uint(r[2]), __float_as_uint(r[3])};
  } else {
    return u32x2{f32_to_bf16(r[0]) | (uint32_t(f32_to_bf16(r[1])) << 16),
                 f32_to_bf16(r[2]) | (uint32_t(f32_to_bf16(r[3])) << 16)};
  }
}

template <typename EO>
__device__ __forceinline__ void store_out(const Tile& g, int off, typename Packed<EO>::type v) {
  if constexpr (sizeof(EO) == 4) __builtin_amdgcn_raw_buffer_store_b128(v, g.ro, off, 0, kNT);
  else __builtin_amdgcn_raw_buffer_store_b64(v, g.ro, off, 0, kNT);
}

// The k-tiles of all of a workgroup's output tiles form one stream: k-tile
// k of its n-th tile is stream entry j = n KT + k (KT k-tiles per tile) and
// lives in ring slot j % 4.  Step j waits for entry j, publishes it to every
// wave, refills the slot every wave has just finished with (entry j + 3)
// and multiplies.  After a tile's last step its epilogue goes through the
// slot that step read (kErr: with 8 loads of the original in each of its two
// rounds) and forms the tile's outputs in registers; then it issues the W0
// and s loads of the next tile (18) and only then the 16 stores (none when
// kErr).  Memory instructions complete in issue order, so a wait for the
// next tile's W0 does not wait for this tile's non-temporal stores to leave.
// Every load and store is issued unconditionally, so the count of memory
// instructions issued after entry j when step j waits is a constant: the
// refills of the two steps between (4 each) plus 34 for each tile end among
// the three steps before j.  vmcnt counts up to 63, so 63 stands for any
// larger count.  (The prologue waits for all of its loads, so entries 0..2
// have landed.)
template <int KT>
__host__ __device__ constexpr int step_wait(int k) {
  int ends = 0;
  for (int r = k - 3; r < k; ++r)
    if ((((r + 1) % KT) + KT) % KT == 0) ++ends;
  const int n = 8 + 34 * ends;
  return n < 63 ? n : 63;
}
static_assert(step_wait<8>(0) == 42 && step_wait<8>(3) == 8 && step_wait<8>(7) == 8, "eight k-tiles per tile");
static_assert(step_wait<4>(0) == 42 && step_wait<4>(3) == 8, "four k-tiles per tile");
static_assert(step_wait<2>(1) == 42 && step_wait<2>(0) == 63, "two tile ends among three steps");

template <int V> struct IC { static constexpr int value = V; };

// Output tile number t (of this workgroup's sequence, stream entries from
// J0 mod 4 on); tile(t') gives the views of a later tile.
template <typename EO, bool kErr, int KT, int J0, typename TileFn>
__device__ __forceinline__ void tile_pass(const Dma& d, lds_byte* const (&rdU)[2], lds_byte* const (&rdV)[2],
                                          lds_byte* base, const TileFn& tile, int t, int G, int tiles, Pre& q,
                                          int I, int R, int wo, int wi, int l, double& num, double& den) {
  const int lr = l & 31, h = l >> 5, w = wo * 2 + wi;
  const Tile g = tile(t);
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  auto step = [&](auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr int dn = (k + 3) / KT, kk = (k + 3) % KT;   // entry j + 3: tile t + dn G, k-tile kk
    wait_vm<step_wait<KT>(k)>();
    __syncthreads();
    issue<(J0 + k + 3) % kSlots>(d, tile(t + dn * G), kk, t + dn * G >= tiles, R);
    multiply_step<(J0 + k) % kSlots>(rdU, rdV, acc);
  };
  step(IC<0>{});
  if constexpr (KT > 1) step(IC<1>{});
  if constexpr (KT > 2) { step(IC<2>{}); step(IC<3>{}); }
  if constexpr (KT > 4) { step(IC<4>{}); step(IC<5>{}); step(IC<6>{}); step(IC<7>{}); }

  lds_byte* stage = w < 2 ? base + ((J0 + KT - 1) % kSlots) * kSlotBytes + w * kWaveStage
                          : base + kRingBytes + (w - 2) * kWaveStage;
  typename Packed<EO>::type res[2][8];  // the rebuilt tile in the epilogue layout (kErr: unused)
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    u32x4 o[8];
    if constexpr (kErr) load_orig(o, g, cb, I, wo, wi, l);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int chunk = (8 * rb + 2 * b + h) ^ (lr & 15);
        const f32x16& c = acc[rb][cb];
        *reinterpret_cast<lds_f32x4*>(stage + lr * kStageRow + (chunk << 4)) =
            f32x4{c[4 * b], c[4 * b + 1], c[4 * b + 2], c[4 * b + 3]};
      }
    __syncthreads();
    f32x4 c[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int orel = 4 * p + (l >> 4), chunk = (l & 15) ^ (orel & 15);
      c[p] = *reinterpret_cast<const lds_f32x4*>(stage + orel * kStageRow + (chunk << 4));
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      // Entries outside the matrix: the original, W0 and s read as zero and the product is zero.
      const f32x4 wr = add_scaled(c[p], q.w[cb][p], row_scale(q, cb, p, l));
      if constexpr (kErr) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double ov = double(__uint_as_float(o[p][e])), dd = ov - double(wr[e]);
          num += dd * dd;
          den += ov * ov;
        }
      } else {
        res[cb][p] = pack_out<EO>(wr);
      }
    }
  }
  prefetch(q, tile(t + G), t + G >= tiles, I, wo, wi, l);
  if constexpr (!kErr) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int p = 0; p < 8; ++p) store_out<EO>(g, out_off<EO>(g, I, wo, wi, cb, p, l), res[cb][p]);
  }
}

// kErr = false: out receives the rebuilt weight.  kErr = true: out is the
// fp32 original (read only) and the relative error goes to *result through
// the grid-wide sum of tb_reduce.h (partial, counters).  KT = ktiles(rank).
template <typename EO, bool kErr, int KT>
__global__ __launch_bounds__(kThreads, 2) void reconstruct_persistent_kernel(const bf16_t* __restrict__ s,
                                                                             const bf16_t* __restrict__ w0,
                                                                             const bf16_t* __restrict__ u,
                                                                             const bf16_t* __restrict__ v,
                                                                             EO* __restrict__ out, int O, int I,
                                                                             int R, int tiles_i, int tiles,
                                                                             uint64_t* partial, unsigned* counters,
                                                                             double* result) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kLdsBytes];
  double num = 0.0, den = 0.0;
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6), l = int(threadIdx.x) & 63;
  const int wi = w & 1, wo = w >> 1, lr = l & 31, h = l >> 5;
  const int G = int(gridDim.x);
  int t = int(blockIdx.x);
  if (t >= tiles) return;

  lds_byte* base = (lds_byte*)ring;
  Dma d;
  d.row = w * 32 + (l >> 2);
  d.c = (l & 3) ^ ((l >> 4) & 3);
  d.dst = __builtin_amdgcn_readfirstlane(unsigned(uintptr_t(base)) + unsigned(w) * 2048u);
  // Fragment bases per k16 step: U row 64 wo + lane % 32, V row 64 wi + lane % 32
  // (the V operand sits kOpBytes into each slot).
  lds_byte* rdU[2];
  lds_byte* rdV[2];
  {
    const int x = (lr >> 2) & 3;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk = ((2 * ks + h) ^ x) << 4;
      rdU[ks] = opaque(base + (wo * 64 + lr) * 64 + chunk);
      rdV[ks] = opaque(base + (wi * 64 + lr) * 64 + chunk);
    }
  }

  // Tiles past the workgroup's last are dummies: their loads return zeros
  // into free slots and registers, and nothing of them is stored.
  const auto tile = [&](int tt) { return tile_at<EO>(tt < tiles ? tt : t, tiles_i, s, w0, u, v, out, O, I, R); };
  Pre q;  // W0 and s of the current tile
  // Stream entries 0..2 and the first tile's W0 and s, all landed before the
  // first step.
  issue<0>(d, tile(t), 0, false, R);
  issue<1>(d, tile(t + (1 / KT) * G), 1 % KT, t + (1 / KT) * G >= tiles, R);
  issue<2>(d, tile(t + (2 / KT) * G), 2 % KT, t + (2 / KT) * G >= tiles, R);
  prefetch(q, tile(t), false, I, wo, wi, l);
  wait_vm<0>();
  // One tile per round when KT is a multiple of 4, two when it is 2, so that
  // every slot index is a constant.
  for (;;) {
    tile_pass<EO, kErr, KT, 0>(d, rdU, rdV, base, tile, t, G, tiles, q, I, R, wo, wi, l, num, den);
    if ((t += G) >= tiles) break;
    if constexpr (KT % 4 != 0) {
      tile_pass<EO, kErr, KT, KT % 4>(d, rdU, rdV, base, tile, t, G, tiles, q, I, R, wo, wi, l, num, den);
      if ((t += G) >= tiles) break;
    }
  }
  wait_vm<0>();  // no load into LDS may still be in flight when the workgroup ends
  if constexpr (kErr) {
    __syncthreads();  // the ring is free: its first 4 KB hold the reduction, then the arrival verdict
    double* sa = reinterpret_cast<double*>(ring);
    double* sb = sa + kThreads;
    reduce::block_reduce2<kThreads>(num, den, sa, sb);
    reduce::finish_ratio<kThreads>(num, den, partial, counters, result, sa, sb, *reinterpret_cast<unsigned*>(sb + kThreads));
  }
}

template <typename EO, bool kErr>
hipError_t launch(const void* s, const void* w0, const void* u, const void* v, EO* out, int64_t O, int64_t I,
                  int64_t R, int grid, int tiles_i, int tiles, uint64_t* partial, unsigned* counters, double* result,
                  hipStream_t stream) {
#define TB_RP_LAUNCH(K)                                                                                              \
  hipLaunchKernelGGL((reconstruct_persistent_kernel<EO, kErr, K>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, \
                     static_cast<const bf16_t*>(s), static_cast<const bf16_t*>(w0), static_cast<const bf16_t*>(u),  \
                     static_cast<const bf16_t*>(v), out, int(O), int(I), int(R), tiles_i, tiles, partial, counters, \
                     result)
  // The error variant takes at least four k-tiles: its two-k-tile form,
  // two tiles per loop round, would spill.
  const int kt = ktiles(R) < 4 && kErr ? 4 : ktiles(R);
  switch (kt) {
    case 2: if constexpr (!kErr) TB_RP_LAUNCH(2); break;
    case 4: TB_RP_LAUNCH(4); break;
    default: TB_RP_LAUNCH(8); break;
  }
#undef TB_RP_LAUNCH
  return hipGetLastError();
}

}  // namespace rp

// The persistent kernel: bf16 bundles, 0 < rank <= 256 with rank % 8 == 0,
// and 32-bit lane offsets within a 128-row band of the output.
bool persistent_supported(int64_t O, int64_t I, int64_t R) {
  return R > 0 && R % 8 == 0 && R <= 8 * rp::BK && I < (1 << 22) && O < (1 << 24);
}

template <typename EI, typename EO>
hipError_t launch_typed(const void* s, const void* w0, const void* u, const void* v, void* w_out, int64_t O, int64_t I,
                        int64_t R, hipStream_t stream) {
  if (R == 0) {
    const int64_t n = O * I;
    int64_t blocks = (n + 512 * (kThreads / kWave) - 1) / (512 * (kThreads / kWave));
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL((reconstruct_rank0_kernel<EI, EO>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       static_cast<const EI*>(s), static_cast<const EI*>(w0), static_cast<EO*>(w_out), n, int(I));
  } else if (sizeof(EI) == 2 && persistent_supported(O, I, R)) {
    int cus = 0;
    if (int e = device_cu_count(&cus)) return hipError_t(e);
    const int tiles_i = int((I + rp::BT - 1) / rp::BT), tiles = tiles_i * int((O + rp::BT - 1) / rp::BT);
    return rp::launch<EO, false>(s, w0, u, v, static_cast<EO*>(w_out), O, I, R, tiles < 2 * cus ? tiles : 2 * cus, tiles_i,
                                 tiles, nullptr, nullptr, nullptr, stream);
  } else if (sizeof(EI) == 2 && R % 8 == 0 && (O + rebuild::t128::BT - 1) / rebuild::t128::BT <= 65535) {
    dim3 grid(unsigned((I + rebuild::t128::BT - 1) / rebuild::t128::BT), unsigned((O + rebuild::t128::BT - 1) / rebuild::t128::BT));
    hipLaunchKernelGGL((mm::reconstruct_mfma_kernel<EO>), grid, dim3(kThreads), 0, stream,
                       static_cast<const bf16_t*>(s), static_cast<const bf16_t*>(w0), static_cast<const bf16_t*>(u),
                       static_cast<const bf16_t*>(v), static_cast<EO*>(w_out), int(O), int(I), int(R));
  } else {
    dim3 grid(unsigned((I + 63) / 64), unsigned((O + 63) / 64));
    hipLaunchKernelGGL((reconstruct_lowrank_kernel<EI, EO>), grid, dim3(kThreads), 0, stream, static_cast<const EI*>(s),
                       static_cast<const EI*>(w0), static_cast<const EI*>(u), static_cast<const EI*>(v),
                       static_cast<EO*>(w_out), int(O), int(I), int(R));
  }
  return hipGetLastError();
}

}  // namespace

bool persistent_error_supported(int64_t out_dim, int64_t in_dim, int64_t rank) {
  return persistent_supported(out_dim, in_dim, rank);
}

hipError_t launch_reconstruction_error_persistent(const void* s, const void* w0, const void* u, const void* v,
                                                  const float* orig, int64_t O, int64_t I, int64_t R, double* result,
                                                  void* workspace, int cus, hipStream_t stream) {
  const int tiles_i = int((I + rp::BT - 1) / rp::BT), tiles = tiles_i * int((O + rp::BT - 1) / rp::BT);
  int grid = tiles < 2 * cus ? tiles : 2 * cus;
  if (grid > reduce::kMaxPartials) grid = reduce::kMaxPartials;
  return rp::launch<float, true>(s, w0, u, v, const_cast<float*>(orig), O, I, R, grid, tiles_i, tiles,
                                 reduce::partials(workspace), reduce::counters(workspace), result, stream);
}

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
