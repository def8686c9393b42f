// Theta-bundle projection for few tokens (m <= 64): one launch.
//
//   y = s (.) (x . W0^T) + (x . V) . U^T        ("The theta bundle": the
//   transpose of weight = diag(s) W0 + U V^T applied to x)
//
// At these token counts the projection is bound by HBM bandwidth: every byte
// of W0 is read once, and U, V, s once.  The grid holds two kinds of
// workgroup, the producers first, so that on every XCD the hardware dispatches
// them ahead of any streaming workgroup; producers never wait, so the
// streamers' waits on them always end.
//
//   producers (rank > 0): T = x . V.  Producer (kt, cb) owns the 64 columns
//     [64cb, 64cb+64) of T over the k-slice kt of in_dim: no exchange with
//     other producers until the end.  Its waves take k32 steps round-robin,
//     each loading a 32 x 64 block of V in whole 128-byte row segments
//     (transposed through a wave-private LDS tile) and the
//     x fragments, and multiply on the matrix cores; the eight partials are
//     summed in LDS in a fixed order.  With several k-slices each producer
//     stores its fp32 partial and the last of the column block to arrive sums
//     them in k-slice order; the final block is published as T [16*NT][Rp] in
//     the operand type and counted in a done word.
//   streamers: the output rows are cut into NRB balanced row blocks of at
//     most 16*TILES rows and in_dim into KS k-slices; streamer (rb, ks) owns
//     one pair.  Each of its eight waves takes k32 steps round-robin and keeps
//     D steps of W0 fragments (A operand, 16 rows x 32 k per tile, straight
//     from HBM into registers) and x fragments (B operand, 16 tokens, served
//     by the L2) in flight: one continuous software pipeline per wave with no
//     workgroup barrier.  Afterwards each wave scales its rows by s (fetched
//     at the start); the streamer of the last k-slice also adds its waves'
//     k32 steps of T . U^T once every column block of T is published (U
//     fetched before the stream).  The eight partials are summed in LDS in a
//     fixed order.
//     With one k-slice the result is stored rounded once; otherwise each
//     streamer stores its fp32 partial, and the last of the row block to
//     arrive sums the KS partials in k-slice order and stores y.
//
// Data crossing workgroups (T partials, y partials, counters) moves only
// through device-scope (sc1) 32-bit accesses, coherent across XCDs without
// writing back or invalidating any L2; a writer drains its stores before it
// counts itself in.  Every wait is bounded: a timeout sets the sticky error
// word and poisons the affected y with NaN.
#include "tb_device.h"
#include "tb_host.h"

namespace tb {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;

// Control words: [kErr] sticky timeout flag, [kDone] column blocks of T
// published; from word kCbCounters on, one arrival counter per column block
// of T (k-sliced producers), from kRbCounters on one per row block (k-sliced
// streamers); from kFinishBase on, the rank streamers past their read of T,
// counted into kFinishGroups group counters (64 words apart) and a top
// counter bumped by the last of each group, so that a few hundred increments
// do not queue on one word.
enum Ctrl { kErr = 2, kParity = 3, kDone = 5 };
constexpr int kFinishBase = int(kCtrlBlockBytes / 4) - kFinishWords;
constexpr int kFinishGroups = 16;
constexpr int kCbCounters = 64;
constexpr int kRbCounters = kCbCounters + kMaxGroupCounters / 2;

struct DecodeArgs {
  const void* x;
  const void* s;
  const void* w0;
  const void* u;
  const void* v;
  void* y;
  int M, O, I, R;
  int NCB, KT;       // producers: NCB column blocks x KT k-slices
  int NRB, KS, RBR;  // streamers: NRB row blocks x KS k-slices; RBR rows per block at most
  unsigned* ctrl;
  unsigned* err;  // sticky timeout word (word kErr of the first projection's control region)
  int polls;      // bound of the streamers' wait for T, in polls
  float* tpart;  // [KT][16*NT][Rp] fp32 partials (KT > 1)
  void* tfull;   // [16*NT][Rp] T in the operand type
  float* ypart;  // [NRB][KS][16*NT][RBR] fp32 (KS > 1)
};

// The x . V exchange in the control block (when it fits): T [16*NT][Rp] in
// the operand type, packed into 32-bit words (two bf16 or one fp32) and stored
// complemented.  A NaN is stored as the canonical quiet NaN, so no payload is
// all ones and no stored word is zero: a zero word is one not written yet.
// Producers store their columns once; each rank-streamer wave polls just the
// words it multiplies, so T needs no separate done count, no drain before it
// and no extra round trip to learn that it is complete.  A launch exchanges T
// in the half of the exchange words that its control block's parity word
// names; its producers clear the other half once they are done, and the last
// rank streamer flips the parity, so the next launch finds a cleared half and
// no launch spends time clearing on its critical path.  Every workgroup reads
// the parity before it counts itself in anywhere, so none can see the flip.
__device__ __forceinline__ uint16_t t_bf16(float v) { return v != v ? uint16_t(0x7FC0u) : f32_to_bf16(v); }
__device__ __forceinline__ uint32_t t_f32(float v) { return v != v ? 0x7FC00000u : __float_as_uint(v); }
template <typename E> __host__ __device__ constexpr int t_words(int NT, int Rp) {
  return 16 * NT * Rp * int(sizeof(E)) / 4;
}

// Device-scope (sc1) 32-bit accesses: coherent across XCDs without touching
// the rest of the L2.
__device__ __forceinline__ uint32_t load_coherent(const void* p) {
  return __hip_atomic_load(static_cast<const uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(void* p, uint32_t v) {
  __hip_atomic_store(static_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned add_coherent(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait (relaxed polling, no cache invalidation): at most `polls`
// polls (about 0.1 us apart).
__device__ __forceinline__ bool wait_for_count(const unsigned* counter, unsigned target, int polls) {
  for (int it = 0; it < polls; ++it) {
    if (load_coherent(counter) >= target) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// Wait until this wave's outstanding memory operations have completed: its
// device-scope stores are then visible to every XCD.
__device__ __forceinline__ void drain_stores() { __builtin_amdgcn_s_waitcnt(0); }

template <typename E> constexpr int frag_vgprs() { return sizeof(E) == 2 ? 4 : 8; }

// Eight elements k..k+7 of one row of a [rows][R] matrix (zero past R).
template <typename E>
__device__ __forceinline__ Frag8<E> load_row8(const E* row, int k, int R, bool aligned) {
  if (k >= R) return zero_frag<E>();
  return aligned ? load_frag<E>(row + k) : load_frag_partial<E>(row + k, min(8, R - k));
}

// ---------------------------------------------------------------------------
// Producers.
// ---------------------------------------------------------------------------
constexpr int kVtPitch = 40;  // elements per column of a wave's transposed 64 x 32 V tile (fp32 V)
constexpr int kVsPitch = 160; // bytes per row of a wave's staged 32 x 64 V tile (bf16 V): 5 KB, as the above
static_assert(32 * kVsPitch <= 64 * kVtPitch * 2, "staged tile fits the wave's LDS share");
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4v lds_u32x4;
constexpr int kMaxKT = 16;    // k-slices of the producers at most
constexpr int kCbCols = 64;   // columns of T per producer: 128 contiguous bytes of a bf16 row of V

// k32 steps in flight per producer wave (registers: 4 V pieces and NT x
// fragments per step).
template <typename E, int NT> constexpr int producer_depth() {
  return sizeof(E) == 2 ? (NT == 1 ? 3 : (NT == 2 ? 2 : 1)) : 1;
}

template <typename E, int NT>
constexpr int producer_smem() {
  using Raw = typename std::conditional<sizeof(E) == 2, uint16_t, float>::type;
  constexpr int tiles = kWaves * kCbCols * kVtPitch * int(sizeof(Raw));
  constexpr int reduce = kWaves * NT * kWave * 16 + 16 * NT * kCbCols * 4;
  return tiles > reduce ? tiles : reduce;
}

// TCTRL: T goes out as the control block's coded words; else into tfull,
// counted in kDone.
template <typename E, int NT, bool TCTRL>
__device__ void produce_t(const DecodeArgs& a, int p, uint8_t* smem) {
  using Raw = typename std::conditional<sizeof(E) == 2, uint16_t, float>::type;
  constexpr int D = producer_depth<E, NT>();
  const E* X = static_cast<const E*>(a.x);
  const E* V = static_cast<const E*>(a.v);
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), l = tid % kWave;
  const int lr = l & 15, q4 = l >> 4, kq = q4 * 8;
  const int M = a.M, I = a.I, R = a.R;
  const int cb = p % a.NCB, kt = p / a.NCB;
  const int S = (I + 31) / 32;
  const int s0 = int(int64_t(kt) * S / a.KT), s1 = int(int64_t(kt + 1) * S / a.KT);
  const int n = s1 - s0 > w ? (s1 - s0 - w + kWaves - 1) / kWaves : 0;
  const bool valigned = (R % 8) == 0;
  // A step's 32 x 64 block of V is four loads per lane: load q covers rows
  // 8q .. 8q+7 with lane l taking row 8q + l/8, columns 8*(l%8) .. +7, so
  // each load reads whole 128-byte row segments.
  const int vr = l >> 3, vc = cb * kCbCols + (l & 7) * 8;
  Raw* vt = reinterpret_cast<Raw*>(smem) + w * (kCbCols * kVtPitch);  // [64 cols][kVtPitch], this wave's
  // The sticky error word as this launch found it (thread 0's copy decides,
  // after the k-loop): a workspace left by a timed-out wait may hold stale
  // counts, so a poisoned launch publishes nothing and counts nothing.
  const uint32_t err_at_entry = load_coherent(a.err);
  const uint32_t parity = TCTRL ? load_coherent(&a.ctrl[kParity]) & 1u : 0u;
  __shared__ unsigned s_poisoned_p;

  f32x4 acc[4][NT];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[j][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (n > 0) {
    Frag8<E> vf[D][4], xf[D][NT];
    auto issue = [&](Frag8<E> (&fv)[4], Frag8<E> (&fx)[NT], int i) {
      const int k0 = (s0 + w + i * kWaves) * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = k0 + 8 * q + vr;
        fv[q] = row < I ? load_row8<E>(V + size_t(row) * R, vc, R, valigned) : zero_frag<E>();
      }
      const bool kv = k0 + kq < I;
#pragma unroll
      for (int c = 0; c < NT; ++c)
        fx[c] = load_frag_if<E>(X + size_t(min(c * 16 + lr, M - 1)) * I + (kv ? k0 + kq : 0), kv);
    };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(vf[d], xf[d], min(d, n - 1));
    for (int i0 = 0; i0 < n; i0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (i0 + d < n) {
          Frag8<E> fb[4];
          if constexpr (sizeof(E) == 2) {
            // Stage the block as it sits in memory (32 rows of k, 160-byte
            // pitch) and read each lane's eight consecutive k of one column
            // with the transposing LDS read: within 16 lanes, lane i receives
            // element i % 4 of the 8-byte chunks addressed by lanes 4e + i / 4,
            // so lanes pointing at rows kb + (lane % 16) / 4, columns
            // nb + 4 (lane % 4) receive k = kb .. kb+3 of column nb + lane % 16.
            // The pitch puts the four rows of one read on distinct banks.
            lds_u8* st = (lds_u8*)vt;  // vt lies in LDS
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<lds_u32x4*>(st + (8 * q + vr) * kVsPitch + (l & 7) * 16) =
                  u32x4v{vf[d][q].v.x, vf[d][q].v.y, vf[d][q].v.z, vf[d][q].v.w};
            __builtin_amdgcn_wave_barrier();
            const int rr = 8 * (l >> 4) + ((l & 15) >> 2), cc = 4 * (l & 3);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              lds_u8* pr = st + rr * kVsPitch + (16 * j + cc) * 2;
              const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>(pr));
              const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>(pr + 4 * kVsPitch));
              fb[j].v = make_uint4(uint32_t(uint16_t(lo[0])) | (uint32_t(uint16_t(lo[1])) << 16),
                                   uint32_t(uint16_t(lo[2])) | (uint32_t(uint16_t(lo[3])) << 16),
                                   uint32_t(uint16_t(hi[0])) | (uint32_t(uint16_t(hi[1])) << 16),
                                   uint32_t(uint16_t(hi[2])) | (uint32_t(uint16_t(hi[3])) << 16));
            }
          } else {
            // Transpose the block through the wave's LDS tile: column j holds
            // k = 0..31 contiguously.
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              Raw vals[8];
              __builtin_memcpy(vals, &vf[d][q], sizeof(vals));
#pragma unroll
              for (int e = 0; e < 8; ++e) vt[((l & 7) * 8 + e) * kVtPitch + 8 * q + vr] = vals[e];
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int j = 0; j < 4; ++j)
              fb[j] = load_frag<E>(reinterpret_cast<const E*>(&vt[(16 * j + lr) * kVtPitch + kq]));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < NT; ++c) acc[j][c] = mma_k32(xf[d][c], fb[j], acc[j][c]);
          __builtin_amdgcn_sched_barrier(0);
          mfma_operand_guard();
          __builtin_amdgcn_sched_barrier(0);
          issue(vf[d], xf[d], min(i0 + d + D, n - 1));
        }
      }
    }
  }

  // Sum the eight waves' tiles in a fixed order, one 16-column tile at a
  // time; C holds tokens 4*(l/16)+e of token tile c, column lr of the tile.
  // The block's result goes to LDS as [16*NT tokens][64 columns].
  f32x4* red = reinterpret_cast<f32x4*>(smem);  // [kWaves][NT][kWave]
  float* blk = reinterpret_cast<float*>(smem + kWaves * NT * kWave * 16);
  if (tid == 0) s_poisoned_p = err_at_entry;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    __syncthreads();  // the V tiles, or the previous tile's sums, are done with
#pragma unroll
    for (int c = 0; c < NT; ++c) red[(w * NT + c) * kWave + l] = acc[j][c];
    __syncthreads();
    if (w < NT) {
      f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < kWaves; ++v) sum += red[(v * NT + w) * kWave + l];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = w * 16 + q4 * 4 + e;
        blk[tok * kCbCols + 16 * j + lr] = tok < M ? sum[e] : 0.f;
      }
    }
  }
  __syncthreads();

  // With one k-slice the block is final.  Otherwise store this slice's
  // partial; the last producer of the column block to arrive sums the KT
  // partials in k-slice order.  Either way the final block is published in
  // the operand type, two columns per 32-bit word: as coded words in the
  // control block (TCTRL), else in tfull and counted in kDone.
  const int Rp = a.NCB * kCbCols;
  const int col0 = cb * kCbCols;
  if (s_poisoned_p != 0u) return;
  __shared__ unsigned s_last;
  bool last = true;
  if (a.KT > 1) {
    float* tp = a.tpart + size_t(kt) * (16 * NT) * Rp + col0;
    for (int i = tid; i < 16 * NT * kCbCols; i += kThreads)
      store_coherent(&tp[(i / kCbCols) * Rp + i % kCbCols], __float_as_uint(blk[i]));
    drain_stores();
    __syncthreads();
    if (tid == 0) s_last = add_coherent(&a.ctrl[kCbCounters + cb], 1u) == unsigned(a.KT - 1);
    __syncthreads();
    last = s_last;
  }
  // Share of the other exchange half that this producer clears when done.
  const auto clear_other_half = [&] {
    uint32_t* other = a.ctrl + kTWordBase + (1u - parity) * kTHalfWords;
    const int np = a.NCB * a.KT, per = (kTHalfWords + np - 1) / np;
    for (int i = p * per + tid; i < min(kTHalfWords, (p + 1) * per); i += kThreads) store_coherent(&other[i], 0u);
  };
  if (!last) {
    if constexpr (TCTRL) clear_other_half();
    return;
  }
  for (int i = tid; i < 16 * NT * kCbCols / 2; i += kThreads) {  // word i: token i/32, columns 2*(i%32) and +1
    const int tok = i / (kCbCols / 2), col = 2 * (i % (kCbCols / 2));
    float v0 = 0.f, v1 = 0.f;
    if (a.KT > 1) {
      // All partials are fetched at once (one round trip), then summed in
      // k-slice order.
      float p0[kMaxKT], p1[kMaxKT];
#pragma unroll
      for (int k = 0; k < kMaxKT; ++k) {
        const float* src = a.tpart + (size_t(k) * (16 * NT) + tok) * Rp + col0 + col;
        const bool other = k < a.KT && k != kt;
        p0[k] = other ? __uint_as_float(load_coherent(src)) : blk[tok * kCbCols + col];
        p1[k] = other ? __uint_as_float(load_coherent(src + 1)) : blk[tok * kCbCols + col + 1];
      }
#pragma unroll
      for (int k = 0; k < kMaxKT; ++k)
        if (k < a.KT) {
          v0 += p0[k];
          v1 += p1[k];
        }
    } else {
      v0 = blk[tok * kCbCols + col];
      v1 = blk[tok * kCbCols + col + 1];
    }
    if constexpr (TCTRL) {
      uint32_t* tw = a.ctrl + kTWordBase + parity * kTHalfWords;
      if constexpr (sizeof(E) == 2) {
        store_coherent(&tw[(tok * Rp + col0 + col) / 2], ~(uint32_t(t_bf16(v0)) | (uint32_t(t_bf16(v1)) << 16)));
      } else {
        store_coherent(&tw[tok * Rp + col0 + col], ~t_f32(v0));
        store_coherent(&tw[tok * Rp + col0 + col + 1], ~t_f32(v1));
      }
    } else if constexpr (sizeof(E) == 2) {
      uint32_t* tf = static_cast<uint32_t*>(a.tfull);
      store_coherent(&tf[(size_t(tok) * Rp + col0 + col) / 2], uint32_t(f32_to_bf16(v0)) | (uint32_t(f32_to_bf16(v1)) << 16));
    } else {
      float* tf = static_cast<float*>(a.tfull);
      store_coherent(&tf[size_t(tok) * Rp + col0 + col], __float_as_uint(v0));
      store_coherent(&tf[size_t(tok) * Rp + col0 + col + 1], __float_as_uint(v1));
    }
  }
  if constexpr (TCTRL) {
    // The coded words need no count: the arrival counter is cleared for the
    // next launch, then this producer's share of the other half.
    if (tid == 0 && a.KT > 1) store_coherent(&a.ctrl[kCbCounters + cb], 0u);
    clear_other_half();
    return;
  }
  drain_stores();
  __syncthreads();
  if (tid == 0) {
    if (a.KT > 1) store_coherent(&a.ctrl[kCbCounters + cb], 0u);
    add_coherent(&a.ctrl[kDone], 1u);
  }
}

// ---------------------------------------------------------------------------
// Streamers.
// ---------------------------------------------------------------------------
// k32 steps in flight per wave: D steps of TILES W0 fragments and NT x
// fragments take at most 64 VGPRs.
template <typename E, int NT, int TILES> constexpr int pipe_depth() {
  return 64 / ((TILES + NT) * frag_vgprs<E>()) > 0 ? 64 / ((TILES + NT) * frag_vgprs<E>()) : 1;
}

// T for token row `tok`, columns k..k+7 (published by the producers of this
// launch): device-scope 32-bit loads.
template <typename E>
__device__ __forceinline__ Frag8<E> load_t(const DecodeArgs& a, int tok, int k) {
  const uint32_t* q = static_cast<const uint32_t*>(a.tfull) + (size_t(tok) * (a.NCB * kCbCols) + k) * sizeof(E) / 4;
  Frag8<E> f;
  if constexpr (sizeof(E) == 2) {
    f.v = make_uint4(load_coherent(q), load_coherent(q + 1), load_coherent(q + 2), load_coherent(q + 3));
  } else {
    f.lo = make_float4(__uint_as_float(load_coherent(q)), __uint_as_float(load_coherent(q + 1)),
                       __uint_as_float(load_coherent(q + 2)), __uint_as_float(load_coherent(q + 3)));
    f.hi = make_float4(__uint_as_float(load_coherent(q + 4)), __uint_as_float(load_coherent(q + 5)),
                       __uint_as_float(load_coherent(q + 6)), __uint_as_float(load_coherent(q + 7)));
  }
  return f;
}

template <typename E, int NT, int TILES, bool TCTRL>
__device__ void stream_rows(const DecodeArgs& a, int b, uint8_t* smem) {
  constexpr int D = pipe_depth<E, NT, TILES>();
  constexpr int kPairs = TILES * NT;
  const E* X = static_cast<const E*>(a.x);
  const E* W0 = static_cast<const E*>(a.w0);
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), l = tid % kWave;
  const int lr = l & 15, q4 = l >> 4, kq = q4 * 8;
  const int M = a.M, I = a.I, R = a.R, KS = a.KS, RBR = a.RBR;
  const int rb = b / KS, ks = b % KS;
  const int r0 = int(int64_t(rb) * a.O / a.NRB), r1 = int(int64_t(rb + 1) * a.O / a.NRB);
  const int nrows = r1 - r0;
  const bool rank_unit = R > 0 && ks == KS - 1;
  // The sticky error word as this launch found it (thread 0's copy decides,
  // after the stream): a poisoned launch writes NaN to its rows and leaves
  // every counter alone.
  const uint32_t err_at_entry = load_coherent(a.err);
  const uint32_t parity = TCTRL && rank_unit ? load_coherent(&a.ctrl[kParity]) & 1u : 0u;
  __shared__ unsigned s_poisoned;

  // LDS: the cross-wave reduction, then the row scale, then the block's
  // result [16*NT][RBR].
  f32x4* red = reinterpret_cast<f32x4*>(smem);
  float* sbuf = reinterpret_cast<float*>(smem + kWaves * 4 * kWave * 16);
  float* res = sbuf + 16 * TILES;

  // The row scale, fetched now and used after the stream (no s: unit scale).
  const E* S_ = static_cast<const E*>(a.s);
  const float s_mine = tid < nrows ? (S_ ? to_f32<E>(S_[r0 + tid]) : 1.f) : 0.f;

  // Byte offsets, from the block's first row, of the row of each tile this
  // lane loads, clamped into the block (rows past it are computed on
  // duplicate data and never stored); likewise for the token rows of x.  The
  // bases are uniform, so the loads take scalar base + 32-bit vector offset.
  const char* wbase = reinterpret_cast<const char*>(W0 + size_t(r0) * I);
  const char* xbase = reinterpret_cast<const char*>(X);
  uint32_t woff[TILES], xoff[NT];
#pragma unroll
  for (int t = 0; t < TILES; ++t) woff[t] = uint32_t(min(t * 16 + lr, nrows - 1)) * uint32_t(I) * sizeof(E);
#pragma unroll
  for (int c = 0; c < NT; ++c) xoff[c] = uint32_t(min(c * 16 + lr, M - 1)) * uint32_t(I) * sizeof(E);

  // U for this wave's first k32 step of the rank, fetched before the stream
  // when it fits the register budget (else after it).
  constexpr bool kPrefetchU = TILES * frag_vgprs<E>() <= 16;
  const int RS = (R + 31) / 32;
  const bool ualigned = (R % 8) == 0;
  const E* Ub = static_cast<const E*>(a.u) + size_t(r0) * R;
  Frag8<E> uf[TILES];
  if (kPrefetchU && rank_unit && w < RS) {
#pragma unroll
    for (int t = 0; t < TILES; ++t) uf[t] = load_row8<E>(Ub + size_t(min(t * 16 + lr, nrows - 1)) * R, w * 32 + kq, R, ualigned);
  }

  f32x4 acc[TILES][NT];
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma_step = [&](const Frag8<E> (&fw)[TILES], const Frag8<E> (&fx)[NT]) {
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int c = 0; c < NT; ++c) acc[t][c] = mma_k32(fw[t], fx[c], acc[t][c]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_operand_guard();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Full k32 steps sa + w, sa + w + 8, ... of this k-slice: n of them for
  // this wave, in a software pipeline D steps deep.  The loop body is
  // straight-line code: loads are unconditional (step indexes clamped into
  // the slice, so refills past a wave's last step re-read it and go unused),
  // and every wave runs the same whole rounds (those of wave 0, which has the
  // most steps) and meets the others at a barrier after each: left alone the
  // waves drift apart by many microseconds and the stragglers finish with
  // few loads in flight.  The remainder after whole rounds is consumed after
  // the loop.
  const int s_full = I / 32;
  const int sa = int(int64_t(ks) * s_full / KS), sb = int(int64_t(ks + 1) * s_full / KS);
  const int n = sb - sa > w ? (sb - sa - w + kWaves - 1) / kWaves : 0;
  const int n0 = (sb - sa + kWaves - 1) / kWaves;  // wave 0's steps, the most
  if (n0 > 0) {
    Frag8<E> wf[D][TILES], xf[D][NT];
#define TB_ISSUE(SLOT, IDX)                                                                               \
    do {                                                                                                  \
      const uint32_t kb_ = uint32_t(min(sa + w + (IDX) * kWaves, sb - 1) * 32 + kq) * sizeof(E);          \
      _Pragma("unroll") for (int t = 0; t < TILES; ++t)                                                   \
        wf[SLOT][t] = load_frag<E>(reinterpret_cast<const E*>(wbase + (woff[t] + kb_)));                  \
      _Pragma("unroll") for (int c = 0; c < NT; ++c)                                                      \
        xf[SLOT][c] = load_frag<E>(reinterpret_cast<const E*>(xbase + (xoff[c] + kb_)));                  \
    } while (0)
#pragma unroll
    for (int d = 0; d < D; ++d) TB_ISSUE(d, d);
    const int whole = n0 / D * D;
    for (int i0 = 0; i0 < whole; i0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (i0 + d < n) mma_step(wf[d], xf[d]);
        TB_ISSUE(d, i0 + d + D);
        // Keep each slot's refill right behind its use: clustering the
        // refills at the end of the round would drain the pipeline.
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_barrier();
    }
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
      if (whole + d < n) mma_step(wf[d], xf[d]);
#undef TB_ISSUE
  }
  // The partial last step (in_dim not a multiple of 32), masked per lane.
  if (s_full * 32 < I && ks == KS - 1 && w == 0) {
    const int k = s_full * 32 + kq;
    const bool kv = k < I;
    const uint32_t kb = uint32_t(kv ? k : I - 8) * sizeof(E);
    Frag8<E> fw[TILES], fx[NT];
#pragma unroll
    for (int t = 0; t < TILES; ++t) fw[t] = load_frag_if<E>(reinterpret_cast<const E*>(wbase + (woff[t] + kb)), kv);
#pragma unroll
    for (int c = 0; c < NT; ++c) fx[c] = load_frag_if<E>(reinterpret_cast<const E*>(xbase + (xoff[c] + kb)), kv);
    mma_step(fw, fx);
  }

  // Row scale: C rows 4*(l/16)+e of each tile.
  if (tid < nrows) sbuf[tid] = s_mine;
  if (tid == 0) s_poisoned = err_at_entry;
  __syncthreads();
  E* Y = static_cast<E*>(a.y);
  if (s_poisoned != 0u) {
    const E nan = from_f32<E>(__builtin_nanf(""));
    for (int i = tid; i < M * nrows; i += kThreads) Y[size_t(i / nrows) * a.O + r0 + i % nrows] = nan;
    return;
  }
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = t * 16 + q4 * 4 + e;
      const float sc = row < nrows ? sbuf[row] : 0.f;
#pragma unroll
      for (int c = 0; c < NT; ++c) acc[t][c][e] *= sc;
    }

  // The rank-r delta: this wave's k32 steps of T . U^T, once T is complete.
  __shared__ unsigned s_ok;
  if (TCTRL && rank_unit) {
    // Each wave loads its U fragments, then polls the coded words of T it
    // multiplies (the first poll overlaps U's loads); a wave that gives up
    // turns the whole workgroup's result into NaN.
    if (tid == 0) s_ok = 1u;
    __syncthreads();
    const uint32_t* tw = a.ctrl + kTWordBase + parity * kTHalfWords;
    const int Rp = a.NCB * kCbCols;
    for (int rs = w; rs < RS; rs += kWaves) {
      if (rs != w || !kPrefetchU) {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
          uf[t] = load_row8<E>(Ub + size_t(min(t * 16 + lr, nrows - 1)) * R, rs * 32 + kq, R, ualigned);
      }
      constexpr int kW = sizeof(E) == 2 ? 4 : 8;  // words of one lane's 8 columns
      uint32_t words[NT][kW];
      // Thousands of waves poll at once: one lane probes one word of the
      // fragment until it is written, then the wave loads the fragment and
      // checks every word.  (Polling whole fragments flooded the memory-side
      // cache that also serves the W0 stream: 60-layer gate,up 98 -> 106 us;
      // loading the whole fragment at the first attempt and probing only
      // after that cost gate,up 1 us.)
      bool ready = false;
      const uint32_t* probe = tw + (rs * 32) * int(sizeof(E)) / 4;
      for (int it = 0; it < a.polls; ++it) {
        uint32_t seen = 1u;
        if (l == 0) seen = load_coherent(probe);
        if (__builtin_amdgcn_readfirstlane(seen) == 0u) {
          __builtin_amdgcn_s_sleep(8);
          continue;
        }
        bool mine = true;
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const uint32_t* q = tw + ((c * 16 + lr) * Rp + rs * 32 + kq) * int(sizeof(E)) / 4;
#pragma unroll
          for (int e = 0; e < kW; ++e) {
            words[c][e] = load_coherent(q + e);
            mine = mine && words[c][e] != 0u;
          }
        }
        if (__builtin_amdgcn_ballot_w64(!mine) == 0) {
          ready = true;
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      if (!ready) {
        if (l == 0) s_ok = 0u;   // only ever cleared: a benign race between waves
        break;
      }
      Frag8<E> ft[NT];
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        if constexpr (sizeof(E) == 2) {
          ft[c].v = make_uint4(~words[c][0], ~words[c][1], ~words[c][2], ~words[c][3]);
        } else {
          ft[c].lo = make_float4(__uint_as_float(~words[c][0]), __uint_as_float(~words[c][1]),
                                 __uint_as_float(~words[c][2]), __uint_as_float(~words[c][3]));
          ft[c].hi = make_float4(__uint_as_float(~words[c][4]), __uint_as_float(~words[c][5]),
                                 __uint_as_float(~words[c][6]), __uint_as_float(~words[c][7]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int c = 0; c < NT; ++c) acc[t][c] = mma_k32(uf[t], ft[c], acc[t][c]);
      __builtin_amdgcn_sched_barrier(0);
      mfma_operand_guard();
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    if (s_ok == 0u) {
      if (tid == 0) atomicOr(a.err, 1u);
      const float nan = __builtin_nanf("");
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int c = 0; c < NT; ++c) acc[t][c] = f32x4{nan, nan, nan, nan};
    }
  } else if (rank_unit) {
    // One wave polls the done word (every wave polling it would hammer the
    // line the producers count into) and shares the outcome through LDS.
    if (w == 0) {
      const bool ok0 = wait_for_count(&a.ctrl[kDone], unsigned(a.NCB), a.polls);
      if (l == 0) s_ok = ok0 ? 1u : 0u;
    }
    __syncthreads();
    const bool ok = s_ok != 0u;
    if (!ok && w == 0 && l == 0) atomicOr(a.err, 1u);
    for (int rs = w; rs < RS; rs += kWaves) {
      if (rs != w || !kPrefetchU) {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
          uf[t] = load_row8<E>(Ub + size_t(min(t * 16 + lr, nrows - 1)) * R, rs * 32 + kq, R, ualigned);
      }
      Frag8<E> ft[NT];
#pragma unroll
      for (int c = 0; c < NT; ++c) ft[c] = load_t<E>(a, c * 16 + lr, rs * 32 + kq);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int c = 0; c < NT; ++c) acc[t][c] = mma_k32(uf[t], ft[c], acc[t][c]);
      __builtin_amdgcn_sched_barrier(0);
      mfma_operand_guard();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!ok) {
      const float nan = __builtin_nanf("");
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int c = 0; c < NT; ++c) acc[t][c] = f32x4{nan, nan, nan, nan};
    }
  }

  // Every wave is past its read of T: count this rank streamer in now (the
  // answer is needed only at the end, so the atomic's round trip overlaps the
  // reduction and the stores).
  const unsigned fin_groups = unsigned(min(a.NRB, kFinishGroups)), fin_g = unsigned(rb) % fin_groups;
  unsigned fin_old = 0;
  if (rank_unit) {
    __syncthreads();
    if (tid == 0) fin_old = add_coherent(&a.ctrl[kFinishBase + 64 * int(fin_g)], 1u);
  }

  // Sum the eight waves' partials in a fixed order, four (tile, token tile)
  // pairs per round, into the block's result.
#pragma unroll
  for (int p0 = 0; p0 < kPairs; p0 += 4) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (p0 + q < kPairs) red[(w * 4 + q) * kWave + l] = acc[(p0 + q) / NT][(p0 + q) % NT];
    __syncthreads();
    if (w < 4 && p0 + w < kPairs) {
      f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < kWaves; ++v) sum += red[(v * 4 + w) * kWave + l];
      const int t = (p0 + w) / NT, c = (p0 + w) % NT;
#pragma unroll
      for (int e = 0; e < 4; ++e) res[(c * 16 + lr) * RBR + t * 16 + q4 * 4 + e] = sum[e];
    }
  }
  __syncthreads();

  // Store y, or this k-slice's partial (the last of the row block to arrive
  // sums all KS partials in k-slice order).
  const int nel = M * nrows;
  if (KS == 1) {
    for (int i = tid; i < nel; i += kThreads) {
      const int tok = i / nrows, row = i % nrows;
      Y[size_t(tok) * a.O + r0 + row] = from_f32<E>(res[tok * RBR + row]);
    }
  } else {
    // If the row block's other k-slices have all counted in already (the
    // slice that waited for T usually arrives last), this workgroup sums
    // their partials at once and stores none of its own; otherwise it stores
    // its partial and counts in.  Either way the sum runs in k-slice order.
    __shared__ unsigned s_last;
    if (tid == 0) s_last = load_coherent(&a.ctrl[kRbCounters + rb]) == unsigned(KS - 1) ? 1u : 0u;
    __syncthreads();
    if (!s_last) {
      float* mine = a.ypart + (size_t(rb) * KS + ks) * (16 * NT) * RBR;
      for (int i = tid; i < nel; i += kThreads) {
        const int tok = i / nrows, row = i % nrows;
        store_coherent(&mine[tok * RBR + row], __float_as_uint(res[tok * RBR + row]));
      }
      drain_stores();
      __syncthreads();
      if (tid == 0) s_last = add_coherent(&a.ctrl[kRbCounters + rb], 1u) == unsigned(KS - 1);
      __syncthreads();
    }
    if (s_last) {
      const float* blk = a.ypart + size_t(rb) * KS * (16 * NT) * RBR;
      for (int i = tid; i < nel; i += kThreads) {
        const int tok = i / nrows, row = i % nrows;
        float sum = 0.f;
        for (int k = 0; k < KS; ++k)
          sum += k == ks ? res[tok * RBR + row]
                         : __uint_as_float(load_coherent(&blk[(size_t(k) * (16 * NT) + tok) * RBR + row]));
        Y[size_t(tok) * a.O + r0 + row] = from_f32<E>(sum);
      }
      if (tid == 0) store_coherent(&a.ctrl[kRbCounters + rb], 0u);
    }
  }

  // The last of a group clears its counter and bumps the top counter; the
  // last there, the last rank streamer past its read of T, resets the
  // producers' count, or flips the exchange parity.
  if (rank_unit && tid == 0) {
    const unsigned members = (unsigned(a.NRB) - fin_g + fin_groups - 1) / fin_groups;
    if (fin_old == members - 1) {
      store_coherent(&a.ctrl[kFinishBase + 64 * int(fin_g)], 0u);
      unsigned* top = &a.ctrl[kFinishBase + 64 * kFinishGroups];
      if (add_coherent(top, 1u) == fin_groups - 1) {
        store_coherent(top, 0u);
        if (TCTRL) store_coherent(&a.ctrl[kParity], parity ^ 1u);
        else store_coherent(&a.ctrl[kDone], 0u);
      }
    }
  }
}

constexpr int kReduceBytes = kWaves * 4 * kWave * 16;  // the streamers' cross-wave reduction

template <typename E, int NT, int TILES>
constexpr int smem_bytes() {
  constexpr int streamer = kReduceBytes + int(sizeof(float)) * (16 * TILES + 16 * NT * 16 * TILES);
  return streamer > producer_smem<E, NT>() ? streamer : producer_smem<E, NT>();
}

// One launch serves a group of independent projections of the same token
// count and tile shape: all of their producers first (in projection order),
// then all of their streamers, so a streamer's producers always have lower
// block indexes and have been dispatched before it.
struct GroupArgs {
  int n;
  int p_end[kMaxProjections];  // producers of projections 0..j: blocks [0, p_end[j])
  int s_end[kMaxProjections];  // streamers of projections 0..j: blocks [p_end[n-1], p_end[n-1] + s_end[j])
  DecodeArgs a[kMaxProjections];
};

// Waves per SIMD that the register budget is cut for: four (two workgroups
// per compute unit), except for the variants of 32 tokens x 96 rows and of
// 64 tokens x 64 or 96 rows, whose accumulators need more registers (one
// workgroup per compute unit).
// fp32 fragments take twice the registers: every fp32 variant is cut for two
// waves per SIMD, and the planner plans them so.
template <typename E, int NT, int TILES> constexpr int decode_waves_per_eu() {
  return sizeof(E) == 4 || NT * TILES >= 12 ? 2 : 4;
}

template <typename E, int NT, int TILES, bool TCTRL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<E, NT, TILES>()))) void
decode_kernel(GroupArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[smem_bytes<E, NT, TILES>()];
  const int b = int(blockIdx.x), np = g.p_end[g.n - 1];
  int j = 0;
  if (b < np) {
    while (b >= g.p_end[j]) ++j;
    produce_t<E, NT, TCTRL>(g.a[j], b - (j ? g.p_end[j - 1] : 0), smem);
  } else {
    const int bs = b - np;
    while (bs >= g.s_end[j]) ++j;
    stream_rows<E, NT, TILES, TCTRL>(g.a[j], bs - (j ? g.s_end[j - 1] : 0), smem);
  }
}

template <typename E, int NT, int TILES>
hipError_t launch_t(bool tctrl, const GroupArgs& g, hipStream_t stream) {
  const dim3 grid(g.p_end[g.n - 1] + g.s_end[g.n - 1]);
  if (tctrl) hipLaunchKernelGGL((decode_kernel<E, NT, TILES, true>), grid, dim3(kThreads), 0, stream, g);
  else hipLaunchKernelGGL((decode_kernel<E, NT, TILES, false>), grid, dim3(kThreads), 0, stream, g);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_e(int NT, int TILES, bool tctrl, const GroupArgs& g, hipStream_t stream) {
  if (NT == 1) {
    switch (TILES) {
      case 1: return launch_t<E, 1, 1>(tctrl, g, stream);
      case 2: return launch_t<E, 1, 2>(tctrl, g, stream);
      case 4: return launch_t<E, 1, 4>(tctrl, g, stream);
      default: return launch_t<E, 1, 6>(tctrl, g, stream);
    }
  }
  if (NT == 2) {
    switch (TILES) {
      case 1: return launch_t<E, 2, 1>(tctrl, g, stream);
      case 2: return launch_t<E, 2, 2>(tctrl, g, stream);
      case 4: return launch_t<E, 2, 4>(tctrl, g, stream);
      default: return launch_t<E, 2, 6>(tctrl, g, stream);
    }
  }
  if (TILES == 1) return launch_t<E, 4, 1>(tctrl, g, stream);
  if (TILES == 2) return launch_t<E, 4, 2>(tctrl, g, stream);
  if (TILES == 4) return launch_t<E, 4, 4>(tctrl, g, stream);
  return launch_t<E, 4, 6>(tctrl, g, stream);
}

}  // namespace

namespace {
// Rows of a streaming workgroup at most (six 16-row tiles at every NT).
// Every row block re-reads x, so the more tokens, the more wide blocks matter.
int64_t decode_max_rows(int) { return 96; }
// Producer k-slices: about 768 of in_dim (three k32 steps per wave, one
// round of loads at 16 tokens) when T must be ready early; about 5632
// (22 steps per wave) when the launch streams at least 56 Mi elements of W0
// (112 MiB of bf16, over ~20 us), which hides the longer chain and leaves
// fewer producers to take compute units from the streamers.  (Slices sized
// to half of a compute unit's share of W0 were tried: the q,k,v producers
// then finished long before the streams, but their extra compute units made
// the streams and the 60-layer stack at 16 tokens slower, 227 -> 234 us per
// layer.)
constexpr int64_t kShortSlice = 768, kLongSlice = 5632;
// A short reduction (in_dim <= 1536) is split into slices of about 144: its
// producers then finish in a few microseconds, while one producer per column
// block spent ~9 us streaming its V columns alone (stamped) and left the
// streamers waiting.  26-layer banded stack at 1 / 4 / 16 tokens, one box,
// slices of 1152 / 576 / 288 / 192 / 144 / 96 / 72: 1.432 / 1.465 / 1.389 /
// 1.349 / 1.332 / 1.367 / 1.394 ms per step at 1 token, the same order at 4
// and 16.
constexpr int64_t kTinySlice = 144, kShortReduction = 1536;
constexpr int64_t kLongStreamElems = int64_t(56) << 20;
// x sizes (tokens x in_dim) up to which the streamers take one k-slice each:
// the x that every row block re-reads is small next to the cost of combining
// k-slice partials across workgroups.  Measured per call, one slice against
// the k-sliced plan: 60-layer o at 1 / 8 tokens 25.6 -> 23.1 / 26.9 -> 25.8
// us, down at 1 token 45.8 -> 42.4 us; 26-layer down at 4 / 8 tokens 15.0 ->
// 13.0 / 15.1 -> 13.7 us.  60-layer down at 8 tokens (172K elements of x)
// loses 2.4 us, at 16 tokens 8.5 us.
constexpr int64_t kOneSliceX = 65536;
}  // namespace

DecodePlan plan_decode(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, int streamers, int cus,
                       int64_t stream_elems) {
  DecodePlan p{};
  p.NT = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
  const int64_t max_rows = decode_max_rows(p.NT);
  const int64_t s_full = in_dim / 32;
  // Streamers.  Every streamer of a row block reads all of x for its k-slice,
  // so the x traffic grows with the number of row blocks.  A small x
  // (kOneSliceX): one k-slice, as many row blocks as streamers (no partials
  // to combine across workgroups).  Otherwise use as few blocks as the widest
  // tile set allows and split in_dim so that there is about one streamer per
  // compute unit (each wave keeping at least four k32 steps).
  const int64_t nrb_min = (out_dim + max_rows - 1) / max_rows;
  int64_t ks = 1, nrb;
  if (m * in_dim <= kOneSliceX) {
    nrb = nrb_min > streamers ? nrb_min : int64_t(streamers);
  } else if (nrb_min >= streamers) {
    nrb = streamers;
    while ((out_dim + nrb - 1) / nrb > max_rows) nrb += streamers;
  } else {
    ks = streamers / nrb_min;
    const int64_t ks_cap = s_full / 32 > 1 ? s_full / 32 : 1;
    if (ks > ks_cap) ks = ks_cap;
    if (ks > 16) ks = 16;
    nrb = streamers / ks;
    if (nrb < nrb_min) nrb = nrb_min;
  }
  if (nrb > out_dim) nrb = out_dim;
  if (ks > 1 && nrb > kMaxGroupCounters / 2) ks = 1;  // one arrival counter per row block
  const int64_t tiles = ((out_dim + nrb - 1) / nrb + 15) / 16;
  p.TILES = tiles <= 1 ? 1 : (tiles <= 2 ? 2 : (tiles <= 4 ? 4 : 6));
  p.NRB = int(nrb);
  p.KS = int(ks);
  p.NB = p.NRB * p.KS;
  // Producers: 64 columns of T each, over k-slices of in_dim.
  if (rank > 0) {
    p.NCB = int((rank + kCbCols - 1) / kCbCols);
    const int64_t slice = in_dim <= kShortReduction        ? kTinySlice
                          : stream_elems >= kLongStreamElems ? kLongSlice
                                                             : kShortSlice;
    int64_t kt = (in_dim + slice - 1) / slice;
    if (kt > kMaxKT) kt = kMaxKT;
    if (p.NCB > kMaxGroupCounters / 2) kt = 1;  // one arrival counter per column block
    p.KT = int(kt);
  } else {
    p.NCB = 0;
    p.KT = 1;
  }
  p.NP = p.NCB * p.KT;
  const size_t rows16 = size_t(16 * p.NT);
  const size_t rbr = size_t(16 * p.TILES);
  size_t off = 0;
  p.off_tpart = off;  // [KT][16*NT][Rp] fp32 (KT > 1)
  off = align_up(off + (p.KT > 1 ? size_t(p.KT) * rows16 * size_t(p.NCB) * kCbCols * 4 : 0), 256);
  p.off_tfull = off;  // [16*NT][Rp], fp32 or bf16
  off = align_up(off + rows16 * size_t(p.NCB) * kCbCols * 4, 256);
  p.off_ypart = off;  // [NRB][KS][16*NT][RBR] fp32
  off = align_up(off + (p.KS > 1 ? size_t(p.NRB) * size_t(p.KS) * rows16 * rbr * 4 : 0), 256);
  p.bytes = off;
  return p;
}

DecodePlan plan_decode_spared(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, int cus, int64_t stream_elems) {
  const DecodePlan p = plan_decode(m, out_dim, in_dim, rank, cus, cus, stream_elems);
  if (p.NP == 0 || 4 * p.NP >= cus) return p;
  // The producer count does not depend on the streamers.
  return plan_decode(m, out_dim, in_dim, rank, cus - p.NP, cus, stream_elems);
}

bool plan_decode_shared(int n, const Projection* projs, int64_t m, int cus, int slots, int64_t stream_elems,
                        DecodePlan* plans) {
  int64_t producers = 0;
  double w0 = 0.0;
  for (int j = 0; j < n; ++j) {
    producers += plan_decode(m, projs[j].out_dim, projs[j].in_dim, projs[j].rank, cus, cus, stream_elems).NP;
    w0 += double(projs[j].out_dim) * double(projs[j].in_dim);
  }
  const int64_t slots_total = int64_t(slots) * cus, streamers = slots_total - producers;
  if (slots < 1 || slots > kMaxDecodeSlots || streamers < 4 * int64_t(n)) return false;
  int64_t total = producers;
  for (int j = 0; j < n; ++j) {
    const Projection& q = projs[j];
    const int64_t b = int64_t(double(streamers) * double(q.out_dim) * double(q.in_dim) / w0);
    plans[j] = plan_decode(m, q.out_dim, q.in_dim, q.rank, int(b > 1 ? b : 1), cus, stream_elems);
    total += plans[j].NB;
    if (plans[j].NT != plans[0].NT || plans[j].TILES != plans[0].TILES) return false;
  }
  return total <= slots_total;
}

// With KS > 1 the planner takes NRB = streamers / KS row blocks of at most
// decode_max_rows(NT) rows, so NRB * KS never exceeds the budget.  The
// buffers before the y partials do not depend on the budget and are largest
// with the short producer k-slices.
size_t decode_bytes_bound(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, int cus) {
  const DecodePlan p = plan_decode(m, out_dim, in_dim, rank, cus, cus, 0);
  const size_t ypart = size_t(kMaxDecodeSlots) * size_t(cus) * size_t(16 * p.NT) * size_t(decode_max_rows(p.NT)) * 4;
  return p.off_ypart + align_up(ypart, 256);
}

hipError_t launch_forward_decode_group(int n, const DecodePlan* plans, const Projection* projs, tb_dtype dtype,
                                       int64_t m, unsigned* ctrl, char* data, unsigned* err_word, hipStream_t stream) {
  if (n < 1 || n > kMaxProjections) return hipErrorInvalidValue;
  GroupArgs g{};
  g.n = n;
  char* ws = data;
  int np = 0, nb = 0;
  bool tctrl = true;
  for (int j = 0; j < n; ++j) {
    const DecodePlan& p = plans[j];
    const Projection& q = projs[j];
    if (p.NT != plans[0].NT || p.TILES != plans[0].TILES) return hipErrorInvalidValue;
    DecodeArgs& a = g.a[j];
    a.x = q.x; a.s = q.s; a.w0 = q.w0; a.u = q.u; a.v = q.v; a.y = q.y;
    a.M = int(m); a.O = int(q.out_dim); a.I = int(q.in_dim); a.R = int(q.rank);
    a.NCB = p.NCB; a.KT = p.KT;
    a.NRB = p.NRB; a.KS = p.KS; a.RBR = 16 * p.TILES;
    a.ctrl = ctrl + j * (kCtrlBlockBytes / 4);
    a.err = err_word;
    a.polls = decode_wait_polls();
    a.tpart = reinterpret_cast<float*>(ws + p.off_tpart);
    a.tfull = ws + p.off_tfull;
    a.ypart = reinterpret_cast<float*>(ws + p.off_ypart);
    // T through the control block's coded words when every member's fits.
    tctrl = tctrl && (dtype == TB_BF16 ? t_words<bf16_t>(p.NT, p.NCB * kCbCols)
                                       : t_words<float>(p.NT, p.NCB * kCbCols)) <= kTHalfWords;
    np += p.NP;
    nb += p.NB;
    g.p_end[j] = np;
    g.s_end[j] = nb;
    ws += p.bytes;  // the next projection's buffers
  }
  if (dtype == TB_BF16) return launch_e<bf16_t>(plans[0].NT, plans[0].TILES, tctrl, g, stream);
  return launch_e<float>(plans[0].NT, plans[0].TILES, tctrl, g, stream);
}

hipError_t launch_forward_decode(const DecodePlan& p, tb_dtype dtype, const void* x, const void* s, const void* w0,
                                 const void* u, const void* v, void* y, int64_t m, int64_t out_dim, int64_t in_dim,
                                 int64_t rank, unsigned* ctrl, char* data, unsigned* err_word, hipStream_t stream) {
  const Projection q{x, s, w0, u, v, y, out_dim, in_dim, rank};
  return launch_forward_decode_group(1, &p, &q, dtype, m, ctrl, data, err_word, stream);
}

}  // namespace tb
