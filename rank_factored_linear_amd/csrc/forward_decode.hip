// Fused theta-bundle projection for few tokens (m <= 64): one launch.
//
//   y = s (.) (x . W0^T) + (x . V) . U^T        ("The theta bundle": the
//   transpose of weight = diag(s) W0 + U V^T applied to x)
//
// At these token counts the projection is bound by HBM bandwidth: every byte
// of W0 is read once, and U, V, s once.  The grid holds two kinds of
// workgroups, told apart by their index:
//
//   producers (indices 0..NP-1) compute T = x . V on the matrix cores, each
//     over four k32 steps of in_dim, into private partials.  They meet at a
//     barrier (they hold the lowest indices, so they are dispatched first and
//     are all resident), then each sums one slice of T over all partials in a
//     fixed order and stores it; the last to finish raises a ready flag that
//     carries this call's epoch.
//   consumers (the rest) each own a contiguous, balanced range of at most
//     16*RT output rows over the whole of in_dim.  Eight waves take the k32
//     steps round-robin, streaming W0 rows through v_mfma 16x16x32 with x as
//     the 16-token B operand (zero padded), and reduce in LDS in a fixed
//     order.  The epilogue scales each row by s, waits for the flag, adds
//     T . U^T on the matrix cores and stores y rounded once.
//
// All data that crosses workgroups (partials, T, counters, flag) is written
// and read with device-scope (sc1) accesses, which are coherent across XCDs
// without writing back or invalidating the L2; a writer waits for its stores
// to complete (s_waitcnt) before it counts itself in.  No workgroup ever
// fences, takes a ticket or waits on a consumer, and the flag needs no reset
// because each call brings a new epoch.  Every wait is bounded: a timeout
// sets an error word and poisons the output with NaN instead of hanging.
#include "tb_device.h"
#include "tb_host.h"

namespace tb {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kVCols = 256;          // columns of V per producer pass
constexpr int kVPitch = 40;          // LDS pitch (elements) of the transposed V tile
constexpr int kStageChunks = 32 * (kVCols / 8) / kThreads;  // 16-byte V chunks per thread per step
constexpr int kMaxProducers = 256;   // at most one per compute unit: all resident together
constexpr int kStepsPerProducer = 4;  // k32 steps of V per producer (one batch of loads)

// Control words: [kFlag] T-ready epoch, [kErr] sticky timeout flag,
// [kArrive] / [kDepart] producer barrier, [kPublished] T slices stored.
enum Ctrl { kFlag = 1, kErr = 2, kArrive = 3, kDepart = 4, kPublished = 5 };

// Loads kept in flight per wave scale down with the token tiles so that the
// kernel fits 128 VGPRs (two 512-thread workgroups per compute unit).
constexpr int per_tile_budget(int base, int nt) { return base / nt > 0 ? base / nt : 1; }

struct DecodeArgs {
  const void* x;
  const void* s;
  const void* w0;
  const void* u;
  const void* v;
  void* y;
  int M, O, I, R;
  int S, NP, NB;
  unsigned epoch;
  unsigned* ctrl;
  float* tpart;
  float* tfull;
};

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

// B fragment of T (published zero padded as [16*NT][Rp]) read coherently.
template <typename E> __device__ __forceinline__ Frag8<E> load_t_frag(const void* p);
template <> __device__ __forceinline__ Frag8<bf16_t> load_t_frag<bf16_t>(const void* p) {
  const uint32_t* q = static_cast<const uint32_t*>(p);
  Frag8<bf16_t> f;
  f.v = make_uint4(load_coherent(q), load_coherent(q + 1), load_coherent(q + 2), load_coherent(q + 3));
  return f;
}
template <> __device__ __forceinline__ Frag8<float> load_t_frag<float>(const void* p) {
  const uint32_t* q = static_cast<const uint32_t*>(p);
  Frag8<float> f;
  f.lo = make_float4(__uint_as_float(load_coherent(q)), __uint_as_float(load_coherent(q + 1)),
                     __uint_as_float(load_coherent(q + 2)), __uint_as_float(load_coherent(q + 3)));
  f.hi = make_float4(__uint_as_float(load_coherent(q + 4)), __uint_as_float(load_coherent(q + 5)),
                     __uint_as_float(load_coherent(q + 6)), __uint_as_float(load_coherent(q + 7)));
  return f;
}

// Bounded waits (about 0.1 s at most; relaxed polling, no cache invalidation).
__device__ __forceinline__ bool wait_for_epoch(const unsigned* flag, unsigned epoch) {
  for (int it = 0; it < (1 << 20); ++it) {
    if (load_coherent(flag) == epoch) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}
__device__ __forceinline__ bool wait_for_count(const unsigned* counter, unsigned target) {
  for (int it = 0; it < (1 << 20); ++it) {
    if (load_coherent(counter) >= target) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// Wait until this wave's outstanding memory operations have completed: its
// device-scope stores are then visible to every XCD.  Each wave runs it before
// the barrier that precedes an arrival.
__device__ __forceinline__ void drain_stores() { __builtin_amdgcn_s_waitcnt(0); }

// ---------------------------------------------------------------------------
// Producer: partial T over k32 steps [p*S/NP, (p+1)*S/NP) of in_dim, then,
// after the producer barrier, one slice of T summed over all partials.
// ---------------------------------------------------------------------------
// Chunk c of a 32 x kVCols tile of V is row (c % 32), columns 8*(c / 32)..+7:
// consecutive lanes take consecutive rows, so their transposed LDS stores
// fall in consecutive banks.
template <typename E>
__device__ __forceinline__ Frag8<E> load_v_chunk(const E* V, int k0, int jc0, int I, int R, bool valigned, int c) {
  const int row = c % 32, cg = (c / 32) * 8;
  const int gi = k0 + row, gj = jc0 + cg;
  if (gi >= I || gj >= R) return zero_frag<E>();
  const E* src = V + size_t(gi) * R + gj;
  return (valigned && gj + 8 <= R) ? load_frag<E>(src) : load_frag_partial<E>(src, min(8, R - gj));
}

template <typename E, typename Raw>
__device__ __forceinline__ void store_v_chunk(Raw* vt, int c, const Frag8<E>& f) {
  const int row = c % 32, cg = (c / 32) * 8;
  Raw vals[8];
  __builtin_memcpy(vals, &f, sizeof(vals));
#pragma unroll
  for (int e = 0; e < 8; ++e) vt[(cg + e) * kVPitch + row] = vals[e];
}

template <typename E, int NT>
__device__ void produce_xv(const DecodeArgs& a, int p, void* smem) {
  using Raw = typename std::conditional<sizeof(E) == 2, uint16_t, float>::type;
  // k32 steps whose loads are in flight together (bounded by registers).
  constexpr int kBatch = per_tile_budget(sizeof(E) == 2 ? 4 : 2, NT);
  Raw* vt = static_cast<Raw*>(smem);  // [kVCols][kVPitch]
  const E* X = static_cast<const E*>(a.x);
  const E* V = static_cast<const E*>(a.v);
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int lr = l & 15, kq = (l >> 4) * 8;
  const int M = a.M, I = a.I, R = a.R;
  const int s0 = int(int64_t(p) * a.S / a.NP), s1 = int(int64_t(p + 1) * a.S / a.NP);
  const bool valigned = (R % 8) == 0;
  const int n = M * R;
  float* tp = a.tpart + size_t(p) * n;
  constexpr int kTilesPerWave = kVCols / 16 / kWaves;  // 2

  for (int jc0 = 0; jc0 < R; jc0 += kVCols) {
    f32x4 acc[NT][kTilesPerWave];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int c = 0; c < kTilesPerWave; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int b0 = s0; b0 < s1; b0 += kBatch) {
      // Issue every load of the batch first.
      Frag8<E> rv[kBatch][kStageChunks], rx[kBatch][NT];
#pragma unroll
      for (int bi = 0; bi < kBatch; ++bi) {
        const int k0 = (b0 + bi) * 32;
        const bool live = b0 + bi < s1;
#pragma unroll
        for (int q = 0; q < kStageChunks; ++q)
          rv[bi][q] = live ? load_v_chunk<E>(V, k0, jc0, I, R, valigned, tid + kThreads * q) : zero_frag<E>();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int tok = t * 16 + lr;
          rx[bi][t] = load_frag_if<E>(X + size_t(tok) * I + k0 + kq, live && tok < M && k0 + kq < I);
        }
      }
#pragma unroll
      for (int bi = 0; bi < kBatch; ++bi) {
        if (b0 + bi >= s1) break;
        __syncthreads();  // the previous step's reads of vt are done
#pragma unroll
        for (int q = 0; q < kStageChunks; ++q) store_v_chunk<E, Raw>(vt, tid + kThreads * q, rv[bi][q]);
        __syncthreads();
#pragma unroll
        for (int c = 0; c < kTilesPerWave; ++c) {
          const int col = (w * kTilesPerWave + c) * 16 + lr;
          const Frag8<E> fv = load_frag<E>(reinterpret_cast<const E*>(&vt[col * kVPitch + kq]));
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t][c] = mma_k32(rx[bi][t], fv, acc[t][c]);
        }
      }
    }
    // C layout: lane holds tokens 4*(l/16)+e of tile t, column lr of tile c.
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int c = 0; c < kTilesPerWave; ++c) {
        const int j = jc0 + (w * kTilesPerWave + c) * 16 + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tok = t * 16 + (l >> 4) * 4 + e;
          if (tok < M && j < R) store_coherent(&tp[size_t(tok) * R + j], __float_as_uint(acc[t][c][e]));
        }
      }
  }

  // Barrier of the producers.  The last to depart resets the counters (every
  // producer has seen the full count by then).
  __shared__ unsigned s_ok;
  __shared__ float s_red[kThreads];
  drain_stores();
  __syncthreads();
  if (tid == 0) {
    add_coherent(&a.ctrl[kArrive], 1u);
    const bool ok = wait_for_count(&a.ctrl[kArrive], unsigned(a.NP));
    if (!ok) atomicOr(&a.ctrl[kErr], 1u);
    if (add_coherent(&a.ctrl[kDepart], 1u) == unsigned(a.NP - 1)) {
      store_coherent(&a.ctrl[kArrive], 0u);
      store_coherent(&a.ctrl[kDepart], 0u);
    }
    s_ok = ok;
  }
  __syncthreads();

  // This producer's slice of T, published zero padded as [16*NT][Rp] in the
  // operand type, two elements per 32-bit word.  `tpo` threads share one word:
  // each sums a contiguous run of partials, then the runs are added in order.
  const int Rp = (R + 31) / 32 * 32;
  const int n_words = 16 * NT * Rp / 2;
  const int w0_ = int(int64_t(p) * n_words / a.NP), w1_ = int(int64_t(p + 1) * n_words / a.NP);
  const int nw = w1_ - w0_;
  int tpo = 1;
  while (tpo * 2 * nw <= kThreads && tpo * 2 <= a.NP) tpo *= 2;
  const int per_pass = kThreads / tpo;
  const int sub = tid % tpo, q0 = sub * a.NP / tpo, q1 = (sub + 1) * a.NP / tpo;
  for (int wb = w0_; wb < w1_; wb += per_pass) {
    const int word = wb + tid / tpo;
    float part[2] = {0.f, 0.f};
    if (word < w1_) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int idx = 2 * word + h, tok = idx / Rp, j = idx % Rp;
        if (tok < M && j < R) {
          const float* src = a.tpart + size_t(tok) * R + j;
          int q = q0;
          for (; q + 8 <= q1; q += 8) {
            float v8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v8[u] = __uint_as_float(load_coherent(src + size_t(q + u) * n));
#pragma unroll
            for (int u = 0; u < 8; ++u) part[h] += v8[u];
          }
          for (; q < q1; ++q) part[h] += __uint_as_float(load_coherent(src + size_t(q) * n));
        }
      }
    }
    __syncthreads();
    s_red[tid] = part[0];
    __syncthreads();
    float lo = 0.f;
    if (sub == 0)
      for (int k = 0; k < tpo; ++k) lo += s_red[tid + k];
    __syncthreads();
    s_red[tid] = part[1];
    __syncthreads();
    if (sub == 0 && word < w1_) {
      float hi = 0.f;
      for (int k = 0; k < tpo; ++k) hi += s_red[tid + k];
      if (!s_ok) lo = hi = __builtin_nanf("");
      uint32_t bits;
      if constexpr (sizeof(E) == 2) {
        bits = uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
        store_coherent(reinterpret_cast<uint32_t*>(a.tfull) + word, bits);
      } else {
        store_coherent(reinterpret_cast<uint32_t*>(a.tfull) + 2 * word, __float_as_uint(lo));
        store_coherent(reinterpret_cast<uint32_t*>(a.tfull) + 2 * word + 1, __float_as_uint(hi));
      }
    }
  }
  drain_stores();
  __syncthreads();
  if (tid == 0 && add_coherent(&a.ctrl[kPublished], 1u) == unsigned(a.NP - 1)) {
    store_coherent(&a.ctrl[kPublished], 0u);
    store_coherent(&a.ctrl[kFlag], a.epoch);
  }
}

// ---------------------------------------------------------------------------
// Consumer: output rows [c*16*RT, (c+1)*16*RT) over the whole of in_dim.
// ---------------------------------------------------------------------------
template <typename E, int NT, int RT, int UNR>
__device__ void consume(const DecodeArgs& a, int c, f32x4* red) {
  const E* X = static_cast<const E*>(a.x);
  const E* W0 = static_cast<const E*>(a.w0);
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int lr = l & 15, kq = (l >> 4) * 8;
  const int M = a.M, I = a.I, R = a.R;
  // Balanced contiguous row range [o_base, o_end) of this workgroup; the
  // tiles' rows past o_end are masked.
  const int o_base = int(int64_t(c) * a.O / a.NB), o_end = int(int64_t(c + 1) * a.O / a.NB);

  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int st = w; st < a.S; st += kWaves * UNR) {
    Frag8<E> fa[UNR][RT], fb[UNR][NT];
#pragma unroll
    for (int uu = 0; uu < UNR; ++uu) {
      const int step = st + kWaves * uu;
      const int k = step * 32 + kq;
      const bool kv = step < a.S && k < I;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int row = o_base + rt * 16 + lr;
        fa[uu][rt] = load_frag_if<E>(W0 + size_t(row) * I + k, kv && row < o_end);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int tok = t * 16 + lr;
        fb[uu][t] = load_frag_if<E>(X + size_t(tok) * I + k, kv && tok < M);
      }
    }
#pragma unroll
    for (int uu = 0; uu < UNR; ++uu)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[rt][t] = mma_k32(fa[uu][rt], fb[uu][t], acc[rt][t]);
  }

  // Fixed-order reduction over the eight waves; wave q < RT*NT keeps tile q.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t) red[((w * RT + rt) * NT + t) * kWave + l] = acc[rt][t];
  __syncthreads();

  const bool mine = w < RT * NT;
  const int rt = mine ? w / NT : 0, t = mine ? w % NT : 0;
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
  if (mine) {
#pragma unroll
    for (int q = 0; q < kWaves; ++q) sum += red[((q * RT + rt) * NT + t) * kWave + l];
  }

  // Epilogue: row scale, then the rank-r delta, then one rounding.
  const E* S_ = static_cast<const E*>(a.s);
  const int orow0 = o_base + rt * 16 + (l >> 4) * 4;
  const int tok = t * 16 + lr;
  if (mine) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[e] *= (orow0 + e < o_end) ? to_f32<E>(S_[orow0 + e]) : 0.f;
  }

  bool ok = true;
  if (R > 0) {
    __shared__ unsigned s_ok;
    if (tid == 0) {
      const bool got = wait_for_epoch(&a.ctrl[kFlag], a.epoch);
      if (!got) atomicOr(&a.ctrl[kErr], 1u);
      s_ok = got;
    }
    __syncthreads();
    ok = s_ok;
    if (mine) {
      const E* U = static_cast<const E*>(a.u);
      const E* T = reinterpret_cast<const E*>(a.tfull);
      const int urow = o_base + rt * 16 + lr;
      const int Rp = (R + 31) / 32 * 32;
      const bool aligned = (R % 8) == 0;
      constexpr int kEpi = 4;  // k32 steps of the rank tail whose loads are in flight together
      for (int kb = 0; kb < R; kb += 32 * kEpi) {
        Frag8<E> fu[kEpi], ft[kEpi];
#pragma unroll
        for (int q = 0; q < kEpi; ++q) {
          const int j = kb + 32 * q + kq;
          fu[q] = zero_frag<E>();
          ft[q] = zero_frag<E>();
          if (j < Rp) ft[q] = load_t_frag<E>(T + size_t(tok) * Rp + j);
          if (urow < o_end && j < R)
            fu[q] = aligned ? load_frag<E>(U + size_t(urow) * R + j) : load_frag_partial<E>(U + size_t(urow) * R + j, min(8, R - j));
        }
#pragma unroll
        for (int q = 0; q < kEpi; ++q) sum = mma_k32(fu[q], ft[q], sum);
      }
    }
  }
  if (!mine) return;
  if (!ok) sum = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};

  E* Y = static_cast<E*>(a.y);
  if (tok < M) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (orow0 + e < o_end) Y[size_t(tok) * a.O + orow0 + e] = from_f32<E>(sum[e]);
  }
}

template <typename E, int NT, int RT>
__global__ __launch_bounds__(kThreads) void forward_decode_kernel(DecodeArgs a) {
  constexpr int kConsumerLds = kWaves * RT * NT * kWave * 16;
  constexpr int kProducerLds = kVCols * kVPitch * int(sizeof(E));
  constexpr int kLds = kConsumerLds > kProducerLds ? kConsumerLds : kProducerLds;
  __shared__ float4 smem[kLds / 16];
  if (int(blockIdx.x) < a.NP) {
    produce_xv<E, NT>(a, int(blockIdx.x), smem);
  } else {
    constexpr int UNR = per_tile_budget(sizeof(E) == 2 ? 4 : 2, NT);
    consume<E, NT, RT, UNR>(a, int(blockIdx.x) - a.NP, reinterpret_cast<f32x4*>(smem));
  }
}

template <typename E, int NT, int RT>
hipError_t launch_t(const DecodeArgs& a, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL((forward_decode_kernel<E, NT, RT>), dim3(blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const DecodePlan& p, const DecodeArgs& a, hipStream_t stream) {
  const int blocks = p.NP + p.NG;
  if (p.NT == 1) {
    switch (p.RT) {
      case 4: return launch_t<E, 1, 4>(a, blocks, stream);
      case 3: return launch_t<E, 1, 3>(a, blocks, stream);
      case 2: return launch_t<E, 1, 2>(a, blocks, stream);
      default: return launch_t<E, 1, 1>(a, blocks, stream);
    }
  }
  if (p.NT == 2) {
    if (p.RT == 2) return launch_t<E, 2, 2>(a, blocks, stream);
    return launch_t<E, 2, 1>(a, blocks, stream);
  }
  return launch_t<E, 4, 1>(a, blocks, stream);
}

}  // namespace

DecodePlan plan_decode(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, int cus) {
  DecodePlan p{};
  p.NT = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
  p.S = int((in_dim + 31) / 32);
  // Consumers: a multiple of the compute-unit count, each with a balanced row
  // range of at most 16 * (4 / NT) rows; RT tiles cover the widest range.
  const int64_t max_rows = 16 * (4 / p.NT);
  int64_t nb = cus;
  while ((out_dim + nb - 1) / nb > max_rows) nb += cus;
  if (nb > out_dim) nb = out_dim;
  p.NG = int(nb);
  const int64_t rows = (out_dim + nb - 1) / nb;
  p.RT = int((rows + 15) / 16);
  if (rank > 0) {
    int np = (p.S + kStepsPerProducer - 1) / kStepsPerProducer;
    const int cap = cus < kMaxProducers ? cus : kMaxProducers;
    if (np > cap) np = cap;
    if (np < 1) np = 1;
    p.NP = np;
  } else {
    p.NP = 0;
  }
  const size_t rp = size_t((rank + 31) / 32 * 32);
  size_t off = kControlBytes;
  p.off_tpart = off;  // NP partials of [m][rank] fp32
  off = align_up(off + size_t(p.NP) * size_t(m) * size_t(rank) * 4, 256);
  p.off_tfull = off;  // T, [16*NT][rp], fp32 or bf16
  off = align_up(off + size_t(16 * p.NT) * rp * 4, 256);
  p.bytes = off;
  return p;
}

hipError_t launch_forward_decode(const DecodePlan& p, tb_dtype dtype, const void* x, const void* s, const void* w0,
                                 const void* u, const void* v, void* y, int64_t m, int64_t out_dim, int64_t in_dim,
                                 int64_t rank, void* workspace, unsigned epoch, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  DecodeArgs a;
  a.x = x; a.s = s; a.w0 = w0; a.u = u; a.v = v; a.y = y;
  a.M = int(m); a.O = int(out_dim); a.I = int(in_dim); a.R = int(rank);
  a.S = p.S; a.NP = p.NP; a.NB = p.NG;
  a.epoch = epoch;
  a.ctrl = reinterpret_cast<unsigned*>(ws);
  a.tpart = reinterpret_cast<float*>(ws + p.off_tpart);
  a.tfull = reinterpret_cast<float*>(ws + p.off_tfull);
  if (dtype == TB_BF16) return launch_e<bf16_t>(p, a, stream);
  return launch_e<float>(p, a, stream);
}

}  // namespace tb
