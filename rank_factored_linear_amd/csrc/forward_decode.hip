// Fused theta-bundle projection for few tokens (m <= 64): one launch.
//
//   y = s (.) (x . W0^T) + (x . V) . U^T        ("The theta bundle": the
//   transpose of weight = diag(s) W0 + U V^T applied to x)
//
// At these token counts the projection is bound by HBM bandwidth: every byte
// of W0 is read once, and U, V, s once.  Workgroups take a role from a ticket
// counter in the workspace, in the order they start running:
//
//   producers (tickets 0..NP-1) compute T = x . V.  Each first sums its
//     slice of in_dim into a private partial; after all producers arrive
//     (they are all resident, see below) each sums one slice of the M x r
//     outputs over the partials in a fixed order.  The last to finish raises
//     the T-ready flag.
//   consumers (the other tickets) each own 64 output rows and one slice of
//     in_dim.  Four waves stream the W0 rows through v_mfma 16x16x32 (x is the
//     16-token B operand, zero-padded), reduce in LDS in a fixed order, and,
//     when in_dim is split over KS workgroups, the last of the KS to arrive
//     sums the KS partials in slice order.  That workgroup scales each row by
//     s, waits for T, adds T . U^T with the matrix cores and stores y.
//
// Deadlock freedom: a workgroup takes its ticket after it starts running, so
// any consumer that waits for T runs after all NP producer tickets have been
// taken by running workgroups, and producers wait only for each other
// (NP <= compute units / 2, so all of them are resident together).  Every
// wait is bounded (tb::wait_at_least); a timeout sets an error word and
// poisons the output with NaN instead of hanging.
//
// The last workgroup to finish returns every control word to zero, so the
// same workspace serves the next call on the stream.
#include "tb_device.h"
#include "tb_host.h"

namespace tb {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;          // output rows per consumer workgroup
constexpr int kStageRows = 256;    // rows of x staged in LDS per producer pass

enum Ctrl { kTicket = 0, kDone = 1, kArrive1 = 2, kArrive2 = 3, kTReady = 4, kErr = 5 };

struct DecodeArgs {
  const void* x;
  const void* s;
  const void* w0;
  const void* u;
  const void* v;
  void* y;
  int M, O, I, R;
  int NG, KS, S, NP;
  unsigned total;
  unsigned* ctrl;
  unsigned* gcount;
  float* tpart;
  float* tfull;
  float4* ppart;
};

template <typename E>
__device__ void produce_xv(const DecodeArgs& a, int p, int NT, float* smem) {
  const E* X = static_cast<const E*>(a.x);
  const E* V = static_cast<const E*>(a.v);
  const int tid = threadIdx.x;
  const int M = a.M, I = a.I, R = a.R;
  const int i0 = int(int64_t(p) * I / a.NP), i1 = int(int64_t(p + 1) * I / a.NP);
  const int RC = R < kThreads ? R : kThreads;   // columns per pass
  const int PH = kThreads / RC;                 // row phases
  const int jl = tid % RC, ph = tid / RC;
  float* xs = smem;                   // [16][kStageRows]
  float* red = smem + 16 * kStageRows;  // [PH][16][RC]
  float* tp = a.tpart + size_t(p) * M * R;

  for (int tg = 0; tg < NT; ++tg) {
    for (int jc0 = 0; jc0 < R; jc0 += RC) {
      const int j = jc0 + jl;
      float acc[16];
#pragma unroll
      for (int mm = 0; mm < 16; ++mm) acc[mm] = 0.f;
      for (int c0 = i0; c0 < i1; c0 += kStageRows) {
        const int cn = min(kStageRows, i1 - c0);
        for (int idx = tid; idx < 16 * kStageRows; idx += kThreads) {
          const int mm = idx / kStageRows, ii = idx % kStageRows;
          const int tok = tg * 16 + mm;
          xs[idx] = (tok < M && ii < cn) ? to_f32<E>(X[size_t(tok) * I + c0 + ii]) : 0.f;
        }
        __syncthreads();
        if (ph < PH && j < R) {
          for (int ii = ph; ii < cn; ii += PH) {
            const float vj = to_f32<E>(V[size_t(c0 + ii) * R + j]);
#pragma unroll
            for (int mm = 0; mm < 16; ++mm) acc[mm] += xs[mm * kStageRows + ii] * vj;
          }
        }
        __syncthreads();
      }
      if (ph < PH) {
#pragma unroll
        for (int mm = 0; mm < 16; ++mm) red[(ph * 16 + mm) * RC + jl] = acc[mm];
      }
      __syncthreads();
      for (int idx = tid; idx < 16 * RC; idx += kThreads) {
        const int mm = idx / RC, jj = idx % RC;
        float sum = 0.f;
        for (int q = 0; q < PH; ++q) sum += red[(q * 16 + mm) * RC + jj];
        const int tok = tg * 16 + mm;
        if (tok < M && jc0 + jj < R) tp[size_t(tok) * R + jc0 + jj] = sum;
      }
      __syncthreads();
    }
  }

  // All producers' partials complete: reduce one slice of the M x R outputs.
  __threadfence();
  __syncthreads();
  __shared__ unsigned s_ok;
  if (tid == 0) {
    atomic_add_agent(&a.ctrl[kArrive1], 1u);
    const bool ok = wait_at_least(&a.ctrl[kArrive1], unsigned(a.NP));
    if (!ok) atomicOr(&a.ctrl[kErr], 1u);
    s_ok = ok;
  }
  __syncthreads();
  __threadfence();
  const int n = M * R;
  const int q0 = int(int64_t(p) * n / a.NP), q1 = int(int64_t(p + 1) * n / a.NP);
  for (int idx = q0 + tid; idx < q1; idx += kThreads) {
    float sum = 0.f;
    for (int q = 0; q < a.NP; ++q) sum += a.tpart[size_t(q) * n + idx];
    a.tfull[idx] = s_ok ? sum : __builtin_nanf("");
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomic_add_agent(&a.ctrl[kArrive2], 1u);
    if (prev == unsigned(a.NP - 1)) atomic_store_agent(&a.ctrl[kTReady], 1u);
  }
}

template <typename E, int NT, int UNR>
__device__ void consume(const DecodeArgs& a, int c, f32x4* red) {
  const E* X = static_cast<const E*>(a.x);
  const E* W0 = static_cast<const E*>(a.w0);
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int lr = l & 15, kq = (l >> 4) * 8;
  const int M = a.M, O = a.O, I = a.I, R = a.R;
  const int g = c / a.KS, ks = c % a.KS;
  const int o_base = g * kRows;
  const int s_begin = int(int64_t(ks) * a.S / a.KS), s_end = int(int64_t(ks + 1) * a.S / a.KS);

  f32x4 acc[4][NT];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Waves take the k32 steps of the slice round-robin, UNR steps at a time.
  for (int st = s_begin + w; st < s_end; st += 4 * UNR) {
    Frag8<E> fa[UNR][4], fb[UNR][NT];
#pragma unroll
    for (int uu = 0; uu < UNR; ++uu) {
      const int step = st + 4 * uu;
      const int k = step * 32 + kq;
      const bool kv = step < s_end && k < I;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int row = o_base + rt * 16 + lr;
        fa[uu][rt] = load_frag_if<E>(W0 + size_t(row) * I + k, kv && row < O);
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
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[rt][t] = mma_k32(fa[uu][rt], fb[uu][t], acc[rt][t]);
  }

  // Fixed-order reduction of the four waves; wave w keeps row tile w.
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t) red[((w * 4 + rt) * NT + t) * kWave + l] = acc[rt][t];
  __syncthreads();
  f32x4 sum[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    sum[t] = red[((0 * 4 + w) * NT + t) * kWave + l];
    sum[t] += red[((1 * 4 + w) * NT + t) * kWave + l];
    sum[t] += red[((2 * 4 + w) * NT + t) * kWave + l];
    sum[t] += red[((3 * 4 + w) * NT + t) * kWave + l];
  }

  __shared__ unsigned s_flag;
  if (a.KS > 1) {
    float4* slot = a.ppart + (size_t(g * a.KS + ks) * 4 + w) * NT * kWave;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (t * 16 + lr < M) slot[t * kWave + l] = make_float4(sum[t].x, sum[t].y, sum[t].z, sum[t].w);
    __threadfence();
    __syncthreads();
    if (tid == 0) s_flag = (atomic_add_agent(&a.gcount[g], 1u) == unsigned(a.KS - 1));
    __syncthreads();
    if (!s_flag) return;
    __threadfence();
#pragma unroll
    for (int t = 0; t < NT; ++t) sum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < a.KS; ++q) {
      const float4* sl = a.ppart + (size_t(g * a.KS + q) * 4 + w) * NT * kWave;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t * 16 + lr < M) {
          const float4 v4 = sl[t * kWave + l];
          sum[t] += f32x4{v4.x, v4.y, v4.z, v4.w};
        }
      }
    }
    if (tid == 0) atomic_store_agent(&a.gcount[g], 0u);
  }

  // Epilogue: row scale, then the rank-r delta, then one rounding.
  const E* S_ = static_cast<const E*>(a.s);
  const int orow0 = o_base + w * 16 + (l >> 4) * 4;
  float sc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sc[e] = (orow0 + e < O) ? to_f32<E>(S_[orow0 + e]) : 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[t][e] *= sc[e];

  if (R > 0) {
    if (tid == 0) {
      const bool ok = wait_at_least(&a.ctrl[kTReady], 1u);
      if (!ok) atomicOr(&a.ctrl[kErr], 1u);
      s_flag = ok;
    }
    __syncthreads();
    __threadfence();
    const bool ok = s_flag;
    const E* U = static_cast<const E*>(a.u);
    const int urow = o_base + w * 16 + lr;
    const bool aligned = (R % 8) == 0;
    for (int kk = 0; kk < R; kk += 32) {
      const int j = kk + kq;
      Frag8<E> fu = zero_frag<E>();
      if (urow < O && j < R)
        fu = aligned ? load_frag<E>(U + size_t(urow) * R + j) : load_frag_partial<E>(U + size_t(urow) * R + j, min(8, R - j));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int tok = t * 16 + lr;
        float tv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tv[e] = (tok < M && j + e < R) ? a.tfull[size_t(tok) * R + j + e] : 0.f;
        sum[t] = mma_k32(fu, frag_from_f32<E>(tv), sum[t]);
      }
    }
    if (!ok) {
#pragma unroll
      for (int t = 0; t < NT; ++t) sum[t] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
  }

  E* Y = static_cast<E*>(a.y);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = t * 16 + lr;
    if (tok < M) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (orow0 + e < O) Y[size_t(tok) * O + orow0 + e] = from_f32<E>(sum[t][e]);
    }
  }
}

template <typename E, int NT>
__global__ __launch_bounds__(kThreads) void forward_decode_kernel(DecodeArgs a) {
  constexpr int kConsumerLds = 4 * 4 * NT * kWave * 16;           // bytes
  constexpr int kProducerLds = (16 * kStageRows + 16 * kThreads) * 4;
  constexpr int kLds = kConsumerLds > kProducerLds ? kConsumerLds : kProducerLds;
  __shared__ float4 smem[kLds / 16];
  __shared__ unsigned s_ticket;
  if (threadIdx.x == 0) s_ticket = atomic_add_agent(&a.ctrl[kTicket], 1u);
  __syncthreads();
  const unsigned ticket = s_ticket;
  if (ticket < unsigned(a.NP)) {
    produce_xv<E>(a, int(ticket), NT, reinterpret_cast<float*>(smem));
  } else {
    constexpr int UNR = sizeof(E) == 2 ? 4 : 2;
    consume<E, NT, UNR>(a, int(ticket - a.NP), reinterpret_cast<f32x4*>(smem));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomic_add_agent(&a.ctrl[kDone], 1u);
    if (prev == a.total - 1) {
      atomic_store_agent(&a.ctrl[kTicket], 0u);
      atomic_store_agent(&a.ctrl[kArrive1], 0u);
      atomic_store_agent(&a.ctrl[kArrive2], 0u);
      atomic_store_agent(&a.ctrl[kTReady], 0u);
      atomic_store_agent(&a.ctrl[kDone], 0u);
    }
  }
}

template <typename E, int NT>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((forward_decode_kernel<E, NT>), dim3(a.total), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, int cus) {
  DecodePlan p{};
  p.NT = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
  p.NG = int((out_dim + kRows - 1) / kRows);
  p.S = int((in_dim + 31) / 32);
  const int target = 8 * cus;
  int ks = 1;
  if (p.NG < target) {
    ks = (target + p.NG - 1) / p.NG;
    const int max_ks = p.S / 4 > 1 ? p.S / 4 : 1;
    if (ks > max_ks) ks = max_ks;
  }
  if (ks > 1 && p.NG > kMaxGroupCounters) ks = 1;
  p.KS = ks;
  if (rank > 0) {
    int np = int((in_dim + 31) / 32);
    if (np > 128) np = 128;
    if (np > cus / 2) np = cus / 2;
    if (np < 1) np = 1;
    p.NP = np;
  } else {
    p.NP = 0;
  }
  size_t off = kControlBytes;
  p.off_tpart = off;
  off = align_up(off + size_t(p.NP) * size_t(m) * size_t(rank) * 4, 256);
  p.off_tfull = off;
  off = align_up(off + size_t(m) * size_t(rank) * 4, 256);
  p.off_ppart = off;
  if (p.KS > 1) off = align_up(off + size_t(p.NG) * p.KS * 4 * p.NT * kWave * 16, 256);
  p.bytes = off;
  return p;
}

hipError_t launch_forward_decode(const DecodePlan& p, tb_dtype dtype, const void* x, const void* s, const void* w0,
                                 const void* u, const void* v, void* y, int64_t m, int64_t out_dim, int64_t in_dim,
                                 int64_t rank, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  DecodeArgs a;
  a.x = x; a.s = s; a.w0 = w0; a.u = u; a.v = v; a.y = y;
  a.M = int(m); a.O = int(out_dim); a.I = int(in_dim); a.R = int(rank);
  a.NG = p.NG; a.KS = p.KS; a.S = p.S; a.NP = p.NP;
  a.total = unsigned(p.NP + p.NG * p.KS);
  a.ctrl = reinterpret_cast<unsigned*>(ws);
  a.gcount = reinterpret_cast<unsigned*>(ws + 256);
  a.tpart = reinterpret_cast<float*>(ws + p.off_tpart);
  a.tfull = reinterpret_cast<float*>(ws + p.off_tfull);
  a.ppart = reinterpret_cast<float4*>(ws + p.off_ppart);
  if (dtype == TB_BF16) {
    if (p.NT == 1) return launch_t<bf16_t, 1>(a, stream);
    if (p.NT == 2) return launch_t<bf16_t, 2>(a, stream);
    return launch_t<bf16_t, 4>(a, stream);
  }
  if (p.NT == 1) return launch_t<float, 1>(a, stream);
  if (p.NT == 2) return launch_t<float, 2>(a, stream);
  return launch_t<float, 4>(a, stream);
}

}  // namespace tb
