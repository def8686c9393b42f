// Analytic decomposition of one projection family into its theta bundle on
// the GPU ("The theta bundle", section "Analytic decomposition"):
//
//   shared block   W0 = mean of the band's weight matrices
//   per-row scale  s[o] = <W[o], W0[o]> / <W0[o], W0[o]>  (0 for a zero row)
//   low-rank       U, V from the randomized SVD (Halko, Martinsson and Tropp,
//                  2009) of the residual W - diag(s) W0, U absorbing the
//                  singular values.
//
// The residual's randomized SVD, for a caller-drawn probe Omega [in, k]:
//   Y = E Omega, Q = basis(Y); power_iters times: Q' = basis(E^T Q),
//   Q = basis(E Q'); B^T = E^T Q; the eigen-decomposition of B B^T = P L P^T
//   gives B = P diag(sigma) Qt with sigma = sqrt(L); U = Q P_r diag(sigma_r),
//   V = B^T P_r diag(1 / sigma_r).
// basis() is CholeskyQR: the fp64 Gram matrix of the columns, a Cholesky
// factor R whose pivots at or below 1e-13 of the largest diagonal entry mark
// directions the columns do not span (their columns of Q are zero), and
// Q = Y R^-1; one round between power iterations, two (CholeskyQR2) for the
// final basis.  The same span as a Householder QR, so the same U V^T up to
// rounding.  The eigenvectors of B B^T are the right singular vectors of its
// Cholesky factor, found by one-sided Jacobi (fp64, round-robin pair order).
// The large products and the triangular solves run as plain fp32 rocBLAS
// calls; the Gram matrices, the Cholesky factor and the Jacobi SVD are the
// kernels below.
#include <rocblas/rocblas.h>

#include <mutex>
#include <vector>

#include "tb_device.h"
#include "tb_host.h"
#include "tb_reduce.h"

namespace tb {

namespace {

constexpr int kThreads = 256;
constexpr int kSolverThreads = 1024;
static_assert(TB_MAX_PROBE <= kSolverThreads, "a thread per pair and per column");
constexpr double kPivotTol = 1e-13;     // Cholesky pivot / largest diagonal entry below which a direction is dropped
constexpr double kSigmaTol = 1e-14;     // eigenvalue / largest below which a singular value counts as zero
// A sweep that sees no |gamma| / sqrt(alpha beta) above kJacobiTol ends the
// iteration.  The factors leave in fp32, so columns orthogonal to 1e-11 are
// plenty, and the rounding floor of a length-k fp64 dot product of two
// orthogonal columns (~k * 1e-16 <= 5e-14) stays well below it.
constexpr double kJacobiTol = 1e-11;
constexpr int kMaxSweeps = 40;
constexpr int kGramTile = 64;
constexpr int kGramRows = 32;           // rows of the input per LDS stage

// ---- shared block ------------------------------------------------------------

struct BandPtrs {
  const void* w[TB_MAX_BAND_LAYERS];
};

// Sum in layer order in fp64, divide by the count, round once to fp32.
template <typename E>
__global__ __launch_bounds__(kThreads) void shared_block_kernel(BandPtrs bp, int n, int64_t count, float* out) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < count; i += stride) {
    double total = 0.0;
    for (int j = 0; j < n; ++j) total = total + double(to_f32<E>(static_cast<const E*>(bp.w[j])[i]));
    out[i] = float(total / double(n));
  }
}

// ---- per-row scale -------------------------------------------------------------

// One workgroup per row: fp64 dot products in a fixed order.
template <typename E>
__global__ __launch_bounds__(kThreads) void row_scale_kernel(const E* __restrict__ w, const float* __restrict__ w0,
                                                             int64_t I, float* __restrict__ s) {
  __shared__ double sa[kThreads], sb[kThreads];
  const int64_t o = blockIdx.x;
  const E* wr = w + o * I;
  const float* w0r = w0 + o * I;
  double num = 0.0, den = 0.0;
  for (int64_t i = threadIdx.x; i < I; i += kThreads) {
    const double a = to_f32<E>(wr[i]), b = w0r[i];
    num += a * b;
    den += b * b;
  }
  reduce::block_reduce2<kThreads>(num, den, sa, sb);
  if (threadIdx.x == 0) s[o] = den != 0.0 ? float(num / den) : 0.f;
}

// ---- batches ------------------------------------------------------------------------
//
// tb_lowrank_factors works on a batch of matrices of one shape.  Each matrix
// has a workspace slice of its own (`stride` bytes apart): the kernels below
// take the batch's first pointer into the workspace and the stride, and a
// grid dimension for the batch index.

template <typename T>
__device__ __forceinline__ T* at_batch(T* p, int64_t stride, int b) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(p) + stride * b);
}
template <typename T>
__device__ __forceinline__ const T* at_batch(const T* p, int64_t stride, int b) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(p) + stride * b);
}

struct WeightPtrs {
  const void* w[TB_MAX_BAND_LAYERS];
  const float* w0[TB_MAX_BAND_LAYERS];
};

// ---- residual --------------------------------------------------------------------

// E = W - diag(s) W0 in fp32, one rounding (fma) per entry.  grid (column
// blocks, row blocks, batch), the first two grid-stride; s is [batch][O].
template <typename E>
__global__ __launch_bounds__(kThreads) void residual_kernel(WeightPtrs wp, const float* __restrict__ s0, int64_t O,
                                                            int64_t I, float* __restrict__ e0, int64_t stride) {
  const int b = blockIdx.z;
  const E* __restrict__ w = static_cast<const E*>(wp.w[b]);
  const float* __restrict__ w0 = wp.w0[b];
  const float* __restrict__ s = s0 + int64_t(b) * O;
  float* __restrict__ e = at_batch(e0, stride, b);
  for (int64_t o = blockIdx.y; o < O; o += gridDim.y) {
    const float so = s[o];
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < I; i += int64_t(gridDim.x) * kThreads) {
      const int64_t at = o * I + i;
      e[at] = fmaf(-so, w0[at], to_f32<E>(w[at]));
    }
  }
}

// ---- least-squares refit of a shared block (alternating least squares) -------------
//
// W0[o] = sum_l s_l[o] (W_l - U_l V_l^T)[o] / sum_l s_l[o]^2, as
//   num = sum_l diag(s_l) W_l             (scaled_sum_kernel, fp64 sums in layer order)
//   num -= [s_1 U_1 | ... | s_n U_n] [V_1 | ... | V_n]^T   (one GEMM, inner dimension n r)
//   W0 = num / den, den[o] = sum_l s_l[o]^2, or the previous row where den is 0.

struct RefinePtrs {
  const void* w[TB_MAX_BAND_LAYERS];
  const float* s[TB_MAX_BAND_LAYERS];
};

template <typename E>
__global__ __launch_bounds__(kThreads) void scaled_sum_kernel(RefinePtrs rp, int n, int64_t O, int64_t I,
                                                              float* __restrict__ num) {
  const int64_t count = O * I, stride = int64_t(gridDim.x) * kThreads;
  for (int64_t at = int64_t(blockIdx.x) * kThreads + threadIdx.x; at < count; at += stride) {
    const int64_t o = at / I;
    double acc = 0.0;
    for (int l = 0; l < n; ++l) acc += double(rp.s[l][o]) * double(to_f32<E>(static_cast<const E*>(rp.w[l])[at]));
    num[at] = float(acc);
  }
}

// Ucat [O][n r] = s_l[o] U_l[o][j] at column l r + j; Vcat [I][n r] = V_l[i][j].
struct FactorPtrs {
  const float* u[TB_MAX_BAND_LAYERS];
  const float* v[TB_MAX_BAND_LAYERS];
  const float* s[TB_MAX_BAND_LAYERS];
};

__global__ __launch_bounds__(kThreads) void pack_factors_kernel(FactorPtrs fp, int n, int64_t O, int64_t I, int r,
                                                                float* __restrict__ ucat, float* __restrict__ vcat) {
  const int64_t nr = int64_t(n) * r, total = (O + I) * nr, stride = int64_t(gridDim.x) * kThreads;
  for (int64_t at = int64_t(blockIdx.x) * kThreads + threadIdx.x; at < total; at += stride) {
    const int64_t row = at / nr, c = at % nr;
    const int l = int(c / r), j = int(c % r);
    if (row < O) ucat[at] = fp.s[l][row] * fp.u[l][row * r + j];
    else vcat[at - O * nr] = fp.v[l][(row - O) * r + j];
  }
}

__global__ __launch_bounds__(kThreads) void refine_finish_kernel(RefinePtrs rp, int n, int64_t O, int64_t I,
                                                                 const float* __restrict__ num,
                                                                 const float* __restrict__ prev,
                                                                 float* __restrict__ out) {
  for (int64_t o = blockIdx.y; o < O; o += gridDim.y) {
    double den = 0.0;
    for (int l = 0; l < n; ++l) den += double(rp.s[l][o]) * double(rp.s[l][o]);
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < I; i += int64_t(gridDim.x) * kThreads)
      out[o * I + i] = den != 0.0 ? float(double(num[o * I + i]) / den) : prev[o * I + i];
  }
}

// ---- Gram matrix C = A^T A (fp64) -------------------------------------------------

// Upper tile (ta <= tb) number `t` of a T x T tile grid.
__device__ __forceinline__ void upper_tile(int t, int T, int& ta, int& tb) {
  int a = 0;
  while (t >= T - a) {
    t -= T - a;
    ++a;
  }
  ta = a;
  tb = a + t;
}

// Workgroup (tile, split) sums rows [split * rows_per, ...) of A [n, k]
// (row-major fp32) into the 64 x 64 tile (ta, tb) of part[split] (fp64).
// Thread (ty, tx) of 16 x 16 holds outputs (ta*64 + 4ty + i, tb*64 + 4tx + j).
__global__ __launch_bounds__(kThreads) void gram_partial_kernel(const float* __restrict__ A0, int64_t n, int k,
                                                                int64_t rows_per, double* __restrict__ part0,
                                                                int64_t stride) {
  __shared__ float as[kGramRows][kGramTile], bs[kGramRows][kGramTile];
  const float* __restrict__ A = at_batch(A0, stride, blockIdx.z);
  double* __restrict__ part = at_batch(part0, stride, blockIdx.z);
  const int T = (k + kGramTile - 1) / kGramTile;
  int ta, tb;
  upper_tile(blockIdx.x, T, ta, tb);
  const int split = blockIdx.y;
  const int64_t r0 = int64_t(split) * rows_per, r1 = r0 + rows_per < n ? r0 + rows_per : n;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int a0 = ta * kGramTile, b0 = tb * kGramTile;
  double acc[4][4] = {};
  for (int64_t r = r0; r < r1; r += kGramRows) {
#pragma unroll
    for (int q = 0; q < kGramRows * kGramTile / kThreads; ++q) {
      const int idx = q * kThreads + tid, rr = idx / kGramTile, cc = idx % kGramTile;
      const int64_t row = r + rr;
      const bool in = row < r1;
      as[rr][cc] = in && a0 + cc < k ? A[row * k + a0 + cc] : 0.f;
      bs[rr][cc] = in && b0 + cc < k ? A[row * k + b0 + cc] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < kGramRows; ++rr) {
      double va[4], vb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        va[i] = as[rr][4 * ty + i];
        vb[i] = bs[rr][4 * tx + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += va[i] * vb[j];
    }
    __syncthreads();
  }
  double* P = part + size_t(split) * k * k;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int a = a0 + 4 * ty + i, b = b0 + 4 * tx + j;
      if (a < k && b < k) P[size_t(a) * k + b] = acc[i][j];
    }
}

// C[a][b] = sum over splits, in split order, of the upper tile holding (a, b)
// or (b, a): C is exactly symmetric.
__global__ __launch_bounds__(kThreads) void gram_reduce_kernel(const double* __restrict__ part0, int k, int splits,
                                                               double* __restrict__ C0, int64_t stride) {
  const double* __restrict__ part = at_batch(part0, stride, blockIdx.y);
  double* __restrict__ C = at_batch(C0, stride, blockIdx.y);
  const int64_t kk = int64_t(k) * k;
  for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < kk; idx += int64_t(gridDim.x) * kThreads) {
    const int a = int(idx / k), b = int(idx % k);
    const bool upper = a / kGramTile <= b / kGramTile;
    const size_t at = upper ? size_t(a) * k + b : size_t(b) * k + a;
    double sum = 0.0;
    for (int sp = 0; sp < splits; ++sp) sum += part[size_t(sp) * kk + at];
    C[idx] = sum;
  }
}

// ---- Cholesky factor (one workgroup, fp64) ------------------------------------------

// C = R^T R (R upper), right-looking, row j of the trailing matrix staged in
// LDS.  A pivot at or below kPivotTol of the largest diagonal entry of C
// drops direction j: row j and column j of R become those of the identity,
// and dropped[j] = 1 (the caller zeroes column j of the input, so that the
// triangular solve gives a zero column of Q and leaves the others alone).
// R32 = R in fp32 (k x k, row-major, zero below the diagonal).  A: k x k scratch.
__global__ __launch_bounds__(kSolverThreads) void cholesky_kernel(const double* __restrict__ C0, int k,
                                                                  double* __restrict__ A0, int* __restrict__ dropped0,
                                                                  float* __restrict__ R320, int64_t stride) {
  const double* __restrict__ C = at_batch(C0, stride, blockIdx.x);
  double* __restrict__ A = at_batch(A0, stride, blockIdx.x);
  int* __restrict__ dropped = at_batch(dropped0, stride, blockIdx.x);
  float* __restrict__ R32 = at_batch(R320, stride, blockIdx.x);
  __shared__ double s_row[TB_MAX_PROBE];
  __shared__ double s_piv, s_max;
  __shared__ int s_drop;
  const int tid = threadIdx.x;
  const int kk = k * k;
  for (int i = tid; i < kk; i += kSolverThreads) A[i] = C[i];
  if (tid == 0) {
    double m = 0.0;
    for (int j = 0; j < k; ++j) m = fmax(m, C[size_t(j) * k + j]);
    s_max = m;
  }
  __syncthreads();
  for (int j = 0; j < k; ++j) {
    if (tid == 0) {
      const double d = A[size_t(j) * k + j];
      const bool drop = !(d > kPivotTol * s_max);
      s_drop = drop;
      s_piv = drop ? 1.0 : sqrt(d);
      dropped[j] = drop;
    }
    __syncthreads();
    const double piv = s_piv;
    const bool drop = s_drop;
    for (int l = j + tid; l < k; l += kSolverThreads) {
      const double v = l == j ? piv : (drop ? 0.0 : A[size_t(j) * k + l] / piv);
      s_row[l] = v;
      A[size_t(j) * k + l] = v;
    }
    __syncthreads();
    if (!drop) {
      const int n = k - j - 1;
      // Trailing update of the upper triangle, four independent entries per
      // thread in flight.
      constexpr int B = 4;
      for (int base = tid; base < n * n; base += B * kSolverThreads) {
        int at[B];
        double val[B], mul[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
          const int idx = base + u * kSolverThreads;
          const int l = j + 1 + idx / n, m = j + 1 + idx % n;
          const bool live = idx < n * n && m >= l;
          at[u] = live ? l * k + m : -1;
          val[u] = live ? A[size_t(l) * k + m] : 0.0;
          mul[u] = live ? s_row[l] * s_row[m] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < B; ++u)
          if (at[u] >= 0) A[at[u]] = val[u] - mul[u];
      }
    }
    __syncthreads();
  }
  // R32: the upper triangle of A; a dropped direction's column is the identity's.
  for (int i = tid; i < kk; i += kSolverThreads) {
    const int r = i / k, c = i % k;
    float v = 0.f;
    if (c >= r && !(dropped[c] && r != c)) v = float(A[i]);
    R32[i] = v;
  }
}

// Zero the columns of X [n, k] whose direction the Cholesky factor dropped.
__global__ __launch_bounds__(kThreads) void zero_dropped_kernel(float* __restrict__ X0, int64_t n, int k,
                                                                const int* __restrict__ dropped0, int64_t stride) {
  float* __restrict__ X = at_batch(X0, stride, blockIdx.y);
  const int* __restrict__ dropped = at_batch(dropped0, stride, blockIdx.y);
  const int64_t total = n * k;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total; i += int64_t(gridDim.x) * kThreads)
    if (dropped[i % k]) X[i] = 0.f;
}

// ---- singular value decomposition of the Cholesky factor (one workgroup, fp64) ---------

// Sum over an aligned group of G lanes.
template <int G>
__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
  for (int m = G / 2; m > 0; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// B B^T = R^T R (R from cholesky_kernel, its dropped rows taken as zero), so
// the eigenvectors of B B^T are the right singular vectors of R.  One-sided
// (Hestenes) Jacobi on the columns of R: each sweep runs the kk - 1 rounds of
// the round-robin (circle) pair order over kk = k rounded up to even, so that
// every pair (p, q) meets once per sweep and the pairs of a round are
// disjoint; a group of G lanes per pair forms alpha = |r_p|^2, beta = |r_q|^2,
// gamma = r_p . r_q and rotates columns p, q of R and of V (J_pp = J_qq = c,
// J_pq = s, J_qp = -s, chosen to make the new columns orthogonal).  Columns
// are stored contiguously (Rc, Vc: column j at j * k), so every access is a
// whole column.  Ends when a whole sweep saw no |gamma| / sqrt(alpha beta)
// above kJacobiTol.  On exit lam[j] = |column j of R V|^2 (the eigenvalues),
// perm the columns by decreasing lam (ties by index), sweeps[0] the sweeps.
template <int G, int kPer>
__global__ __launch_bounds__(kSolverThreads) void jacobi_kernel(const double* __restrict__ Rrow0,
                                                                const int* __restrict__ dropped0, int k,
                                                                double* __restrict__ Rc0, double* __restrict__ Vc0,
                                                                double* __restrict__ lam0, int* __restrict__ perm0,
                                                                int* __restrict__ sweeps0, int64_t stride) {
  const int bt = blockIdx.x;
  const double* __restrict__ Rrow = at_batch(Rrow0, stride, bt);
  const int* __restrict__ dropped = at_batch(dropped0, stride, bt);
  double* __restrict__ Rc = at_batch(Rc0, stride, bt);
  double* __restrict__ Vc = at_batch(Vc0, stride, bt);
  double* __restrict__ lam = at_batch(lam0, stride, bt);
  int* __restrict__ perm = at_batch(perm0, stride, bt);
  int* __restrict__ sweeps = at_batch(sweeps0, stride, bt);
  constexpr int kWavesJ = kSolverThreads / kWave;
  constexpr int kGroups = kSolverThreads / G;                // pairs in flight
  __shared__ double s_red[kWavesJ];
  __shared__ int s_done;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int grp = tid / G, lg = tid % G;
  const int kk = k + (k & 1), P = kk / 2;
  for (int idx = tid; idx < k * k; idx += kSolverThreads) {
    const int j = idx / k, i = idx % k;   // column j, row i
    Rc[idx] = (i <= j && !dropped[i]) ? Rrow[size_t(i) * k + j] : 0.0;
    Vc[idx] = i == j ? 1.0 : 0.0;
  }
  __syncthreads();
  int sweep = 0;
  for (; sweep < kMaxSweeps; ++sweep) {
    double off = 0.0;
    for (int t = 0; t < kk - 1; ++t) {
      for (int pr = grp; pr < P; pr += kGroups) {
        const int a = pr == 0 ? 0 : ((pr - 1 + t) % (kk - 1)) + 1, b = ((kk - 2 - pr + t) % (kk - 1)) + 1;
        const int p = a < b ? a : b, q = a < b ? b : a;
        if (q >= k) continue;
        double* cp = Rc + size_t(p) * k;
        double* cq = Rc + size_t(q) * k;
        double* vp = Vc + size_t(p) * k;
        double* vq = Vc + size_t(q) * k;
        double xp[kPer], xq[kPer], yp[kPer], yq[kPer];
        double al = 0.0, be = 0.0, ga = 0.0;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          const int i = lg + e * G;
          const bool in = i < k;
          xp[e] = in ? cp[i] : 0.0;
          xq[e] = in ? cq[i] : 0.0;
          yp[e] = in ? vp[i] : 0.0;
          yq[e] = in ? vq[i] : 0.0;
        }
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          al += xp[e] * xp[e];
          be += xq[e] * xq[e];
          ga += xp[e] * xq[e];
        }
        al = group_sum<G>(al);
        be = group_sum<G>(be);
        ga = group_sum<G>(ga);
        const double d = sqrt(al * be);
        if (d > 0.0) off = fmax(off, fabs(ga) / d);
        if (ga == 0.0 || !(fabs(ga) > 1e-16 * d)) continue;
        const double z = (be - al) / (2.0 * ga);
        const double tt = z == 0.0            ? 1.0
                          : fabs(z) > 1e150 ? 0.5 / z
                                            : copysign(1.0, z) / (fabs(z) + sqrt(z * z + 1.0));
        const double c = 1.0 / sqrt(tt * tt + 1.0), sn = tt * c;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          const int i = lg + e * G;
          if (i < k) {
            cp[i] = c * xp[e] - sn * xq[e];
            cq[i] = sn * xp[e] + c * xq[e];
            vp[i] = c * yp[e] - sn * yq[e];
            vq[i] = sn * yp[e] + c * yq[e];
          }
        }
      }
      __syncthreads();
    }
    if (l == 0) s_red[w] = off;
    __syncthreads();
    if (tid == 0) {
      double m = 0.0;
      for (int i = 0; i < kWavesJ; ++i) m = fmax(m, s_red[i]);
      s_done = m <= kJacobiTol;
    }
    __syncthreads();
    if (s_done) {
      ++sweep;
      break;
    }
  }
  for (int j = w; j < k; j += kWavesJ) {
    double n2 = 0.0;
    for (int i = l; i < k; i += kWave) n2 += Rc[size_t(j) * k + i] * Rc[size_t(j) * k + i];
    n2 = group_sum<kWave>(n2);
    if (l == 0) lam[j] = n2;
  }
  __syncthreads();
  for (int j = tid; j < k; j += kSolverThreads) {
    const double lj = lam[j];
    int r = 0;
    for (int i = 0; i < k; ++i) r += (lam[i] > lj || (lam[i] == lj && i < j)) ? 1 : 0;
    perm[r] = j;
  }
  if (tid == 0) sweeps[0] = sweep;
}

// Mu = P_r diag(sigma_r), Mv = P_r diag(1 / sigma_r) (fp32, k x r), sigma_j =
// sqrt of the j-th largest eigenvalue, P's columns stored contiguously (Vc);
// a singular value at or below sqrt(kSigmaTol) of the largest counts as zero
// (zero columns in both).
__global__ __launch_bounds__(kThreads) void assemble_kernel(const double* __restrict__ V0, const double* __restrict__ lam0,
                                                            const int* __restrict__ perm0, int k, int r,
                                                            float* __restrict__ Mu0, float* __restrict__ Mv0,
                                                            int64_t stride) {
  const int bt = blockIdx.y;
  const double* __restrict__ V = at_batch(V0, stride, bt);
  const double* __restrict__ lam = at_batch(lam0, stride, bt);
  const int* __restrict__ perm = at_batch(perm0, stride, bt);
  float* __restrict__ Mu = at_batch(Mu0, stride, bt);
  float* __restrict__ Mv = at_batch(Mv0, stride, bt);
  const double lmax = lam[perm[0]];
  for (int idx = blockIdx.x * kThreads + threadIdx.x; idx < k * r; idx += gridDim.x * kThreads) {
    const int a = idx / r, j = idx % r;
    const int col = perm[j];
    const double l = lam[col];
    const bool zero = !(l > kSigmaTol * lmax) || !(lmax > 0.0);
    const double sg = zero ? 0.0 : sqrt(l);
    const double v = V[size_t(col) * k + a];
    Mu[idx] = zero ? 0.f : float(v * sg);
    Mv[idx] = zero ? 0.f : float(v / sg);
  }
}

// ---- host side ------------------------------------------------------------------------

// One rocBLAS handle per (device, stream): a handle's internal workspace
// (the triangular solve keeps inverted diagonal blocks there) must not be
// shared by calls that run at the same time on different streams.
struct Blas {
  std::mutex mu;
  struct Entry {
    int dev;
    hipStream_t stream;
    rocblas_handle h;
  };
  std::vector<Entry> handles;
};
Blas g_blas;

// The handle of (dev, stream), created on first use; the caller holds g_blas.mu.
rocblas_handle handle_for(int dev, hipStream_t stream) {
  for (const auto& e : g_blas.handles)
    if (e.dev == dev && e.stream == stream) return e.h;
  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success) return nullptr;
  g_blas.handles.push_back({dev, stream, h});
  return h;
}

// Row-major C [M x N] = op(A) op(B) with A [M x K] (or [K x M] when ta) and
// B [K x N] (or [N x K] when tb): the column-major product C^T = op(B)^T op(A)^T.
rocblas_status gemm_rm(rocblas_handle h, bool ta, bool tb, int M, int N, int K, const float* A, int lda,
                       const float* B, int ldb, float* C, int ldc) {
  const float one = 1.f, zero = 0.f;
  return rocblas_sgemm(h, tb ? rocblas_operation_transpose : rocblas_operation_none,
                       ta ? rocblas_operation_transpose : rocblas_operation_none, N, M, K, &one, B, ldb, A, lda, &zero,
                       C, ldc);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int gram_splits(int64_t n, int k, int cus) {
  const int T = (k + kGramTile - 1) / kGramTile, tiles = T * (T + 1) / 2;
  int64_t want = (2 * int64_t(cus) + tiles - 1) / tiles;
  const int64_t by_rows = (n + 255) / 256;
  if (want > by_rows) want = by_rows;
  if (want > 32) want = 32;
  return want < 1 ? 1 : int(want);
}

struct Layout {
  size_t e, o1, i1, part, c, a, v, m, lam, perm, drop, sweeps, mu, mv, total;
};

Layout layout(int64_t O, int64_t I, int64_t k, int64_t r, int cus) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  const int64_t nmax = O > I ? O : I;
  const int splits = gram_splits(nmax, int(k), cus);
  L.e = take(size_t(O) * I * 4);
  L.o1 = take(size_t(O) * k * 4);
  L.i1 = take(size_t(I) * k * 4);
  L.part = take(size_t(splits) * k * k * 8);
  L.c = take(size_t(k) * k * 8);
  L.a = take(size_t(k) * k * 8);
  L.v = take(size_t(k) * k * 8);
  L.m = take(size_t(k) * k * 4);
  L.lam = take(size_t(k) * 8);
  L.perm = take(size_t(k) * 4);
  L.drop = take(size_t(k) * 4);
  L.sweeps = take(4);
  L.mu = take(size_t(k) * (r > 0 ? r : 1) * 4);
  L.mv = take(size_t(k) * (r > 0 ? r : 1) * 4);
  L.total = off;
  return L;
}

struct Run {
  char* ws;   // the first matrix's workspace slice; slice b at ws + b * L.total
  Layout L;
  int k, cus, n;
  hipStream_t stream;
  rocblas_handle h;
  int64_t stride() const { return int64_t(L.total); }
  int64_t fstride() const { return int64_t(L.total / 4); }   // in floats (L.total is a multiple of 256)
  template <typename T>
  T* at(size_t off) const {
    return reinterpret_cast<T*>(ws + off);
  }
};

// Row-major strided-batched C [M x N] = op(A) op(B) (see gemm_rm).
rocblas_status gemm_rm_batched(const Run& R, bool ta, bool tb, int M, int N, int K, const float* A, int lda,
                               int64_t sa, const float* B, int ldb, int64_t sb, float* C, int ldc, int64_t sc) {
  const float one = 1.f, zero = 0.f;
  return rocblas_sgemm_strided_batched(R.h, tb ? rocblas_operation_transpose : rocblas_operation_none,
                                       ta ? rocblas_operation_transpose : rocblas_operation_none, N, M, K, &one, B,
                                       ldb, sb, A, lda, sa, &zero, C, ldc, sc, R.n);
}

// C = A^T A for A [rows, k] fp32, every matrix of the batch (A, C at workspace offsets).
hipError_t gram(const Run& R, size_t off_a, int64_t rows, size_t off_c) {
  const int k = R.k, T = (k + kGramTile - 1) / kGramTile, tiles = T * (T + 1) / 2;
  const int splits = gram_splits(rows, k, R.cus);
  const int64_t rows_per = (rows + splits - 1) / splits;
  hipLaunchKernelGGL(gram_partial_kernel, dim3(unsigned(tiles), unsigned(splits), unsigned(R.n)), dim3(kThreads), 0,
                     R.stream, R.at<const float>(off_a), rows, k, rows_per, R.at<double>(R.L.part), R.stride());
  const int64_t kk = int64_t(k) * k;
  const unsigned blocks = unsigned((kk + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(gram_reduce_kernel, dim3(blocks, unsigned(R.n)), dim3(kThreads), 0, R.stream,
                     R.at<const double>(R.L.part), k, splits, R.at<double>(off_c), R.stride());
  return hipGetLastError();
}

// X [rows, k] (workspace offset off_x) <- a basis of its columns by `passes`
// rounds of CholeskyQR (Gram matrix, Cholesky factor R, X <- X R^-1 by a
// triangular solve in place).  One round leaves the columns well
// conditioned (enough between power iterations); two make them orthonormal
// to working precision.
int orthonormalize(const Run& R, size_t off_x, int64_t rows, int passes, const char** what) {
  for (int pass = 0; pass < passes; ++pass) {
    if (hipError_t e = gram(R, off_x, rows, R.L.c)) {
      *what = "Gram matrix";
      return int(e);
    }
    hipLaunchKernelGGL(cholesky_kernel, dim3(unsigned(R.n)), dim3(kSolverThreads), 0, R.stream,
                       R.at<const double>(R.L.c), R.k, R.at<double>(R.L.a), R.at<int>(R.L.drop), R.at<float>(R.L.m),
                       R.stride());
    int64_t blocks = (rows * R.k + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_dropped_kernel, dim3(unsigned(blocks), unsigned(R.n)), dim3(kThreads), 0, R.stream,
                       R.at<float>(off_x), rows, R.k, R.at<const int>(R.L.drop), R.stride());
    if (hipError_t e = hipGetLastError()) {
      *what = "Cholesky factor";
      return int(e);
    }
    // Row-major X [rows, k] is column-major X^T [k, rows]; row-major R
    // (upper) is column-major R^T (lower): solve R^T Z = X^T, Z = (X R^-1)^T.
    const float one = 1.f;
    if (rocblas_strsm_strided_batched(R.h, rocblas_side_left, rocblas_fill_lower, rocblas_operation_none,
                                      rocblas_diagonal_non_unit, R.k, int(rows), &one, R.at<const float>(R.L.m), R.k,
                                      R.fstride(), R.at<float>(off_x), R.k, R.fstride(), R.n) != rocblas_status_success) {
      *what = "rocblas_strsm (basis)";
      return -1;
    }
  }
  return 0;
}

}  // namespace

hipError_t launch_shared_block(tb_dtype dtype, const void* const* weights, int n, int64_t count, float* out,
                               hipStream_t stream) {
  BandPtrs bp{};
  for (int j = 0; j < n; ++j) bp.w[j] = weights[j];
  int64_t blocks = (count + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  if (dtype == TB_BF16)
    hipLaunchKernelGGL(shared_block_kernel<bf16_t>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, bp, n, count,
                       out);
  else
    hipLaunchKernelGGL(shared_block_kernel<float>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, bp, n, count, out);
  return hipGetLastError();
}

hipError_t launch_row_scale(tb_dtype dtype, const void* weight, const float* w0, int64_t O, int64_t I, float* s,
                            hipStream_t stream) {
  if (dtype == TB_BF16)
    hipLaunchKernelGGL(row_scale_kernel<bf16_t>, dim3(unsigned(O)), dim3(kThreads), 0, stream,
                       static_cast<const bf16_t*>(weight), w0, I, s);
  else
    hipLaunchKernelGGL(row_scale_kernel<float>, dim3(unsigned(O)), dim3(kThreads), 0, stream,
                       static_cast<const float*>(weight), w0, I, s);
  return hipGetLastError();
}

size_t refine_workspace_bytes(int64_t O, int64_t I, int64_t n, int64_t r) {
  return align256(size_t(O) * I * 4) + align256(size_t(O) * n * r * 4) + align256(size_t(I) * n * r * 4);
}

int launch_refine_shared_block(tb_dtype dtype, const void* const* weights, const float* const* s,
                               const float* const* u, const float* const* v, int n, int64_t O, int64_t I, int64_t r,
                               const float* prev, float* out, void* workspace, hipStream_t stream, const char** what) {
  char* ws = static_cast<char*>(workspace);
  float* num = reinterpret_cast<float*>(ws);
  float* ucat = reinterpret_cast<float*>(ws + align256(size_t(O) * I * 4));
  float* vcat = reinterpret_cast<float*>(ws + align256(size_t(O) * I * 4) + align256(size_t(O) * n * r * 4));
  RefinePtrs rp{};
  FactorPtrs fp{};
  for (int j = 0; j < n; ++j) {
    rp.w[j] = weights[j];
    rp.s[j] = fp.s[j] = s[j];
    fp.u[j] = u ? u[j] : nullptr;
    fp.v[j] = v ? v[j] : nullptr;
  }
  int64_t blocks = (O * I + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  if (dtype == TB_BF16)
    hipLaunchKernelGGL(scaled_sum_kernel<bf16_t>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, rp, n, O, I, num);
  else
    hipLaunchKernelGGL(scaled_sum_kernel<float>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, rp, n, O, I, num);
  if (hipError_t e = hipGetLastError()) {
    *what = "scaled sum";
    return int(e);
  }
  if (r > 0) {
    int64_t pb = ((O + I) * n * r + kThreads - 1) / kThreads;
    if (pb > 65536) pb = 65536;
    hipLaunchKernelGGL(pack_factors_kernel, dim3(unsigned(pb)), dim3(kThreads), 0, stream, fp, n, O, I, int(r), ucat,
                       vcat);
    if (hipError_t e = hipGetLastError()) {
      *what = "packing the factors";
      return int(e);
    }
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev)) {
      *what = "hipGetDevice";
      return int(e);
    }
    std::lock_guard<std::mutex> lock(g_blas.mu);
    rocblas_handle h = handle_for(dev, stream);
    if (!h || rocblas_set_stream(h, stream) != rocblas_status_success) {
      *what = "rocBLAS handle";
      return -1;
    }
    // num [O, I] -= Ucat [O, nr] . Vcat [I, nr]^T (row-major; column-major num^T = Vcat . Ucat^T).
    const float minus = -1.f, one = 1.f;
    const int K = int(n * r);
    if (rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_none, int(I), int(O), K, &minus, vcat, K, ucat,
                      K, &one, num, int(I)) != rocblas_status_success) {
      *what = "rocblas_sgemm (delta of the block update)";
      return -1;
    }
  }
  const unsigned by = unsigned(O < 4096 ? O : 4096);
  int64_t bx = (I + kThreads - 1) / kThreads;
  if (bx > 64) bx = 64;
  hipLaunchKernelGGL(refine_finish_kernel, dim3(unsigned(bx), by), dim3(kThreads), 0, stream, rp, n, O, I, num, prev,
                     out);
  if (hipError_t e = hipGetLastError()) {
    *what = "block update";
    return int(e);
  }
  return 0;
}

size_t lowrank_workspace_bytes(int64_t O, int64_t I, int64_t k, int64_t r, int cus) {
  return layout(O, I, k, r, cus).total;
}

int launch_lowrank_factors(tb_dtype dtype, const void* const* weights, int n, const float* const* w0s, const float* s,
                           int64_t O, int64_t I, int64_t r, const float* omega, int64_t k, int power_iters,
                           float* u_out, float* v_out, void* workspace, int cus, hipStream_t stream, const char** what) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) {
    *what = "hipGetDevice";
    return int(e);
  }
  std::lock_guard<std::mutex> lock(g_blas.mu);
  rocblas_handle h = handle_for(dev, stream);
  if (!h) {
    *what = "rocblas_create_handle";
    return -1;
  }
  Run R{static_cast<char*>(workspace), layout(O, I, k, r, cus), int(k), cus, n, stream, h};
  if (rocblas_set_stream(R.h, stream) != rocblas_status_success) {
    *what = "rocblas_set_stream";
    return -1;
  }
  const Layout& L = R.L;
  const int Oi = int(O), Ii = int(I), ki = int(k), ri = int(r);
  const int64_t fs = R.fstride();
  float* E = R.at<float>(L.e);
  float* O1 = R.at<float>(L.o1);
  float* I1 = R.at<float>(L.i1);
  auto gemm_fail = [&](const char* w) {
    *what = w;
    return -1;
  };

  {
    WeightPtrs wp{};
    for (int j = 0; j < n; ++j) {
      wp.w[j] = weights[j];
      wp.w0[j] = w0s[j];
    }
    int64_t bx = (I + kThreads - 1) / kThreads;
    if (bx > 64) bx = 64;
    const unsigned by = unsigned(O < 4096 ? O : 4096);
    if (dtype == TB_BF16)
      hipLaunchKernelGGL(residual_kernel<bf16_t>, dim3(unsigned(bx), by, unsigned(n)), dim3(kThreads), 0, stream, wp,
                         s, O, I, E, R.stride());
    else
      hipLaunchKernelGGL(residual_kernel<float>, dim3(unsigned(bx), by, unsigned(n)), dim3(kThreads), 0, stream, wp,
                         s, O, I, E, R.stride());
    if (hipError_t e = hipGetLastError()) {
      *what = "residual";
      return int(e);
    }
  }
  // Range finder: Y = E Omega (each matrix its own probe, [n][I][k]).
  if (gemm_rm_batched(R, false, false, Oi, ki, Ii, E, Ii, fs, omega, ki, I * k, O1, ki, fs) != rocblas_status_success)
    return gemm_fail("rocblas_sgemm (E Omega)");
  // Between power iterations one CholeskyQR round keeps the weak directions;
  // the final basis gets two.
  if (int e = orthonormalize(R, L.o1, O, power_iters > 0 ? 1 : 2, what)) return e;
  for (int it = 0; it < power_iters; ++it) {
    if (gemm_rm_batched(R, true, false, Ii, ki, Oi, E, Ii, fs, O1, ki, fs, I1, ki, fs) != rocblas_status_success)
      return gemm_fail("rocblas_sgemm (E^T Q)");
    if (int e = orthonormalize(R, L.i1, I, 1, what)) return e;
    if (gemm_rm_batched(R, false, false, Oi, ki, Ii, E, Ii, fs, I1, ki, fs, O1, ki, fs) != rocblas_status_success)
      return gemm_fail("rocblas_sgemm (E Q')");
    if (int e = orthonormalize(R, L.o1, O, it + 1 == power_iters ? 2 : 1, what)) return e;
  }
  // B^T = E^T Q, its Gram matrix B B^T, the Cholesky factor of that and the
  // SVD of the factor (the eigenvectors of B B^T).
  if (gemm_rm_batched(R, true, false, Ii, ki, Oi, E, Ii, fs, O1, ki, fs, I1, ki, fs) != rocblas_status_success)
    return gemm_fail("rocblas_sgemm (B^T)");
  if (hipError_t e = gram(R, L.i1, I, L.c)) {
    *what = "Gram matrix of B";
    return int(e);
  }
  hipLaunchKernelGGL(cholesky_kernel, dim3(unsigned(n)), dim3(kSolverThreads), 0, stream, R.at<const double>(L.c), ki,
                     R.at<double>(L.a), R.at<int>(L.drop), R.at<float>(L.m), R.stride());
  {
    const double* A = R.at<const double>(L.a);
    const int* dropped = R.at<const int>(L.drop);
    double* Rc = R.at<double>(L.c);
    double* Vc = R.at<double>(L.v);
    double* lam = R.at<double>(L.lam);
    int* perm = R.at<int>(L.perm);
    int* sw = R.at<int>(L.sweeps);
    // Groups of 16 or 32 lanes per pair keep more pairs in flight; columns
    // longer than 10 entries per lane take a whole wave.
    if (ki <= 160)
      hipLaunchKernelGGL((jacobi_kernel<16, 10>), dim3(unsigned(n)), dim3(kSolverThreads), 0, stream, A, dropped, ki,
                         Rc, Vc, lam, perm, sw, R.stride());
    else if (ki <= 320)
      hipLaunchKernelGGL((jacobi_kernel<32, 10>), dim3(unsigned(n)), dim3(kSolverThreads), 0, stream, A, dropped, ki,
                         Rc, Vc, lam, perm, sw, R.stride());
    else
      hipLaunchKernelGGL((jacobi_kernel<64, 8>), dim3(unsigned(n)), dim3(kSolverThreads), 0, stream, A, dropped, ki,
                         Rc, Vc, lam, perm, sw, R.stride());
    unsigned blocks = unsigned((k * r + kThreads - 1) / kThreads);
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(assemble_kernel, dim3(blocks, unsigned(n)), dim3(kThreads), 0, stream,
                       R.at<const double>(L.v), R.at<const double>(L.lam), R.at<const int>(L.perm), ki, ri,
                       R.at<float>(L.mu), R.at<float>(L.mv), R.stride());
  }
  if (hipError_t e = hipGetLastError()) {
    *what = "singular value decomposition";
    return int(e);
  }
  if (gemm_rm_batched(R, false, false, Oi, ri, ki, O1, ki, fs, R.at<const float>(L.mu), ri, fs, u_out, ri, O * r) !=
      rocblas_status_success)
    return gemm_fail("rocblas_sgemm (U)");
  if (gemm_rm_batched(R, false, false, Ii, ri, ki, I1, ki, fs, R.at<const float>(L.mv), ri, fs, v_out, ri, I * r) !=
      rocblas_status_success)
    return gemm_fail("rocblas_sgemm (V)");
  return 0;
}

}  // namespace tb
