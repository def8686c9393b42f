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
// basis() is CholeskyQR2: the fp64 Gram matrix of the columns, a Cholesky
// factor R whose pivots at or below 1e-13 of the largest diagonal entry mark
// directions the columns do not span (their columns of Q are zero), and
// Q = Y R^-1, twice.  The same span as a Householder QR, so the same U V^T up
// to rounding.  The large products run as plain fp32 GEMMs (rocBLAS); the
// Gram matrices, the Cholesky factor and its inverse and the symmetric
// eigen-decomposition (cyclic Jacobi over a round-robin pair order, fp64) are
// the kernels below.
#include <rocblas/rocblas.h>

#include <mutex>

#include "tb_device.h"
#include "tb_host.h"
#include "tb_reduce.h"

namespace tb {

namespace {

constexpr int kThreads = 256;
constexpr int kSolverThreads = 1024;
constexpr double kPivotTol = 1e-13;     // Cholesky pivot / largest diagonal entry below which a direction is dropped
constexpr double kSigmaTol = 1e-14;     // eigenvalue / largest below which a singular value counts as zero
constexpr double kJacobiTol = 1e-15;    // largest |a_pq| / sqrt(a_pp a_qq) at which a sweep ends the iteration
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

// ---- residual --------------------------------------------------------------------

// E = W - diag(s) W0 in fp32, one rounding (fma) per entry.  grid (column
// blocks, row blocks), both grid-stride.
template <typename E>
__global__ __launch_bounds__(kThreads) void residual_kernel(const E* __restrict__ w, const float* __restrict__ w0,
                                                            const float* __restrict__ s, int64_t O, int64_t I,
                                                            float* __restrict__ e) {
  for (int64_t o = blockIdx.y; o < O; o += gridDim.y) {
    const float so = s[o];
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < I; i += int64_t(gridDim.x) * kThreads) {
      const int64_t at = o * I + i;
      e[at] = fmaf(-so, w0[at], to_f32<E>(w[at]));
    }
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
__global__ __launch_bounds__(kThreads) void gram_partial_kernel(const float* __restrict__ A, int64_t n, int k,
                                                                int64_t rows_per, double* __restrict__ part) {
  __shared__ float as[kGramRows][kGramTile], bs[kGramRows][kGramTile];
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
__global__ __launch_bounds__(kThreads) void gram_reduce_kernel(const double* __restrict__ part, int k, int splits,
                                                               double* __restrict__ C) {
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

// ---- Cholesky factor and its inverse (one workgroup, fp64) -------------------------

// C = R^T R (R upper) with dropped directions: a pivot at or below kPivotTol
// of the largest diagonal entry of C zeroes its row of R and its column and
// row of R^-1.  M = R^-1 in fp32 (k x k, row-major).  A and X: k x k scratch.
__global__ __launch_bounds__(kSolverThreads) void chol_inv_kernel(const double* __restrict__ C, int k,
                                                                  double* __restrict__ A, double* __restrict__ X,
                                                                  int* __restrict__ dropped, float* __restrict__ M) {
  __shared__ double s_piv, s_max;
  __shared__ int s_drop;
  const int tid = threadIdx.x;
  const int64_t kk = int64_t(k) * k;
  for (int64_t i = tid; i < kk; i += kSolverThreads) A[i] = C[i];
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
      s_piv = drop ? 0.0 : sqrt(d);
      dropped[j] = drop;
      A[size_t(j) * k + j] = s_piv;
    }
    __syncthreads();
    const double piv = s_piv;
    const bool drop = s_drop;
    for (int l = j + 1 + tid; l < k; l += kSolverThreads) A[size_t(j) * k + l] = drop ? 0.0 : A[size_t(j) * k + l] / piv;
    __syncthreads();
    if (!drop) {
      const int n = k - j - 1;
      for (int idx = tid; idx < n * n; idx += kSolverThreads) {
        const int l = j + 1 + idx / n, m = j + 1 + idx % n;
        if (m >= l) A[size_t(l) * k + m] -= A[size_t(j) * k + l] * A[size_t(j) * k + m];
      }
    }
    __syncthreads();
  }
  // X = R^-1 by back substitution, one column per thread (k <= kSolverThreads).
  if (tid < k) {
    const int c = tid;
    for (int i = 0; i < k; ++i) X[size_t(i) * k + c] = 0.0;
    if (!dropped[c]) {
      X[size_t(c) * k + c] = 1.0 / A[size_t(c) * k + c];
      for (int i = c - 1; i >= 0; --i) {
        if (dropped[i]) continue;
        double sum = 0.0;
        for (int m = i + 1; m <= c; ++m) sum += A[size_t(i) * k + m] * X[size_t(m) * k + c];
        X[size_t(i) * k + c] = -sum / A[size_t(i) * k + i];
      }
    }
    for (int i = 0; i < k; ++i) M[size_t(i) * k + c] = float(X[size_t(i) * k + c]);
  }
}

// ---- symmetric eigen-decomposition (one workgroup, fp64) -----------------------------

// Cyclic Jacobi: each sweep runs the kk - 1 rounds of the round-robin
// (circle) order over kk = k rounded up to even, so that every pair (p, q)
// is rotated once per sweep and the kk / 2 pairs of a round are disjoint and
// rotate together: rows p, q of A, then columns p, q of A and of V (the
// rotation J with J_pp = J_qq = c, J_pq = s, J_qp = -s, A <- J^T A J,
// V <- V J, chosen to zero a_pq).  Ends when a whole sweep saw no
// |a_pq| / sqrt(a_pp a_qq) above kJacobiTol.  On exit lam holds the
// eigenvalues (diagonal of A) and perm the columns of V by decreasing
// eigenvalue (ties by index); sweeps[0] the sweeps taken.
__global__ __launch_bounds__(kSolverThreads) void jacobi_kernel(double* __restrict__ A, double* __restrict__ V, int k,
                                                                double* __restrict__ lam, int* __restrict__ perm,
                                                                int* __restrict__ sweeps) {
  __shared__ double s_c[kSolverThreads / 2], s_s[kSolverThreads / 2];
  __shared__ int s_p[kSolverThreads / 2], s_q[kSolverThreads / 2];
  __shared__ double s_red[kSolverThreads];
  const int tid = threadIdx.x;
  const int kk = k + (k & 1), P = kk / 2;
  const int64_t k2 = int64_t(k) * k;
  for (int64_t i = tid; i < k2; i += kSolverThreads) V[i] = (i / k == i % k) ? 1.0 : 0.0;
  __syncthreads();
  int sweep = 0;
  for (; sweep < kMaxSweeps; ++sweep) {
    double off = 0.0;
    for (int t = 0; t < kk - 1; ++t) {
      if (tid < P) {
        const auto rot = [&](int x) { return ((x - 1 + t) % (kk - 1)) + 1; };
        const int a = tid == 0 ? 0 : rot(tid), b = rot(kk - 1 - tid);
        const int p = a < b ? a : b, q = a < b ? b : a;
        double c = 1.0, s = 0.0;
        if (q < k) {
          const double apq = A[size_t(p) * k + q], app = A[size_t(p) * k + p], aqq = A[size_t(q) * k + q];
          const double d = sqrt(fabs(app * aqq));
          if (d > 0.0) off = fmax(off, fabs(apq) / d);
          else if (apq != 0.0) off = 1.0;
          if (apq != 0.0 && fabs(apq) > 1e-18 * d) {
            const double th = (aqq - app) / (2.0 * apq);
            const double tt = th == 0.0             ? 1.0
                              : fabs(th) > 1e150 ? 0.5 / th
                                                 : copysign(1.0, th) / (fabs(th) + sqrt(th * th + 1.0));
            c = 1.0 / sqrt(tt * tt + 1.0);
            s = tt * c;
          }
        }
        s_p[tid] = p;
        s_q[tid] = q;
        s_c[tid] = c;
        s_s[tid] = s;
      }
      __syncthreads();
      for (int idx = tid; idx < P * k; idx += kSolverThreads) {   // rows p, q
        const int pr = idx / k, j = idx % k;
        const int p = s_p[pr], q = s_q[pr];
        const double s = s_s[pr];
        if (q >= k || s == 0.0) continue;
        const double c = s_c[pr], x = A[size_t(p) * k + j], y = A[size_t(q) * k + j];
        A[size_t(p) * k + j] = c * x - s * y;
        A[size_t(q) * k + j] = s * x + c * y;
      }
      __syncthreads();
      for (int idx = tid; idx < k * P; idx += kSolverThreads) {   // columns p, q
        const int i = idx / P, pr = idx % P;
        const int p = s_p[pr], q = s_q[pr];
        const double s = s_s[pr];
        if (q >= k || s == 0.0) continue;
        const double c = s_c[pr];
        double x = A[size_t(i) * k + p], y = A[size_t(i) * k + q];
        A[size_t(i) * k + p] = c * x - s * y;
        A[size_t(i) * k + q] = s * x + c * y;
        x = V[size_t(i) * k + p];
        y = V[size_t(i) * k + q];
        V[size_t(i) * k + p] = c * x - s * y;
        V[size_t(i) * k + q] = s * x + c * y;
      }
      __syncthreads();
    }
    s_red[tid] = off;
    __syncthreads();
    for (int h = kSolverThreads / 2; h > 0; h >>= 1) {
      if (tid < h) s_red[tid] = fmax(s_red[tid], s_red[tid + h]);
      __syncthreads();
    }
    const bool done = s_red[0] <= kJacobiTol;
    __syncthreads();
    if (done) {
      ++sweep;
      break;
    }
  }
  for (int j = tid; j < k; j += kSolverThreads) lam[j] = A[size_t(j) * k + j];
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
// sqrt of the j-th largest eigenvalue; a singular value at or below
// sqrt(kSigmaTol) of the largest counts as zero (zero columns in both).
__global__ __launch_bounds__(kThreads) void assemble_kernel(const double* __restrict__ V, const double* __restrict__ lam,
                                                            const int* __restrict__ perm, int k, int r,
                                                            float* __restrict__ Mu, float* __restrict__ Mv) {
  const double lmax = lam[perm[0]];
  for (int idx = blockIdx.x * kThreads + threadIdx.x; idx < k * r; idx += gridDim.x * kThreads) {
    const int a = idx / r, j = idx % r;
    const int col = perm[j];
    const double l = lam[col];
    const bool zero = !(l > kSigmaTol * lmax) || !(lmax > 0.0);
    const double sg = zero ? 0.0 : sqrt(l);
    const double v = V[size_t(a) * k + col];
    Mu[idx] = zero ? 0.f : float(v * sg);
    Mv[idx] = zero ? 0.f : float(v / sg);
  }
}

// ---- host side ------------------------------------------------------------------------

struct Blas {
  std::mutex mu;
  rocblas_handle h[64] = {};
};
Blas g_blas;

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
  size_t e, o1, o2, i1, i2, part, c, a, x, v, m, lam, perm, drop, sweeps, mu, mv, total;
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
  L.o2 = take(size_t(O) * k * 4);
  L.i1 = take(size_t(I) * k * 4);
  L.i2 = take(size_t(I) * k * 4);
  L.part = take(size_t(splits) * k * k * 8);
  L.c = take(size_t(k) * k * 8);
  L.a = take(size_t(k) * k * 8);
  L.x = take(size_t(k) * k * 8);
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
  char* ws;
  Layout L;
  int k, cus;
  hipStream_t stream;
  rocblas_handle h;
};

// C = A^T A for A [n, k] fp32.
hipError_t gram(const Run& R, const float* A, int64_t n, double* C) {
  const int k = R.k, T = (k + kGramTile - 1) / kGramTile, tiles = T * (T + 1) / 2;
  const int splits = gram_splits(n, k, R.cus);
  const int64_t rows_per = (n + splits - 1) / splits;
  double* part = reinterpret_cast<double*>(R.ws + R.L.part);
  hipLaunchKernelGGL(gram_partial_kernel, dim3(unsigned(tiles), unsigned(splits)), dim3(kThreads), 0, R.stream, A, n,
                     k, rows_per, part);
  const int64_t kk = int64_t(k) * k;
  const unsigned blocks = unsigned((kk + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(gram_reduce_kernel, dim3(blocks), dim3(kThreads), 0, R.stream, part, k, splits, C);
  return hipGetLastError();
}

// X [n, k] <- orthonormal basis of its columns (CholeskyQR2), T [n, k] scratch.
int orthonormalize(const Run& R, float* X, float* T, int64_t n, const char** what) {
  double* C = reinterpret_cast<double*>(R.ws + R.L.c);
  float* M = reinterpret_cast<float*>(R.ws + R.L.m);
  for (int pass = 0; pass < 2; ++pass) {
    float* src = pass == 0 ? X : T;
    float* dst = pass == 0 ? T : X;
    if (hipError_t e = gram(R, src, n, C)) {
      *what = "Gram matrix";
      return int(e);
    }
    hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(kSolverThreads), 0, R.stream, C, R.k,
                       reinterpret_cast<double*>(R.ws + R.L.a), reinterpret_cast<double*>(R.ws + R.L.x),
                       reinterpret_cast<int*>(R.ws + R.L.drop), M);
    if (hipError_t e = hipGetLastError()) {
      *what = "Cholesky factor";
      return int(e);
    }
    if (gemm_rm(R.h, false, false, int(n), R.k, R.k, src, R.k, M, R.k, dst, R.k) != rocblas_status_success) {
      *what = "rocblas_sgemm (basis)";
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

size_t lowrank_workspace_bytes(int64_t O, int64_t I, int64_t k, int64_t r, int cus) {
  return layout(O, I, k, r, cus).total;
}

int launch_lowrank_factors(tb_dtype dtype, const void* weight, const float* w0, const float* s, int64_t O, int64_t I,
                           int64_t r, const float* omega, int64_t k, int power_iters, float* u_out, float* v_out,
                           void* workspace, int cus, hipStream_t stream, const char** what) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) {
    *what = "hipGetDevice";
    return int(e);
  }
  if (dev < 0 || dev >= 64) {
    *what = "device index";
    return int(hipErrorInvalidDevice);
  }
  std::lock_guard<std::mutex> lock(g_blas.mu);
  if (!g_blas.h[dev] && rocblas_create_handle(&g_blas.h[dev]) != rocblas_status_success) {
    g_blas.h[dev] = nullptr;
    *what = "rocblas_create_handle";
    return -1;
  }
  Run R{static_cast<char*>(workspace), layout(O, I, k, r, cus), int(k), cus, stream, g_blas.h[dev]};
  if (rocblas_set_stream(R.h, stream) != rocblas_status_success) {
    *what = "rocblas_set_stream";
    return -1;
  }
  float* E = reinterpret_cast<float*>(R.ws + R.L.e);
  float* O1 = reinterpret_cast<float*>(R.ws + R.L.o1);
  float* O2 = reinterpret_cast<float*>(R.ws + R.L.o2);
  float* I1 = reinterpret_cast<float*>(R.ws + R.L.i1);
  float* I2 = reinterpret_cast<float*>(R.ws + R.L.i2);
  const int Oi = int(O), Ii = int(I), ki = int(k), ri = int(r);

  {
    int64_t bx = (I + kThreads - 1) / kThreads;
    if (bx > 64) bx = 64;
    const unsigned by = unsigned(O < 65535 ? O : 65535);
    if (dtype == TB_BF16)
      hipLaunchKernelGGL(residual_kernel<bf16_t>, dim3(unsigned(bx), by), dim3(kThreads), 0, stream,
                         static_cast<const bf16_t*>(weight), w0, s, O, I, E);
    else
      hipLaunchKernelGGL(residual_kernel<float>, dim3(unsigned(bx), by), dim3(kThreads), 0, stream,
                         static_cast<const float*>(weight), w0, s, O, I, E);
    if (hipError_t e = hipGetLastError()) {
      *what = "residual";
      return int(e);
    }
  }
  auto gemm_fail = [&](const char* w) {
    *what = w;
    return -1;
  };
  // Range finder.
  if (gemm_rm(R.h, false, false, Oi, ki, Ii, E, Ii, omega, ki, O1, ki) != rocblas_status_success)
    return gemm_fail("rocblas_sgemm (E Omega)");
  if (int e = orthonormalize(R, O1, O2, O, what)) return e;
  for (int it = 0; it < power_iters; ++it) {
    if (gemm_rm(R.h, true, false, Ii, ki, Oi, E, Ii, O1, ki, I1, ki) != rocblas_status_success)
      return gemm_fail("rocblas_sgemm (E^T Q)");
    if (int e = orthonormalize(R, I1, I2, I, what)) return e;
    if (gemm_rm(R.h, false, false, Oi, ki, Ii, E, Ii, I1, ki, O1, ki) != rocblas_status_success)
      return gemm_fail("rocblas_sgemm (E Q')");
    if (int e = orthonormalize(R, O1, O2, O, what)) return e;
  }
  // B^T = E^T Q, its Gram matrix B B^T and the eigen-decomposition.
  if (gemm_rm(R.h, true, false, Ii, ki, Oi, E, Ii, O1, ki, I1, ki) != rocblas_status_success)
    return gemm_fail("rocblas_sgemm (B^T)");
  double* C = reinterpret_cast<double*>(R.ws + R.L.c);
  if (hipError_t e = gram(R, I1, I, C)) {
    *what = "Gram matrix of B";
    return int(e);
  }
  double* A = reinterpret_cast<double*>(R.ws + R.L.a);
  if (hipError_t e = hipMemcpyAsync(A, C, size_t(k) * k * 8, hipMemcpyDeviceToDevice, stream)) {
    *what = "copy";
    return int(e);
  }
  double* lam = reinterpret_cast<double*>(R.ws + R.L.lam);
  int* perm = reinterpret_cast<int*>(R.ws + R.L.perm);
  hipLaunchKernelGGL(jacobi_kernel, dim3(1), dim3(kSolverThreads), 0, stream, A,
                     reinterpret_cast<double*>(R.ws + R.L.v), ki, lam, perm, reinterpret_cast<int*>(R.ws + R.L.sweeps));
  float* Mu = reinterpret_cast<float*>(R.ws + R.L.mu);
  float* Mv = reinterpret_cast<float*>(R.ws + R.L.mv);
  {
    unsigned blocks = unsigned((k * r + kThreads - 1) / kThreads);
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(assemble_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<const double*>(R.ws + R.L.v), lam, perm, ki, ri, Mu, Mv);
  }
  if (hipError_t e = hipGetLastError()) {
    *what = "eigen-decomposition";
    return int(e);
  }
  if (gemm_rm(R.h, false, false, Oi, ri, ki, O1, ki, Mu, ri, u_out, ri) != rocblas_status_success)
    return gemm_fail("rocblas_sgemm (U)");
  if (gemm_rm(R.h, false, false, Ii, ri, ki, I1, ki, Mv, ri, v_out, ri) != rocblas_status_success)
    return gemm_fail("rocblas_sgemm (V)");
  return 0;
}

}  // namespace tb
