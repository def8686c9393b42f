// Host-side internals of libtb: launch plans and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tb.h"

namespace tb {

constexpr size_t kControlBytes = TB_WORKSPACE_CONTROL_BYTES;
constexpr int kMaxGroupCounters = int(kControlBytes / 4) - 64;  // words 64.. of the control region

// Compute units of the current device (queried once per device).
int device_cu_count(int* cus);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- forward, skinny token counts (m <= kDecodeMaxTokens) -----------------
constexpr int kDecodeMaxTokens = 64;

struct DecodePlan {
  int NT;        // 16-token column tiles (1, 2 or 4)
  int TILES;     // 16-row tiles each streaming workgroup is built for (1, 2, 4 or 6)
  int NRB, KS;   // streaming row blocks and k-slices of in_dim
  int NB;        // streaming workgroups (NRB * KS)
  int NCB, KT;   // x . V producers: 16-column blocks of T and k-slices of in_dim
  int NP;        // producer workgroups (NCB * KT)
  size_t off_tpart, off_tfull, off_ypart, bytes;
};

DecodePlan plan_decode(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, int cus);

hipError_t launch_forward_decode(const DecodePlan& p, tb_dtype dtype, const void* x, const void* s, const void* w0,
                                 const void* u, const void* v, void* y, int64_t m, int64_t out_dim, int64_t in_dim,
                                 int64_t rank, void* workspace, hipStream_t stream);

// ---- forward, prefill token counts (bf16, m > kDecodeMaxTokens) ----------
struct GemmPlan {
  size_t off_t, bytes;
};
GemmPlan plan_gemm(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank);

hipError_t launch_forward_gemm(const GemmPlan& p, const void* x, const void* s, const void* w0, const void* u,
                               const void* v, void* y, int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank,
                               void* workspace, hipStream_t stream);

// ---- reconstruct ----------------------------------------------------------
hipError_t launch_reconstruct(tb_dtype in_dtype, tb_dtype out_dtype, const void* s, const void* w0, const void* u,
                              const void* v, void* w_out, int64_t out_dim, int64_t in_dim, int64_t rank,
                              hipStream_t stream);

// ---- relative Frobenius error ---------------------------------------------
hipError_t launch_frobenius(tb_dtype dtype, const void* a, const void* b, int64_t n, double* result,
                            void* workspace, int cus, hipStream_t stream);

}  // namespace tb
