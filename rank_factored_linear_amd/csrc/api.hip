// C ABI of libtb: host-side argument checks and dispatch.  Every check runs
// before anything is enqueued, so a failing call leaves all outputs untouched.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "tb_host.h"

namespace tb {

namespace {

thread_local char g_last_error[512] = "";

tb_status fail(tb_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

tb_status ok() {
  g_last_error[0] = '\0';
  return TB_OK;
}

tb_status hip_fail(hipError_t e, const char* what) {
  return fail(TB_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t esize(tb_dtype d) { return d == TB_BF16 ? 2 : 4; }
bool valid_dtype(tb_dtype d) { return d == TB_F32 || d == TB_BF16; }

constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices];  // 0 = not queried yet (benign race: every writer stores the same value)

// Shapes the kernels index with 32-bit ints.
constexpr int64_t kMaxDim = int64_t(1) << 30;

tb_status check_dims(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank) {
  if (m < 1 || out_dim < 1 || in_dim < 1 || rank < 0)
    return fail(TB_ERR_INVALID_ARGUMENT, "need m >= 1, out_dim >= 1, in_dim >= 1, rank >= 0 (got %lld, %lld, %lld, %lld)",
                (long long)m, (long long)out_dim, (long long)in_dim, (long long)rank);
  if (m > kMaxDim || out_dim > kMaxDim || in_dim > kMaxDim || rank > kMaxDim)
    return fail(TB_ERR_UNSUPPORTED, "a dimension exceeds 2^30");
  if (in_dim % 8 != 0) return fail(TB_ERR_UNSUPPORTED, "in_dim %lld is not a multiple of 8", (long long)in_dim);
  return TB_OK;
}

}  // namespace

namespace {
std::atomic<int> g_wait_polls{1 << 20};
}  // namespace

int decode_wait_polls() { return g_wait_polls.load(std::memory_order_relaxed); }

int device_cu_count(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev >= 0 && dev < kMaxDevices && g_cus[dev] > 0) {
    *cus = g_cus[dev];
    return 0;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return int(e);
  if (n < 2) n = 2;
  if (dev >= 0 && dev < kMaxDevices) g_cus[dev] = n;
  *cus = n;
  return 0;
}

}  // namespace tb

using namespace tb;

extern "C" {

tb_status tb_band_index(int32_t num_layers, int32_t num_bands, int32_t layer, int32_t* band_out) {
  if (band_out == nullptr) return fail(TB_ERR_INVALID_ARGUMENT, "band_out is NULL");
  if (num_layers < 1) return fail(TB_ERR_INVALID_ARGUMENT, "num_layers %d < 1", num_layers);
  if (num_bands < 1 || num_bands > num_layers)
    return fail(TB_ERR_INVALID_ARGUMENT, "num_bands %d outside [1, %d]", num_bands, num_layers);
  if (layer < 0 || layer >= num_layers)
    return fail(TB_ERR_INVALID_ARGUMENT, "layer %d outside [0, %d)", layer, num_layers);
  // q layers per band, the first m bands one more; they end at layer m(q+1).
  const int32_t q = num_layers / num_bands, m = num_layers % num_bands;
  const int32_t big = m * (q + 1);
  *band_out = layer < big ? layer / (q + 1) : m + (layer - big) / q;
  return ok();
}

namespace {

// Data bytes of one projection's buffers: enough for every plan a call of m
// tokens may take (alone or in a group, whatever its streamer budget; the
// last 64-token slice of a longer fp32 call has a plan of its own).
size_t forward_data_bytes(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, tb_dtype dtype, int cus) {
  if (dtype == TB_BF16 && m > kDecodeMaxTokens) return plan_gemm(1, &out_dim, m, in_dim, rank, cus).bytes;
  size_t bytes = 0;
  const int64_t counts[2] = {m < kDecodeMaxTokens ? m : kDecodeMaxTokens,
                             m > kDecodeMaxTokens ? m % kDecodeMaxTokens : 0};
  for (int64_t mt : counts)
    if (mt > 0) bytes = std::max(bytes, decode_bytes_bound(mt, out_dim, in_dim, rank, cus));
  return bytes;
}

// Whether the members of a group run as one launch of each prefill kernel:
// bf16, more than kDecodeMaxTokens tokens, and one in_dim and rank for all
// (q, k and v of a layer; gate and up).
bool fused_prefill(int n, const tb_projection* projs, int64_t m, tb_dtype dtype) {
  if (dtype != TB_BF16 || m <= kDecodeMaxTokens || n < 2) return false;
  for (int j = 1; j < n; ++j)
    if (projs[j].in_dim != projs[0].in_dim || projs[j].rank != projs[0].rank) return false;
  return true;
}

GemmPlan fused_prefill_plan(int n, const tb_projection* projs, int64_t m, int cus) {
  int64_t outs[TB_MAX_GROUP];
  for (int j = 0; j < n; ++j) outs[j] = projs[j].out_dim;
  return plan_gemm(n, outs, m, projs[0].in_dim, projs[0].rank, cus);
}

// Data bytes of a group: every member's own buffers one after another (the
// members may run as calls of their own), or the fused launch's buffers if
// they are more.
size_t group_data_bytes(int n, const tb_projection* projs, int64_t m, tb_dtype dtype, int cus) {
  size_t total = 0;
  for (int j = 0; j < n; ++j)
    total += forward_data_bytes(m, projs[j].out_dim, projs[j].in_dim, projs[j].rank, dtype, cus);
  if (fused_prefill(n, projs, m, dtype)) total = std::max(total, fused_prefill_plan(n, projs, m, cus).bytes);
  return total;
}

}  // namespace

tb_status tb_linear_forward_workspace_size(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, tb_dtype dtype,
                                           size_t* bytes_out) {
  if (bytes_out == nullptr) return fail(TB_ERR_INVALID_ARGUMENT, "bytes_out is NULL");
  if (!valid_dtype(dtype)) return fail(TB_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(dtype));
  tb_status st = check_dims(m, out_dim, in_dim, rank);
  if (st != TB_OK) return st;
  int cus = 0;
  if (int e = device_cu_count(&cus)) return hip_fail(hipError_t(e), "querying the compute-unit count");
  *bytes_out = kControlBytes + forward_data_bytes(m, out_dim, in_dim, rank, dtype, cus);
  return ok();
}

static_assert(TB_MAX_GROUP == kMaxProjections, "one launch takes every member of a group");

namespace {

// Argument checks shared by tb_linear_forward and each member of a group.
tb_status check_projection(const void* x, const void* s, const void* w0, const void* u, const void* v, const void* y,
                           int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, tb_dtype dtype) {
  if (!valid_dtype(dtype)) return fail(TB_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(dtype));
  tb_status st = check_dims(m, out_dim, in_dim, rank);
  if (st != TB_OK) return st;
  if (!x || !w0 || !y) return fail(TB_ERR_INVALID_ARGUMENT, "x, w0 and y must be non-NULL");
  if (rank > 0 && (!u || !v)) return fail(TB_ERR_INVALID_ARGUMENT, "u and v must be non-NULL when rank > 0");
  if (!aligned16(x) || !aligned16(w0) || (rank > 0 && (!aligned16(u) || !aligned16(v))))
    return fail(TB_ERR_UNSUPPORTED, "x, w0, u and v must be 16-byte aligned");
  if (!aligned_to(s, esize(dtype)) || !aligned_to(y, esize(dtype)))
    return fail(TB_ERR_UNSUPPORTED, "s and y must be aligned to their element size");
  // The few-token path addresses a row block (at most 96 rows) with 32-bit
  // byte offsets.
  const bool decode = !(dtype == TB_BF16 && m > kDecodeMaxTokens);
  if (decode && in_dim * int64_t(esize(dtype)) * 96 >= (int64_t(1) << 32))
    return fail(TB_ERR_UNSUPPORTED, "in_dim %lld is too large for the few-token path", (long long)in_dim);
  return TB_OK;
}

// One projection with checked arguments: the prefill GEMM, or the decode
// kernel over 64-token slices.  ctrl is its control block, data holds
// forward_data_bytes, timeouts are flagged in *err_word.
tb_status forward_one(const void* x, const void* s, const void* w0, const void* u, const void* v, void* y, int64_t m,
                      int64_t out_dim, int64_t in_dim, int64_t rank, tb_dtype dtype, unsigned* ctrl, char* data,
                      unsigned* err_word, int cus, hipStream_t hs) {
  if (dtype == TB_BF16 && m > kDecodeMaxTokens) {
    const GemmPlan p = plan_gemm(1, &out_dim, m, in_dim, rank, cus);
    const Projection q{x, s, w0, u, v, y, out_dim, in_dim, rank};
    hipError_t e = launch_forward_gemm(p, &q, m, in_dim, rank, ctrl, data, err_word, hs);
    if (e != hipSuccess) return hip_fail(e, "launching the prefill projection");
    return ok();
  }
  const int64_t mm = m < kDecodeMaxTokens ? m : kDecodeMaxTokens;
  const size_t es = esize(dtype);
  const int64_t w0_elems = out_dim * in_dim;
  const DecodePlan p = plan_decode_spared(mm, out_dim, in_dim, rank, cus, w0_elems);
  for (int64_t t0 = 0; t0 < m; t0 += kDecodeMaxTokens) {
    const int64_t mt = (m - t0) < kDecodeMaxTokens ? (m - t0) : kDecodeMaxTokens;
    const DecodePlan pt = mt == mm ? p : plan_decode_spared(mt, out_dim, in_dim, rank, cus, w0_elems);
    const char* xt = static_cast<const char*>(x) + size_t(t0) * size_t(in_dim) * es;
    char* yt = static_cast<char*>(y) + size_t(t0) * size_t(out_dim) * es;
    hipError_t e =
        launch_forward_decode(pt, dtype, xt, s, w0, u, v, yt, mt, out_dim, in_dim, rank, ctrl, data, err_word, hs);
    if (e != hipSuccess) return hip_fail(e, "launching the decode projection");
  }
  return ok();
}

}  // namespace

tb_status tb_linear_forward(const void* x, const void* s, const void* w0, const void* u, const void* v, void* y,
                            int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, tb_dtype dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  tb_status st = check_projection(x, s, w0, u, v, y, m, out_dim, in_dim, rank, dtype);
  if (st != TB_OK) return st;
  if (!workspace) return fail(TB_ERR_INVALID_ARGUMENT, "workspace must be non-NULL");
  if (!aligned_to(workspace, 256)) return fail(TB_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  int cus = 0;
  if (int e = device_cu_count(&cus)) return hip_fail(hipError_t(e), "querying the compute-unit count");
  const size_t need = kControlBytes + forward_data_bytes(m, out_dim, in_dim, rank, dtype, cus);
  if (workspace_bytes < need)
    return fail(TB_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  unsigned* ctrl = static_cast<unsigned*>(workspace);
  return forward_one(x, s, w0, u, v, y, m, out_dim, in_dim, rank, dtype, ctrl, static_cast<char*>(workspace) + kControlBytes,
                     ctrl + 2, cus, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---- the forward call that allocates nothing --------------------------------
//
// Its workspace is this file-scope device array, one per GPU, laid out as a
// forward workspace: control words first, then the projection's buffers.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// every host use goes through the address hipGetSymbolAddress gives for the
// current device, looked up once per device.
namespace tb {
namespace {

static_assert(TB_NO_ALLOC_SCRATCH_BYTES >= kControlBytes + (size_t(1) << 20), "scratch holds the control words");
static __device__ __align__(256) unsigned char scratch[TB_NO_ALLOC_SCRATCH_BYTES];

struct ScratchSlot {
  std::once_flag once;
  unsigned char* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// The device address of this device's scratch (set-up on its first use).
hipError_t device_scratch(unsigned char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] {
    void* p = nullptr;
    slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    slot.ptr = static_cast<unsigned char*>(p);
  });
  if (slot.err != hipSuccess) return slot.err;
  *out = slot.ptr;
  return hipSuccess;
}

// Clears one control block (a small kernel rather than a memset, so that the
// call can be captured into a graph).
__global__ void clear_control_block(unsigned* words) {
  const int i = int(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < int(kCtrlBlockBytes / 4)) words[i] = 0u;
}

}  // namespace
}  // namespace tb

extern "C" {

tb_status tb_linear_forward_no_alloc(const void* x, const void* s, const void* w0, const void* u, const void* v,
                                     void* y, int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank,
                                     tb_dtype dtype, void* stream) {
  tb_status st = check_projection(x, s, w0, u, v, y, m, out_dim, in_dim, rank, dtype);
  if (st != TB_OK) return st;
  int cus = 0;
  if (int e = device_cu_count(&cus)) return hip_fail(hipError_t(e), "querying the compute-unit count");
  const size_t need = kControlBytes + forward_data_bytes(m, out_dim, in_dim, rank, dtype, cus);
  if (need > TB_NO_ALLOC_SCRATCH_BYTES)
    return fail(TB_ERR_UNSUPPORTED, "this call needs %zu bytes of scratch, above the %zu of the static buffer "
                "(tb_linear_forward takes a workspace of any size)", need, size_t(TB_NO_ALLOC_SCRATCH_BYTES));
  unsigned char* base = nullptr;
  if (hipError_t e = device_scratch(&base)) return hip_fail(e, "looking up the static scratch");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  unsigned* ctrl = reinterpret_cast<unsigned*>(base);
  // A single call uses control block 0 only.  It starts from zero every time,
  // so a call whose wait timed out does not poison the ones after it.
  hipLaunchKernelGGL(clear_control_block, dim3(unsigned(kCtrlBlockBytes / 4 / 256)), dim3(256), 0, hs, ctrl);
  if (hipError_t e = hipGetLastError()) return hip_fail(e, "clearing the scratch's control words");
  return forward_one(x, s, w0, u, v, y, m, out_dim, in_dim, rank, dtype, ctrl,
                     reinterpret_cast<char*>(base) + kControlBytes, ctrl + 2, cus, hs);
}

tb_status tb_dense_forward(const void* x, const void* w, void* y, int64_t m, int64_t out_dim, int64_t in_dim,
                           tb_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!w) return fail(TB_ERR_INVALID_ARGUMENT, "w must be non-NULL");
  return tb_linear_forward(x, nullptr, w, nullptr, nullptr, y, m, out_dim, in_dim, 0, dtype, workspace, workspace_bytes,
                           stream);
}

tb_status tb_linear_forward_group_workspace_size(int32_t n, const tb_projection* projs, int64_t m, tb_dtype dtype,
                                                 size_t* bytes_out) {
  if (bytes_out == nullptr || projs == nullptr) return fail(TB_ERR_INVALID_ARGUMENT, "projs and bytes_out must be non-NULL");
  if (n < 1 || n > TB_MAX_GROUP) return fail(TB_ERR_INVALID_ARGUMENT, "n %d outside [1, %d]", n, TB_MAX_GROUP);
  if (!valid_dtype(dtype)) return fail(TB_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(dtype));
  for (int j = 0; j < n; ++j) {
    tb_status st = check_dims(m, projs[j].out_dim, projs[j].in_dim, projs[j].rank);
    if (st != TB_OK) return st;
  }
  int cus = 0;
  if (int e = device_cu_count(&cus)) return hip_fail(hipError_t(e), "querying the compute-unit count");
  *bytes_out = kControlBytes + group_data_bytes(n, projs, m, dtype, cus);
  return ok();
}

tb_status tb_linear_forward_group(int32_t n, const tb_projection* projs, int64_t m, tb_dtype dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (projs == nullptr || workspace == nullptr) return fail(TB_ERR_INVALID_ARGUMENT, "projs and workspace must be non-NULL");
  if (n < 1 || n > TB_MAX_GROUP) return fail(TB_ERR_INVALID_ARGUMENT, "n %d outside [1, %d]", n, TB_MAX_GROUP);
  if (!aligned_to(workspace, 256)) return fail(TB_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  for (int j = 0; j < n; ++j) {
    const tb_projection& q = projs[j];
    tb_status st = check_projection(q.x, q.s, q.w0, q.u, q.v, q.y, m, q.out_dim, q.in_dim, q.rank, dtype);
    if (st != TB_OK) return st;
  }
  int cus = 0;
  if (int e = device_cu_count(&cus)) return hip_fail(hipError_t(e), "querying the compute-unit count");
  size_t off[TB_MAX_GROUP], at = kControlBytes;
  for (int j = 0; j < n; ++j) {
    const tb_projection& q = projs[j];
    off[j] = at;
    at += forward_data_bytes(m, q.out_dim, q.in_dim, q.rank, dtype, cus);
  }
  const size_t total = kControlBytes + group_data_bytes(n, projs, m, dtype, cus);
  if (workspace_bytes < total)
    return fail(TB_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is below the %zu needed", workspace_bytes, total);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  unsigned* ctrl = reinterpret_cast<unsigned*>(ws);
  unsigned* err = ctrl + 2;

  if (m <= kDecodeMaxTokens) {
    // One launch needs every member on the same tile shape.  In order: the
    // members sharing one workgroup per compute unit, then two; each member
    // on the plan that leaves its producers' compute units to them; the
    // plain plans; else one launch per member.
    DecodePlan plans[TB_MAX_GROUP];
    Projection dp[TB_MAX_GROUP];
    int64_t w0_elems = 0;
    for (int j = 0; j < n; ++j) {
      const tb_projection& q = projs[j];
      dp[j] = Projection{q.x, q.s, q.w0, q.u, q.v, q.y, q.out_dim, q.in_dim, q.rank};
      w0_elems += q.out_dim * q.in_dim;
    }
    for (int choice = 0; choice < 4; ++choice) {
      bool same = true;
      if (choice < 2) {
        same = plan_decode_shared(n, dp, m, cus, choice + 1, w0_elems, plans);
        // Two workgroups per compute unit only where the variant's registers
        // allow it (bf16 tiles below 12 = NT x TILES; fp32 holds one).
        if (same && choice == 1 && !decode_fits_two_per_cu(dtype, plans[0].NT, plans[0].TILES)) same = false;
      } else {
        for (int j = 0; j < n; ++j) {
          const tb_projection& q = projs[j];
          plans[j] = choice == 2 ? plan_decode_spared(m, q.out_dim, q.in_dim, q.rank, cus, w0_elems)
                                 : plan_decode(m, q.out_dim, q.in_dim, q.rank, cus, cus, w0_elems);
          same = same && plans[j].NT == plans[0].NT && plans[j].TILES == plans[0].TILES;
        }
      }
      // Each member's buffers fit its share of the workspace (by construction).
      for (int j = 0; j < n && same; ++j)
        same = plans[j].bytes <= forward_data_bytes(m, projs[j].out_dim, projs[j].in_dim, projs[j].rank, dtype, cus);
      if (same) {
        hipError_t e = launch_forward_decode_group(n, plans, dp, dtype, m, ctrl, ws + kControlBytes, err, hs);
        if (e != hipSuccess) return hip_fail(e, "launching the grouped decode projections");
        return ok();
      }
    }
  }
  if (fused_prefill(n, projs, m, dtype)) {
    // One x . V launch and one GEMM launch for every member, in control
    // block 0, with the buffers from the data base.
    Projection gp[TB_MAX_GROUP];
    for (int j = 0; j < n; ++j) {
      const tb_projection& q = projs[j];
      gp[j] = Projection{q.x, q.s, q.w0, q.u, q.v, q.y, q.out_dim, q.in_dim, q.rank};
    }
    const GemmPlan p = fused_prefill_plan(n, projs, m, cus);
    hipError_t e = launch_forward_gemm(p, gp, m, projs[0].in_dim, projs[0].rank, ctrl, ws + kControlBytes, err, hs);
    if (e != hipSuccess) return hip_fail(e, "launching the grouped prefill projections");
    return ok();
  }
  for (int j = 0; j < n; ++j) {
    const tb_projection& q = projs[j];
    tb_status st = forward_one(q.x, q.s, q.w0, q.u, q.v, q.y, m, q.out_dim, q.in_dim, q.rank, dtype,
                               ctrl + j * (kCtrlBlockBytes / 4), ws + off[j], err, cus, hs);
    if (st != TB_OK) return st;
  }
  return ok();
}

tb_status tb_reconstruct_weight(const void* s, const void* w0, const void* u, const void* v, void* w_out,
                                int64_t out_dim, int64_t in_dim, int64_t rank, tb_dtype in_dtype, tb_dtype out_dtype,
                                void* stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(TB_ERR_INVALID_ARGUMENT, "unknown dtype");
  tb_status st = check_dims(1, out_dim, in_dim, rank);
  if (st != TB_OK) return st;
  if (!s || !w0 || !w_out) return fail(TB_ERR_INVALID_ARGUMENT, "s, w0 and w_out must be non-NULL");
  if (rank > 0 && (!u || !v)) return fail(TB_ERR_INVALID_ARGUMENT, "u and v must be non-NULL when rank > 0");
  if (!aligned16(w0) || !aligned16(w_out) || (rank > 0 && (!aligned16(u) || !aligned16(v))))
    return fail(TB_ERR_UNSUPPORTED, "w0, w_out, u and v must be 16-byte aligned");
  if (!aligned_to(s, esize(in_dtype))) return fail(TB_ERR_UNSUPPORTED, "s must be aligned to its element size");
  hipError_t e = launch_reconstruct(in_dtype, out_dtype, s, w0, u, v, w_out, out_dim, in_dim, rank,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching reconstruct");
  return ok();
}

tb_status tb_reconstruction_error(const void* s, const void* w0, const void* u, const void* v, const void* original,
                                  int64_t out_dim, int64_t in_dim, int64_t rank, tb_dtype bundle_dtype,
                                  tb_dtype original_dtype, double* result_device, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!valid_dtype(bundle_dtype) || !valid_dtype(original_dtype)) return fail(TB_ERR_INVALID_ARGUMENT, "unknown dtype");
  tb_status st = check_dims(1, out_dim, in_dim, rank);
  if (st != TB_OK) return st;
  if (!s || !w0 || !original || !result_device || !workspace)
    return fail(TB_ERR_INVALID_ARGUMENT, "s, w0, original, result and workspace must be non-NULL");
  if (rank > 0 && (!u || !v)) return fail(TB_ERR_INVALID_ARGUMENT, "u and v must be non-NULL when rank > 0");
  if (!aligned16(w0) || !aligned16(original) || (rank > 0 && (!aligned16(u) || !aligned16(v))))
    return fail(TB_ERR_UNSUPPORTED, "w0, original, u and v must be 16-byte aligned");
  if (!aligned_to(s, esize(bundle_dtype))) return fail(TB_ERR_UNSUPPORTED, "s must be aligned to its element size");
  if (!aligned_to(result_device, 8) || !aligned_to(workspace, 16))
    return fail(TB_ERR_UNSUPPORTED, "result must be 8-byte and workspace 16-byte aligned");
  if (workspace_bytes < TB_FROBENIUS_WORKSPACE_BYTES)
    return fail(TB_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is below %d", workspace_bytes,
                TB_FROBENIUS_WORKSPACE_BYTES);
  if (out_dim > (int64_t(1) << 40) / in_dim) return fail(TB_ERR_UNSUPPORTED, "matrix too large");
  int cus = 0;
  if (int e = device_cu_count(&cus)) return hip_fail(hipError_t(e), "querying the compute-unit count");
  hipError_t e = launch_reconstruction_error(bundle_dtype, original_dtype, s, w0, u, v, original, out_dim, in_dim, rank,
                                             result_device, workspace, cus, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching the reconstruction error");
  return ok();
}

tb_status tb_rel_frobenius_error(const void* original, const void* reconstructed, int64_t rows, int64_t cols,
                                 tb_dtype dtype, double* result_device, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!valid_dtype(dtype)) return fail(TB_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(dtype));
  if (!original || !reconstructed || !result_device || !workspace)
    return fail(TB_ERR_INVALID_ARGUMENT, "original, reconstructed, result and workspace must be non-NULL");
  if (rows < 1 || cols < 1) return fail(TB_ERR_INVALID_ARGUMENT, "rows and cols must be >= 1");
  if (rows > (int64_t(1) << 40) / cols) return fail(TB_ERR_UNSUPPORTED, "matrix too large");
  if (cols % 8 != 0) return fail(TB_ERR_UNSUPPORTED, "cols %lld is not a multiple of 8", (long long)cols);
  if (!aligned16(original) || !aligned16(reconstructed))
    return fail(TB_ERR_UNSUPPORTED, "original and reconstructed must be 16-byte aligned");
  if (!aligned_to(result_device, 8) || !aligned_to(workspace, 16))
    return fail(TB_ERR_UNSUPPORTED, "result must be 8-byte and workspace 16-byte aligned");
  if (workspace_bytes < TB_FROBENIUS_WORKSPACE_BYTES)
    return fail(TB_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is below %d", workspace_bytes, TB_FROBENIUS_WORKSPACE_BYTES);
  int cus = 0;
  if (int e = device_cu_count(&cus)) return hip_fail(hipError_t(e), "querying the compute-unit count");
  hipError_t e = launch_frobenius(dtype, original, reconstructed, rows * cols, result_device, workspace, cus,
                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching the Frobenius reduction");
  return ok();
}

tb_status tb_shared_block(const void* const* weights, int32_t n, int64_t out_dim, int64_t in_dim, tb_dtype weight_dtype,
                          float* w0_out, void* stream) {
  if (!valid_dtype(weight_dtype)) return fail(TB_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(weight_dtype));
  if (!weights || !w0_out) return fail(TB_ERR_INVALID_ARGUMENT, "weights and w0_out must be non-NULL");
  if (n < 1 || n > TB_MAX_BAND_LAYERS) return fail(TB_ERR_INVALID_ARGUMENT, "n %d outside [1, %d]", n, TB_MAX_BAND_LAYERS);
  if (out_dim < 1 || in_dim < 1) return fail(TB_ERR_INVALID_ARGUMENT, "out_dim and in_dim must be >= 1");
  if (out_dim > kMaxDim / in_dim) return fail(TB_ERR_UNSUPPORTED, "matrix too large");
  for (int j = 0; j < n; ++j) {
    if (!weights[j]) return fail(TB_ERR_INVALID_ARGUMENT, "weights[%d] is NULL", j);
    if (!aligned_to(weights[j], esize(weight_dtype))) return fail(TB_ERR_INVALID_ARGUMENT, "weights[%d] misaligned", j);
  }
  if (!aligned_to(w0_out, 4)) return fail(TB_ERR_INVALID_ARGUMENT, "w0_out misaligned");
  hipError_t e = launch_shared_block(weight_dtype, weights, n, out_dim * in_dim, w0_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching the shared block");
  return ok();
}

tb_status tb_row_scale(const void* weight, const float* w0, int64_t out_dim, int64_t in_dim, tb_dtype weight_dtype,
                       float* s_out, void* stream) {
  if (!valid_dtype(weight_dtype)) return fail(TB_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(weight_dtype));
  if (!weight || !w0 || !s_out) return fail(TB_ERR_INVALID_ARGUMENT, "weight, w0 and s_out must be non-NULL");
  if (out_dim < 1 || in_dim < 1) return fail(TB_ERR_INVALID_ARGUMENT, "out_dim and in_dim must be >= 1");
  if (out_dim > kMaxDim / in_dim || out_dim > 0x7fffffff) return fail(TB_ERR_UNSUPPORTED, "matrix too large");
  if (!aligned_to(weight, esize(weight_dtype)) || !aligned_to(w0, 4) || !aligned_to(s_out, 4))
    return fail(TB_ERR_INVALID_ARGUMENT, "weight, w0 or s_out misaligned");
  hipError_t e = launch_row_scale(weight_dtype, weight, w0, out_dim, in_dim, s_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching the row scale");
  return ok();
}

namespace {

tb_status check_lowrank_dims(int64_t out_dim, int64_t in_dim, int64_t rank, int64_t k) {
  if (out_dim < 1 || in_dim < 1) return fail(TB_ERR_INVALID_ARGUMENT, "out_dim and in_dim must be >= 1");
  if (rank < 0 || k < rank) return fail(TB_ERR_INVALID_ARGUMENT, "need 0 <= rank <= k (got %lld, %lld)", (long long)rank,
                                        (long long)k);
  if (k < 1 || k > out_dim || k > in_dim)
    return fail(TB_ERR_INVALID_ARGUMENT, "k %lld outside [1, min(out_dim, in_dim)]", (long long)k);
  if (k > TB_MAX_PROBE) return fail(TB_ERR_UNSUPPORTED, "k %lld above %d", (long long)k, TB_MAX_PROBE);
  if (out_dim >= (int64_t(1) << 31) / in_dim) return fail(TB_ERR_UNSUPPORTED, "out_dim * in_dim must stay below 2^31");
  return TB_OK;
}

}  // namespace

tb_status tb_lowrank_factors_workspace_size(int64_t out_dim, int64_t in_dim, int64_t rank, int64_t k, size_t* bytes_out) {
  if (!bytes_out) return fail(TB_ERR_INVALID_ARGUMENT, "bytes_out is NULL");
  tb_status st = check_lowrank_dims(out_dim, in_dim, rank, k);
  if (st != TB_OK) return st;
  int cus = 0;
  if (int e = device_cu_count(&cus)) return hip_fail(hipError_t(e), "querying the compute-unit count");
  *bytes_out = lowrank_workspace_bytes(out_dim, in_dim, k, rank, cus);
  return ok();
}

tb_status tb_lowrank_factors(const void* weight, const float* w0, const float* s, int64_t out_dim, int64_t in_dim,
                             int64_t rank, tb_dtype weight_dtype, const float* omega, int64_t k, int32_t power_iters,
                             float* u_out, float* v_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(weight_dtype)) return fail(TB_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(weight_dtype));
  tb_status st = check_lowrank_dims(out_dim, in_dim, rank, k);
  if (st != TB_OK) return st;
  if (power_iters < 0 || power_iters > 16) return fail(TB_ERR_INVALID_ARGUMENT, "power_iters %d outside [0, 16]", power_iters);
  if (!weight || !w0 || !s || !omega || !workspace)
    return fail(TB_ERR_INVALID_ARGUMENT, "weight, w0, s, omega and workspace must be non-NULL");
  if (rank > 0 && (!u_out || !v_out)) return fail(TB_ERR_INVALID_ARGUMENT, "u_out and v_out must be non-NULL");
  if (!aligned_to(weight, esize(weight_dtype)) || !aligned_to(w0, 4) || !aligned_to(s, 4) || !aligned_to(omega, 4) ||
      !aligned_to(u_out, 4) || !aligned_to(v_out, 4))
    return fail(TB_ERR_INVALID_ARGUMENT, "a pointer is misaligned");
  if (!aligned_to(workspace, 256)) return fail(TB_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  int cus = 0;
  if (int e = device_cu_count(&cus)) return hip_fail(hipError_t(e), "querying the compute-unit count");
  const size_t need = lowrank_workspace_bytes(out_dim, in_dim, k, rank, cus);
  if (workspace_bytes < need)
    return fail(TB_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  if (rank == 0) return ok();
  const char* what = "";
  const void* const weights[1] = {weight};
  const float* const w0s[1] = {w0};
  const int e = launch_lowrank_factors(weight_dtype, weights, 1, w0s, s, out_dim, in_dim, rank, omega, k, power_iters,
                                       u_out, v_out, workspace, cus, static_cast<hipStream_t>(stream), &what);
  if (e == -1) return fail(TB_ERR_HIP, "%s failed", what);
  if (e != 0) return hip_fail(hipError_t(e), what);
  return ok();
}

tb_status tb_lowrank_factors_batch(const void* const* weights, int32_t n, const float* const* w0s, const float* s,
                                   int64_t out_dim, int64_t in_dim, int64_t rank, tb_dtype weight_dtype,
                                   const float* omega, int64_t k, int32_t power_iters, float* u_out, float* v_out,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(weight_dtype)) return fail(TB_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(weight_dtype));
  if (!weights) return fail(TB_ERR_INVALID_ARGUMENT, "weights must be non-NULL");
  if (n < 1 || n > TB_MAX_BAND_LAYERS) return fail(TB_ERR_INVALID_ARGUMENT, "n %d outside [1, %d]", n, TB_MAX_BAND_LAYERS);
  tb_status st = check_lowrank_dims(out_dim, in_dim, rank, k);
  if (st != TB_OK) return st;
  if (power_iters < 0 || power_iters > 16) return fail(TB_ERR_INVALID_ARGUMENT, "power_iters %d outside [0, 16]", power_iters);
  if (!w0s || !s || !omega || !workspace)
    return fail(TB_ERR_INVALID_ARGUMENT, "w0s, s, omega and workspace must be non-NULL");
  if (rank > 0 && (!u_out || !v_out)) return fail(TB_ERR_INVALID_ARGUMENT, "u_out and v_out must be non-NULL");
  for (int j = 0; j < n; ++j) {
    if (!weights[j] || !w0s[j]) return fail(TB_ERR_INVALID_ARGUMENT, "weights[%d] or w0s[%d] is NULL", j, j);
    if (!aligned_to(weights[j], esize(weight_dtype)) || !aligned_to(w0s[j], 4))
      return fail(TB_ERR_INVALID_ARGUMENT, "weights[%d] or w0s[%d] misaligned", j, j);
  }
  if (!aligned_to(s, 4) || !aligned_to(omega, 4) || !aligned_to(u_out, 4) || !aligned_to(v_out, 4))
    return fail(TB_ERR_INVALID_ARGUMENT, "a pointer is misaligned");
  if (!aligned_to(workspace, 256)) return fail(TB_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  int cus = 0;
  if (int e = device_cu_count(&cus)) return hip_fail(hipError_t(e), "querying the compute-unit count");
  const size_t need = size_t(n) * lowrank_workspace_bytes(out_dim, in_dim, k, rank, cus);
  if (workspace_bytes < need)
    return fail(TB_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  if (rank == 0) return ok();
  const char* what = "";
  const int e = launch_lowrank_factors(weight_dtype, weights, n, w0s, s, out_dim, in_dim, rank, omega, k, power_iters,
                                       u_out, v_out, workspace, cus, static_cast<hipStream_t>(stream), &what);
  if (e == -1) return fail(TB_ERR_HIP, "%s failed", what);
  if (e != 0) return hip_fail(hipError_t(e), what);
  return ok();
}

tb_status tb_refine_shared_block_workspace_size(int64_t out_dim, int64_t in_dim, int32_t n, int64_t rank,
                                                size_t* bytes_out) {
  if (!bytes_out) return fail(TB_ERR_INVALID_ARGUMENT, "bytes_out is NULL");
  if (out_dim < 1 || in_dim < 1 || rank < 0) return fail(TB_ERR_INVALID_ARGUMENT, "need out_dim, in_dim >= 1, rank >= 0");
  if (n < 1 || n > TB_MAX_BAND_LAYERS) return fail(TB_ERR_INVALID_ARGUMENT, "n %d outside [1, %d]", n, TB_MAX_BAND_LAYERS);
  *bytes_out = refine_workspace_bytes(out_dim, in_dim, n, rank);
  return ok();
}

tb_status tb_refine_shared_block(const void* const* weights, const float* const* s, const float* const* u,
                                 const float* const* v, int32_t n, int64_t out_dim, int64_t in_dim, int64_t rank,
                                 tb_dtype weight_dtype, const float* w0_prev, float* w0_out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!valid_dtype(weight_dtype)) return fail(TB_ERR_INVALID_ARGUMENT, "unknown dtype %d", int(weight_dtype));
  if (!weights || !s || !w0_prev || !w0_out || !workspace)
    return fail(TB_ERR_INVALID_ARGUMENT, "weights, s, w0_prev, w0_out and workspace must be non-NULL");
  if (n < 1 || n > TB_MAX_BAND_LAYERS) return fail(TB_ERR_INVALID_ARGUMENT, "n %d outside [1, %d]", n, TB_MAX_BAND_LAYERS);
  if (out_dim < 1 || in_dim < 1 || rank < 0) return fail(TB_ERR_INVALID_ARGUMENT, "need out_dim, in_dim >= 1, rank >= 0");
  if (out_dim >= (int64_t(1) << 31) / in_dim || rank > TB_MAX_PROBE)
    return fail(TB_ERR_UNSUPPORTED, "out_dim * in_dim must stay below 2^31 and rank at most %d", TB_MAX_PROBE);
  if (rank > 0 && (!u || !v)) return fail(TB_ERR_INVALID_ARGUMENT, "u and v must be non-NULL when rank > 0");
  for (int j = 0; j < n; ++j) {
    if (!weights[j] || !s[j] || (rank > 0 && (!u[j] || !v[j])))
      return fail(TB_ERR_INVALID_ARGUMENT, "member %d has a NULL pointer", j);
    if (!aligned_to(weights[j], esize(weight_dtype)) || !aligned_to(s[j], 4) ||
        (rank > 0 && (!aligned_to(u[j], 4) || !aligned_to(v[j], 4))))
      return fail(TB_ERR_INVALID_ARGUMENT, "member %d is misaligned", j);
  }
  if (!aligned_to(w0_prev, 4) || !aligned_to(w0_out, 4) || !aligned_to(workspace, 256))
    return fail(TB_ERR_INVALID_ARGUMENT, "w0_prev, w0_out or workspace misaligned");
  if (workspace_bytes < refine_workspace_bytes(out_dim, in_dim, n, rank))
    return fail(TB_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is below the %zu needed", workspace_bytes,
                refine_workspace_bytes(out_dim, in_dim, n, rank));
  const char* what = "";
  const int e = launch_refine_shared_block(weight_dtype, weights, s, rank > 0 ? u : nullptr, rank > 0 ? v : nullptr, n,
                                           out_dim, in_dim, rank, w0_prev, w0_out, workspace,
                                           static_cast<hipStream_t>(stream), &what);
  if (e == -1) return fail(TB_ERR_HIP, "%s failed", what);
  if (e != 0) return hip_fail(hipError_t(e), what);
  return ok();
}

tb_status tb_debug_set_wait_polls(int32_t polls) {
  if (polls < 0) return fail(TB_ERR_INVALID_ARGUMENT, "polls %d < 0", polls);
  g_wait_polls.store(polls, std::memory_order_relaxed);
  return ok();
}

const char* tb_status_string(tb_status status) {
  switch (status) {
    case TB_OK: return "ok";
    case TB_ERR_INVALID_ARGUMENT: return "invalid argument";
    case TB_ERR_UNSUPPORTED: return "unsupported layout or size";
    case TB_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* tb_last_error(void) { return g_last_error; }

}  // extern "C"
