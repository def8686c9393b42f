// Host-side internals of libtb: launch plans and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tb.h"

namespace tb {

// The workspace starts with kControlBytes of control words: one block of
// kCtrlBlockBytes per member of a grouped call (a single call uses block 0).
// Each projection's buffers follow, at offsets its plan gives from its data
// base; plan.bytes counts the buffers only.
constexpr int kMaxProjections = TB_MAX_GROUP;
constexpr size_t kControlBytes = TB_WORKSPACE_CONTROL_BYTES;
constexpr size_t kCtrlBlockBytes = kControlBytes / kMaxProjections;
// Layout of a control block, in 32-bit words: 0 .. 63 single words (word 2:
// the sticky error flag, word 3: the parity of the x . V exchange);
// 64 .. 64 + kMaxGroupCounters the per-block arrival counters; then the decode
// launches' x . V exchange, two halves of kTHalfWords (T coded so that a zero
// word means "not written yet"; a launch uses the half its parity names and
// clears the other); the last kFinishWords the decode rank streamers' finish
// counters (16 group counters and a top counter, 64 words apart).  Between
// calls every word is zero except the parity word and the exchange half the
// next call does not use.
constexpr int kFinishWords = 17 * 64;
constexpr int kMaxGroupCounters = 1024;
constexpr int kTWordBase = 64 + kMaxGroupCounters;
constexpr int kTHalfWords = (int(kCtrlBlockBytes / 4) - kFinishWords - kTWordBase) / 2 / 64 * 64;
static_assert(kTHalfWords >= 4096, "a half holds 16 tokens x rank 256 in fp32");

// Compute units of the current device (queried once per device).
int device_cu_count(int* cus);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// One projection of a launch: device operands and output, and its shape.
struct Projection {
  const void* x;
  const void* s;
  const void* w0;
  const void* u;
  const void* v;
  void* y;
  int64_t out_dim, in_dim, rank;
};

// ---- forward, skinny token counts (m <= kDecodeMaxTokens) -----------------
constexpr int kDecodeMaxTokens = 64;

// Bound of the decode streamers' wait for x . V, in polls (default 1 << 20,
// about 0.1 s); tb_debug_set_wait_polls changes it for later launches.
int decode_wait_polls();

struct DecodePlan {
  int NT;        // 16-token column tiles (1, 2 or 4)
  int TILES;     // 16-row tiles each streaming workgroup is built for (1, 2, 4 or 6)
  int NRB, KS;   // streaming row blocks and k-slices of in_dim
  int NB;        // streaming workgroups (NRB * KS)
  int NCB, KT;   // x . V producers: 16-column blocks of T and k-slices of in_dim
  int NP;        // producer workgroups (NCB * KT)
  size_t off_tpart, off_tfull, off_ypart, bytes;
};

// streamers: the streaming workgroups to aim for (about one per compute
// unit); cus: the compute units; stream_elems: the W0 elements of the whole
// launch, whose share per compute unit sets how long the producers'
// k-slices may be.
DecodePlan plan_decode(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, int streamers, int cus,
                       int64_t stream_elems);
// The same with the producers' compute units left to them when they are few
// (under a quarter of the chip): a streamer that shares a compute unit with a
// producer finishes several microseconds after the others.
DecodePlan plan_decode_spared(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, int cus, int64_t stream_elems);

// ctrl: the projection's control block; data: its buffers; err_word: where a
// timed-out wait is flagged.
hipError_t launch_forward_decode(const DecodePlan& p, tb_dtype dtype, const void* x, const void* s, const void* w0,
                                 const void* u, const void* v, void* y, int64_t m, int64_t out_dim, int64_t in_dim,
                                 int64_t rank, unsigned* ctrl, char* data, unsigned* err_word, hipStream_t stream);

// Several independent projections of the same token count (<= kDecodeMaxTokens)
// in one launch.  Their plans must agree on NT and TILES.  Projection j uses
// control block j (from ctrl) and the buffers after the plans[0..j-1] bytes
// (from data); timeouts of any member set *err_word.
hipError_t launch_forward_decode_group(int n, const DecodePlan* plans, const Projection* projs, tb_dtype dtype,
                                       int64_t m, unsigned* ctrl, char* data, unsigned* err_word, hipStream_t stream);

// Workgroups per compute unit that a shared plan may fill (the decode kernel
// keeps two resident per compute unit; one for 32 tokens x 96 rows and for
// 64 tokens x 64 or 96 rows).
constexpr int kMaxDecodeSlots = 2;
// Whether a decode variant's registers leave room for two workgroups per
// compute unit (four waves per SIMD).
inline bool decode_fits_two_per_cu(tb_dtype dtype, int NT, int TILES) { return dtype == TB_BF16 && NT * TILES < 12; }
// Plans for the members of one launch that share slots * cus workgroups:
// every producer keeps its workgroup and the streamers are shared out in
// proportion to each member's W0 bytes.  False when the members would not
// agree on one tile shape or would need more workgroups than that.
bool plan_decode_shared(int n, const Projection* projs, int64_t m, int cus, int slots, int64_t stream_elems,
                        DecodePlan* plans);
// Data bytes that cover the plan of any streamer budget up to
// kMaxDecodeSlots * cus.
size_t decode_bytes_bound(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank, int cus);

// ---- forward, prefill token counts (bf16, m > kDecodeMaxTokens) ----------
// One launch of each kernel covers n projections that share the token count,
// in_dim and rank (a single call: n = 1; q, k, v or gate, up of a layer: one
// launch for all of them).  Output tiles are numbered member after member.
struct GemmPlan {
  int n;                // projections in the launch
  int aligned;          // in_dim and rank multiples of 8: x . V by the transposing-read kernel
  int big;              // 1: 256 x 256 kernel (needs aligned); 0: general 128 x 128 kernel
  int grid;             // workgroups (persistent for the 256 x 256 kernel, one per tile for the general one)
  int tiles_m;          // token tiles (256 or 128 rows)
  int tiles_n[kMaxProjections];      // each member's output-column tiles
  int start[kMaxProjections + 1];    // first tile of each member; start[n] = all tiles
  int KT, KR;           // k-tiles (64) of in_dim and of rank
  int split_tiles;      // leading tiles split into S k-slices of kps k-tiles (the remainder round)
  int S, kps;
  int xcd_major;        // workgroup positions spread XCD-major (grid a multiple of 8)
  int xv_rb, xv_cb;     // x . V on the aligned path: 64-token row blocks, column blocks of T (per member)
  int xv_bm, xv_bn;     // tokens and columns of a T block
  int xv_kt, xv_ks, xv_kps;  // its k-tiles (64), k-slices and k-tiles per slice
  size_t off_t[kMaxProjections];  // each member's T (m x rank bf16) from the data base
  size_t off_xvpart, off_part, bytes;
};
// out_dims: the n members' output widths.
GemmPlan plan_gemm(int n, const int64_t* out_dims, int64_t m, int64_t in_dim, int64_t rank, int cus);

// ctrl: the launch's control block (arrival counters); data: the plan's
// buffers; err_word: the sticky error word of the workspace; while it is set
// the launch writes NaN to every y and touches no counter.
hipError_t launch_forward_gemm(const GemmPlan& p, const Projection* projs, int64_t m, int64_t in_dim, int64_t rank,
                               unsigned* ctrl, char* data, const unsigned* err_word, hipStream_t stream);

// ---- reconstruct ----------------------------------------------------------
hipError_t launch_reconstruct(tb_dtype in_dtype, tb_dtype out_dtype, const void* s, const void* w0, const void* u,
                              const void* v, void* w_out, int64_t out_dim, int64_t in_dim, int64_t rank,
                              hipStream_t stream);

// ---- reconstruction error without the rebuilt weight -----------------------
// bf16 bundles of rank 193..256 (multiple of 8) against an fp32 original: the
// persistent direct-to-LDS rebuild kernel with an error epilogue.
bool persistent_error_supported(int64_t out_dim, int64_t in_dim, int64_t rank);
hipError_t launch_reconstruction_error_persistent(const void* s, const void* w0, const void* u, const void* v,
                                                  const float* orig, int64_t out_dim, int64_t in_dim, int64_t rank,
                                                  double* result, void* workspace, int cus, hipStream_t stream);
hipError_t launch_reconstruction_error(tb_dtype bundle_dtype, tb_dtype orig_dtype, const void* s, const void* w0,
                                       const void* u, const void* v, const void* orig, int64_t out_dim, int64_t in_dim,
                                       int64_t rank, double* result, void* workspace, int cus, hipStream_t stream);

// ---- relative Frobenius error ---------------------------------------------
hipError_t launch_frobenius(tb_dtype dtype, const void* a, const void* b, int64_t n, double* result,
                            void* workspace, int cus, hipStream_t stream);

// ---- analytic decomposition (decompose.hip) ---------------------------------
hipError_t launch_shared_block(tb_dtype dtype, const void* const* weights, int n, int64_t count, float* out,
                               hipStream_t stream);
hipError_t launch_row_scale(tb_dtype dtype, const void* weight, const float* w0, int64_t out_dim, int64_t in_dim,
                            float* s, hipStream_t stream);
// Least-squares refit of one band's shared block from its n layers' weights,
// scales and factors (u, v may be NULL when rank is 0).
size_t refine_workspace_bytes(int64_t out_dim, int64_t in_dim, int64_t n, int64_t rank);
int launch_refine_shared_block(tb_dtype dtype, const void* const* weights, const float* const* s,
                               const float* const* u, const float* const* v, int n, int64_t out_dim, int64_t in_dim,
                               int64_t rank, const float* prev, float* out, void* workspace, hipStream_t stream,
                               const char** what);
// Bytes of one matrix's workspace slice; a batch of n takes n slices.
size_t lowrank_workspace_bytes(int64_t out_dim, int64_t in_dim, int64_t k, int64_t rank, int cus);
// A batch of n matrices of one shape, each with its W0: s [n][out], omega [n][in][k],
// u_out [n][out][rank], v_out [n][in][rank].  0 on success; a hipError_t
// code, or -1 for a rocBLAS failure, with *what naming the step.
int launch_lowrank_factors(tb_dtype dtype, const void* const* weights, int n, const float* const* w0s, const float* s,
                           int64_t out_dim, int64_t in_dim, int64_t rank, const float* omega, int64_t k, int power_iters,
                           float* u_out, float* v_out, void* workspace, int cus, hipStream_t stream, const char** what);

}  // namespace tb
