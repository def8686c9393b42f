/*
 * tb.h -- C ABI of the theta-bundle projection library (libtb.so), gfx950.
 *
 * The theta bundle ("The theta bundle", weightless docs, component table)
 * replaces a projection's dense weight [out_dim, in_dim] by
 *     W0 [out_dim, in_dim]   shared by every layer of a band, per family,
 *     s  [out_dim]           per layer, a scale of each output row of W0,
 *     U  [out_dim, rank]     per layer, left factor of the low-rank delta,
 *     V  [in_dim,  rank]     per layer, right factor of the low-rank delta,
 * with the weight rebuilt as diag(s) . W0 + U . V^T.  The band whose W0 a
 * layer uses comes from the contiguous band map ("Banded sharing", section
 * "How layers map to bands").
 *
 * Conventions shared by every entry point
 *   - Matrices are dense, row-major, with the leading dimension equal to the
 *     row length.  All pointers except band_out are DEVICE pointers on the
 *     current HIP device.  The caller owns all memory and the library keeps
 *     no caller pointer after a call returns.  The forward, reconstruct and
 *     error calls allocate and free nothing.  Two exceptions, both held until
 *     the process ends: tb_linear_forward_no_alloc's static device scratch
 *     (one per GPU, set up on its first call there), and the decomposition
 *     calls that multiply through rocBLAS (tb_lowrank_factors,
 *     tb_lowrank_factors_batch, tb_refine_shared_block), which create one
 *     rocBLAS handle per (device, stream) on first use; rocBLAS allocates
 *     that handle's own device workspace then.  Those three calls are
 *     therefore not for HIP graph capture or allocation-free callers.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued on it asynchronously; outputs are valid once
 *     the caller synchronises that stream.  No entry point synchronises.
 *   - Arguments are checked on the host before anything is enqueued.  On any
 *     status other than TB_OK nothing was enqueued and no output was written.
 *     tb_last_error() then describes the problem (per calling thread).
 *   - Matrix base pointers (x, w0, u, v, original, reconstructed, w_out) must
 *     be 16-byte aligned and in_dim / cols must be a multiple of 8; otherwise
 *     the call returns TB_ERR_UNSUPPORTED.  Every Gemma-shaped projection
 *     satisfies this.  s and y need only element alignment.
 *   - Sizes are 64-bit; an element count must fit in int64.
 */
#ifndef TB_H
#define TB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tb_status {
  TB_OK = 0,
  TB_ERR_INVALID_ARGUMENT = 1, /* a NULL pointer, a size out of range, ...  */
  TB_ERR_UNSUPPORTED = 2,      /* alignment / divisibility / dtype combination */
  TB_ERR_HIP = 3               /* the HIP runtime refused a query or launch  */
} tb_status;

typedef enum tb_dtype {
  TB_F32 = 0,  /* IEEE binary32 */
  TB_BF16 = 1  /* bfloat16, round-to-nearest-even on every store */
} tb_dtype;

/* Most projections one tb_linear_forward_group call takes. */
#define TB_MAX_GROUP 8

/* Leading bytes of a forward workspace that hold control words: one block of
 * 64 KiB for each member a grouped call may have (a single call uses block 0). */
#define TB_WORKSPACE_CONTROL_BYTES (TB_MAX_GROUP * 65536)

/* Fixed workspace size of tb_rel_frobenius_error. */
#define TB_FROBENIUS_WORKSPACE_BYTES 65536

/* Most layers one band may hold in tb_shared_block. */
#define TB_MAX_BAND_LAYERS 128

/* Widest random probe (k = rank + oversampling) of tb_lowrank_factors. */
#define TB_MAX_PROBE 512

/*
 * tb_band_index -- band of one layer ("Banded sharing", "How layers map to
 * bands").  The num_layers layers are split into num_bands contiguous bands
 * whose sizes differ by at most one, the earlier bands taking the remainder:
 * with q = num_layers / num_bands and m = num_layers % num_bands, bands
 * 0..m-1 hold q+1 layers and the others q.  num_bands = 1 shares one W0 by
 * all layers; num_bands = num_layers is passthrough (band == layer).
 *
 *   num_layers >= 1, 1 <= num_bands <= num_layers, 0 <= layer < num_layers,
 *   band_out is a HOST pointer.  Host-only and pure; it touches no device.
 *   Errors: TB_ERR_INVALID_ARGUMENT (band_out untouched).
 */
tb_status tb_band_index(int32_t num_layers, int32_t num_bands, int32_t layer, int32_t *band_out);

/*
 * tb_linear_forward_workspace_size -- bytes of workspace tb_linear_forward
 * needs for these sizes on the current device (host-only query; it reads the
 * device's compute-unit count once).  *bytes_out >= TB_WORKSPACE_CONTROL_BYTES.
 */
tb_status tb_linear_forward_workspace_size(int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank,
                                           tb_dtype dtype, size_t *bytes_out);

/*
 * tb_linear_forward -- one theta-bundle projection.
 *
 *     y[t, o] = s[o] * sum_i x[t, i] W0[o, i]  +  sum_j (sum_i x[t, i] V[i, j]) U[o, j]
 *
 * i.e. y = s (.) (x . W0^T) + (x . V) . U^T, the transpose of the
 * reconstruction formula weight = diag(s) W0 + U V^T ("The theta bundle"),
 * applied without forming the weight.  W0 is the block of the layer's band
 * (the caller selects it with tb_band_index).
 *
 *   x  [m, in_dim]        activations              (dtype)
 *   s  [out_dim]          row scale                (dtype; NULL: every row's scale is 1)
 *   w0 [out_dim, in_dim]  shared block             (dtype)
 *   u  [out_dim, rank]    left factor              (dtype; NULL allowed iff rank == 0)
 *   v  [in_dim, rank]     right factor             (dtype; NULL allowed iff rank == 0)
 *   y  [m, out_dim]       output                   (dtype), written, must not alias inputs
 *   m >= 1 tokens, out_dim >= 1, in_dim >= 8 and % 8 == 0, rank >= 0.
 *   Arithmetic: products and sums in fp32 (bf16 inputs are exact in fp32);
 *   the scale multiplies fp32 sums of x . W0^T before the delta is added
 *   (where a reduction over in_dim is split across workgroups, each part's
 *   sum is scaled and the parts are then added in a fixed order); for
 *   bf16 the intermediate x . V is rounded to bf16 before it meets U.  y is
 *   rounded once at the end.  Results are deterministic run to run.  For
 *   m <= 64, in_dim * element size * 96 must stay below 2^32 (else
 *   TB_ERR_UNSUPPORTED).
 *   workspace: device buffer of at least tb_linear_forward_workspace_size()
 *   bytes, 256-byte aligned.  Its first TB_WORKSPACE_CONTROL_BYTES bytes are
 *   control words: they must be zero before the first call that uses the
 *   buffer and must not be changed by the caller afterwards (each completed
 *   call, single or grouped, leaves all of them ready for the next; some
 *   carry state from call to call).  Word 2
 *   (uint32) is a sticky error flag: it becomes nonzero only when a bounded
 *   internal wait times out (the rows of y behind that wait are NaN), and a
 *   timed-out call may leave other control words stale.  While word 2 is set,
 *   every forward call on the workspace (tb_linear_forward, tb_dense_forward,
 *   tb_linear_forward_group) writes NaN to all of its y and reads or writes no
 *   other control word; zeroing the first TB_WORKSPACE_CONTROL_BYTES bytes
 *   again makes the workspace usable.  Calls that may run at the same time
 *   (different streams) must not share a workspace.
 *   Errors: TB_ERR_INVALID_ARGUMENT, TB_ERR_UNSUPPORTED, TB_ERR_HIP.
 */
tb_status tb_linear_forward(const void *x, const void *s, const void *w0, const void *u, const void *v,
                            void *y, int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank,
                            tb_dtype dtype, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the device scratch that tb_linear_forward_no_alloc uses (96 MiB on
 * every GPU the library runs on, held until the process ends). */
#define TB_NO_ALLOC_SCRATCH_BYTES (96u << 20)

/*
 * tb_linear_forward_no_alloc -- tb_linear_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same computation, kernels, results
 * (bit for bit) and argument rules as tb_linear_forward, but the workspace is
 * the library's own static device array of TB_NO_ALLOC_SCRATCH_BYTES on the
 * current device; the call allocates and frees nothing.
 *   Every call on one GPU shares that GPU's array: calls that may overlap on
 *   one GPU (several streams, several host threads) race and must be
 *   serialised by the caller.  Each call first clears the array's control
 *   words (a small kernel on `stream`), so a call whose internal wait timed
 *   out (word 2 set, its y NaN) does not affect the next.  The array keeps
 *   the last call's contents.
 *   Errors: as tb_linear_forward; TB_ERR_UNSUPPORTED when the call would need
 *   more than TB_NO_ALLOC_SCRATCH_BYTES of workspace
 *   (tb_linear_forward_workspace_size tells), with nothing enqueued.
 */
tb_status tb_linear_forward_no_alloc(const void *x, const void *s, const void *w0, const void *u, const void *v,
                                     void *y, int64_t m, int64_t out_dim, int64_t in_dim, int64_t rank,
                                     tb_dtype dtype, void *stream);

/*
 * tb_dense_forward -- y = x . W^T for a weight held whole: the
 * materialise-once serving mode, where W = tb_reconstruct_weight(s, W0, U, V)
 * is formed once in the operand type ("Banded sharing", "Set G for serving":
 * the serve command that precomputes the weight outside the model graph;
 * "Quality": that path costs nothing measurable) and each call then streams
 * W alone.  It is tb_linear_forward with s = NULL (unit scale), rank 0:
 * the same kernels, workspace (tb_linear_forward_workspace_size with rank
 * 0), arithmetic, determinism, limits and errors.
 *
 *   x [m, in_dim], w [out_dim, in_dim], y [m, out_dim], all dtype, device.
 */
tb_status tb_dense_forward(const void *x, const void *w, void *y, int64_t m, int64_t out_dim, int64_t in_dim,
                           tb_dtype dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * One projection of a group: the arguments of tb_linear_forward that may
 * differ between its members (same meaning, layout and alignment rules).
 */
typedef struct tb_projection {
  const void *x;
  const void *s;
  const void *w0;
  const void *u;
  const void *v;
  void *y;
  int64_t out_dim, in_dim, rank;
} tb_projection;

/*
 * tb_linear_forward_group_workspace_size -- bytes of workspace
 * tb_linear_forward_group needs for these projections (only their out_dim,
 * in_dim and rank are read) at m tokens: the control bytes plus each
 * member's buffers.
 */
tb_status tb_linear_forward_group_workspace_size(int32_t n, const tb_projection *projs, int64_t m, tb_dtype dtype,
                                                 size_t *bytes_out);

/*
 * tb_linear_forward_group -- n independent theta-bundle projections (the
 * computation of tb_linear_forward for each member) over the same token
 * count m and dtype.  Layers apply several projections to one input (q/k/v,
 * gate/up); each member still names its own x, which may be shared.  For
 * m <= 64 the members run in one launch when their plans can share one tile
 * shape, so the fixed cost of a launch and the wait for x . V are paid once.
 * For bf16 and m > 64, members that share in_dim and rank run as one x . V
 * launch and one GEMM launch over all their output tiles.  In one launch the
 * chip is shared out between the members, which may split a member's
 * reductions over in_dim differently from its own call, so its result may
 * differ from tb_linear_forward's in the last bits (same error bound; a given
 * group is deterministic run to run).  Other cases run the members one after
 * another, each exactly as its own call.
 *   n: 1 .. TB_MAX_GROUP.  projs: host array of n members (no y may alias
 *   any member's input or another member's y).
 *   workspace: as for tb_linear_forward, at least
 *   tb_linear_forward_group_workspace_size() bytes; member j uses control
 *   block j and its own buffers after the control bytes (a fused prefill
 *   launch uses block 0 and the buffers from the start).  A timed-out wait in
 *   any member sets word 2 of the workspace.
 *   Errors: TB_ERR_INVALID_ARGUMENT, TB_ERR_UNSUPPORTED, TB_ERR_HIP; a
 *   member that fails validation fails the call before anything is launched.
 */
tb_status tb_linear_forward_group(int32_t n, const tb_projection *projs, int64_t m, tb_dtype dtype, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * tb_reconstruct_weight -- w_out = diag(s) . W0 + U . V^T ("The theta bundle",
 * reconstruct_weight(s, W0, U, V)).
 *
 *   s [out_dim], w0 [out_dim, in_dim], u [out_dim, rank], v [in_dim, rank]
 *   in in_dtype; w_out [out_dim, in_dim] in out_dtype.  rank >= 0 (u, v may
 *   be NULL iff rank == 0), in_dim % 8 == 0.  fp32 accumulation; with
 *   rank == 0 and fp32 output the result is exact (s * W0 of bf16 inputs is
 *   representable in fp32).  Errors as above.
 */
tb_status tb_reconstruct_weight(const void *s, const void *w0, const void *u, const void *v, void *w_out,
                                int64_t out_dim, int64_t in_dim, int64_t rank,
                                tb_dtype in_dtype, tb_dtype out_dtype, void *stream);

/*
 * tb_rel_frobenius_error -- ||original - reconstructed||_F / ||original||_F
 * ("Quality", section "Reconstruction error"; the argument order of
 * relative_frobenius_error(original, reconstructed) in "The theta bundle").
 *
 *   original, reconstructed: [rows, cols] in dtype, cols % 8 == 0.
 *   result_device: DEVICE pointer to one double, written.  Differences,
 *   squares and sums are taken in fp64 in a fixed order (deterministic).
 *   When the difference is zero the result is 0; when only the original is
 *   zero it is +inf.  workspace: >= TB_FROBENIUS_WORKSPACE_BYTES device bytes,
 *   16-byte aligned.  Bytes [TB_FROBENIUS_WORKSPACE_BYTES - 8192,
 *   TB_FROBENIUS_WORKSPACE_BYTES) hold arrival counters: zero them before
 *   the first use; every call leaves them zero (the rest needs no
 *   initialisation).  Calls that share a workspace must not overlap (keep
 *   them on one stream).  Errors as above.
 */
tb_status tb_rel_frobenius_error(const void *original, const void *reconstructed, int64_t rows, int64_t cols,
                                 tb_dtype dtype, double *result_device, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * tb_reconstruction_error -- relative_frobenius_error(original,
 * reconstruct_weight(s, W0, U, V)) without writing the rebuilt weight ("The
 * theta bundle", reconstruction formula; "Quality", section "Reconstruction
 * error").  The rebuilt entries are formed in fp32 as tb_reconstruct_weight
 * forms them for fp32 output; differences, squares and sums are taken in
 * fp64 in a fixed order (deterministic).
 *
 *   s [out_dim], w0 [out_dim, in_dim], u [out_dim, rank], v [in_dim, rank]
 *   in bundle_dtype (u, v may be NULL iff rank == 0); original
 *   [out_dim, in_dim] in original_dtype; in_dim % 8 == 0.  result_device:
 *   DEVICE pointer to one double, written (0 when the two agree, +inf when
 *   only the original is zero).  workspace: as for tb_rel_frobenius_error
 *   (same size; the same arrival counters, zero before the first use and left
 *   zero by every call).  Errors as above.
 */
tb_status tb_reconstruction_error(const void *s, const void *w0, const void *u, const void *v, const void *original,
                                  int64_t out_dim, int64_t in_dim, int64_t rank, tb_dtype bundle_dtype,
                                  tb_dtype original_dtype, double *result_device, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Analytic decomposition of one projection family ("The theta bundle",
 * section "Analytic decomposition"), in three steps per band and layer.
 * Outputs are fp32; the caller casts them for the forward path.
 *
 * tb_shared_block -- W0 = the mean of the band's weight matrices (Shared
 * block): summed in layer order in fp64, divided by n, rounded once to fp32.
 *   weights: HOST array of n DEVICE pointers, each [out_dim, in_dim] of
 *   weight_dtype; 1 <= n <= TB_MAX_BAND_LAYERS.  w0_out: device fp32
 *   [out_dim, in_dim].  Errors: TB_ERR_INVALID_ARGUMENT, TB_ERR_HIP.
 */
tb_status tb_shared_block(const void *const *weights, int32_t n, int64_t out_dim, int64_t in_dim,
                          tb_dtype weight_dtype, float *w0_out, void *stream);

/*
 * tb_row_scale -- s[o] = <weight[o], W0[o]> / <W0[o], W0[o]>, the per-row
 * least-squares fit of the weight against its band's block (Per-row scale);
 * 0 for a zero row of W0 (the minimum-norm solution).  fp64 sums in a fixed
 * order, one rounding to fp32.
 *   weight [out_dim, in_dim] (weight_dtype), w0 fp32 [out_dim, in_dim],
 *   s_out fp32 [out_dim], all device.  Errors: TB_ERR_INVALID_ARGUMENT, TB_ERR_HIP.
 */
tb_status tb_row_scale(const void *weight, const float *w0, int64_t out_dim, int64_t in_dim, tb_dtype weight_dtype,
                       float *s_out, void *stream);

/*
 * tb_lowrank_factors_workspace_size -- bytes of workspace tb_lowrank_factors
 * needs (host-only query; it reads the device's compute-unit count once).
 */
tb_status tb_lowrank_factors_workspace_size(int64_t out_dim, int64_t in_dim, int64_t rank, int64_t k,
                                            size_t *bytes_out);

/*
 * tb_lowrank_factors -- U [out_dim, rank], V [in_dim, rank] with U V^T the
 * rank-r cut of the residual E = weight - diag(s) W0 by the randomized SVD
 * the section names for large matrices (Low-rank residual; Halko,
 * Martinsson and Tropp, 2009).  U absorbs the singular values (columns by
 * decreasing singular value); a singular value at or below 1e-7 of the
 * largest counts as zero and gives zero columns in U and V.
 *   omega [in_dim, k] fp32: the random probe, drawn by the caller
 *   (k = rank + oversampling); power_iters re-orthonormalised power
 *   iterations (0..16).  The probe's range is found as in the method: Y = E
 *   omega, orthonormalised; each power iteration maps through E^T and E,
 *   orthonormalising each time; then the SVD of the k x in_dim projection.
 *   With k = min(out_dim, in_dim) the result is the exact truncated SVD up to
 *   rounding.  E is formed in fp32 (one rounding per entry), products in fp32,
 *   Gram matrices, Cholesky factors and the eigen-decomposition in fp64.
 *   weight (weight_dtype), w0, s, omega, u_out, v_out: device, 4-byte aligned.
 *   0 <= rank <= k <= min(out_dim, in_dim, TB_MAX_PROBE); out_dim * in_dim <
 *   2^31.  rank 0 writes nothing.  workspace: at least
 *   tb_lowrank_factors_workspace_size() bytes, 256-byte aligned, no initial
 *   contents.  Calls that may run at the same time must not share it.
 *   Errors: TB_ERR_INVALID_ARGUMENT, TB_ERR_UNSUPPORTED, TB_ERR_HIP (also for
 *   a failing rocBLAS call).
 */
tb_status tb_lowrank_factors(const void *weight, const float *w0, const float *s, int64_t out_dim, int64_t in_dim,
                             int64_t rank, tb_dtype weight_dtype, const float *omega, int64_t k, int32_t power_iters,
                             float *u_out, float *v_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * tb_lowrank_factors_batch -- tb_lowrank_factors for n matrices of one shape
 * (the layers of a projection family, each with its band's W0), in one pass:
 * every step runs on all of them together, so the single-workgroup solvers
 * of the n matrices share the chip.  Each matrix's result equals what
 * tb_lowrank_factors computes for it up to the rounding of the batched
 * products.
 *   weights, w0s: HOST arrays of n DEVICE pointers ([out_dim, in_dim]; weights
 *   of weight_dtype, w0s fp32), 1 <= n <= TB_MAX_BAND_LAYERS; s [n][out_dim],
 *   omega [n][in_dim][k],
 *   u_out [n][out_dim][rank], v_out [n][in_dim][rank], all fp32 device and
 *   contiguous.  workspace: n times tb_lowrank_factors_workspace_size()
 *   bytes, 256-byte aligned.  Other rules and errors as tb_lowrank_factors.
 */
tb_status tb_lowrank_factors_batch(const void *const *weights, int32_t n, const float *const *w0s, const float *s,
                                   int64_t out_dim, int64_t in_dim, int64_t rank, tb_dtype weight_dtype,
                                   const float *omega, int64_t k, int32_t power_iters, float *u_out, float *v_out,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * tb_refine_shared_block -- one least-squares refit of a band's shared block
 * with each layer's scale and factors held fixed, the alternating least
 * squares the "Quality" page reports on (Research: why shared configurations
 * need training): row by row
 *     W0[o] = sum_l s_l[o] (W_l - U_l V_l^T)[o] / sum_l s_l[o]^2,
 * and a row whose scales are all zero keeps its w0_prev value (a reading).
 * num = sum_l diag(s_l) W_l in fp64 sums (layer order, rounded to fp32),
 * minus the n layers' deltas as one fp32 GEMM of inner dimension n * rank
 * (rocBLAS), then the division in fp64.
 *   weights: HOST array of n DEVICE pointers ([out_dim, in_dim], weight_dtype);
 *   s, u, v: HOST arrays of n DEVICE fp32 pointers ([out_dim], [out_dim,
 *   rank], [in_dim, rank]; u, v may be NULL when rank is 0); w0_prev, w0_out:
 *   device fp32 [out_dim, in_dim] (they may be the same buffer).
 *   1 <= n <= TB_MAX_BAND_LAYERS, 0 <= rank <= TB_MAX_PROBE, out_dim *
 *   in_dim < 2^31.  workspace: tb_refine_shared_block_workspace_size()
 *   bytes, 256-byte aligned.  Errors: TB_ERR_INVALID_ARGUMENT,
 *   TB_ERR_UNSUPPORTED, TB_ERR_HIP.
 */
tb_status tb_refine_shared_block_workspace_size(int64_t out_dim, int64_t in_dim, int32_t n, int64_t rank,
                                                size_t *bytes_out);
tb_status tb_refine_shared_block(const void *const *weights, const float *const *s, const float *const *u,
                                 const float *const *v, int32_t n, int64_t out_dim, int64_t in_dim, int64_t rank,
                                 tb_dtype weight_dtype, const float *w0_prev, float *w0_out, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * tb_debug_set_wait_polls -- bound, in polls about 0.1 us apart, of the
 * forward kernels' internal waits (a decode streamer waiting for the x . V
 * products of its launch; a k-slice of a split prefill tile waiting for the
 * tile's other slices); default 1 << 20 (about 0.1 s).  It applies to
 * launches enqueued after the call, process-wide.  For tests of the timeout
 * path: 0 makes every such wait give up at once, so word 2 of the workspace
 * is set and y is NaN, with every kernel exiting normally.
 *   polls >= 0.  Errors: TB_ERR_INVALID_ARGUMENT.  Host-only.
 */
tb_status tb_debug_set_wait_polls(int32_t polls);

/* Static description of a status code. */
const char *tb_status_string(tb_status status);

/* Description of the last failure on the calling thread ("" if none). */
const char *tb_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TB_H */
