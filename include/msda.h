/*
 * msda.h - C ABI of the MI355X (gfx950) multi-scale deformable attention core.
 *
 * The operator is the bracket of Deformable DETR's Eq. 1 as chapter 1 of the
 * msda-triton course defines it ("1. Deformable attention, from scratch",
 * sections "The equation, term by term", "Bilinear interpolation: reading
 * between the pixels" and "The simplest possible implementation"): for every
 * batch b, query q and head m,
 *
 *   out[b, q, m*D + d] = sum_{l<L} sum_{k<K} A[b,q,m,l,k] * bilinear_l(x, y)[d]
 *
 * where (x, y) = (loc_x * W_l - 0.5, loc_y * H_l - 0.5) is the pixel-centre
 * mapping of sampling_locations[b,q,m,l,k,:], the bilinear sample blends the
 * four surrounding pixels of level l of value[b, :, m, :], and a corner that
 * falls outside the H_l x W_l map contributes zero.  Attention weights are
 * used as given (the DeformOps page, section "Multi-scale deformable
 * attention", describes that default).  The backward returns the gradients of
 * <out, grad_out> with respect to value, sampling_locations and
 * attention_weights.  The *_softmax entry points implement the same page's
 * "softmax" method: they take raw attention logits z of the same shape and
 * use A = softmax of z over the L*K samples of each (b, q, m).
 *
 * Tensor layouts (all row-major, contiguous, on the device that runs the
 * stream):
 *   value               [B, S, M, D]        S = sum_l H_l * W_l
 *   spatial_shapes      [L, 2] int64        rows (H_l, W_l)
 *   level_start_index   [L]    int64        exclusive prefix sum of H_l * W_l
 *   sampling_locations  [B, Q, M, L, K, 2]  last axis (x, y), normalised
 *   attention_weights   [B, Q, M, L, K]
 *   out, grad_out       [B, Q, M * D]
 *   grad_value          [B, S, M, D]
 *   grad_loc            [B, Q, M, L, K, 2]
 *   grad_attn           [B, Q, M, L, K]
 * All floating tensors of one call share `dtype`.  spatial_shapes and
 * level_start_index are device pointers; they are read by the kernels only.
 *
 * Conventions shared by every entry point:
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     allocates no device memory, frees nothing and keeps no pointer after
 *     the call returns.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream) and the call returns without waiting for it.  Buffers must
 *     stay valid until that work completes.  A workspace holds the call's
 *     intermediate state until then: calls whose work may overlap (on
 *     different streams) need workspaces of their own.
 *   - Outputs are overwritten, never accumulated into.
 *   - Errors: a non-OK status is returned before anything is enqueued when the
 *     arguments are rejected; msda_last_error() then describes the reason.
 *     MSDA_ERR_HIP reports a failed launch.
 *   - Supported: dtype FP32, BF16 or FP16 (IEEE binary16); D in {8, 16, 32, 64}; 1 <= L <= 16;
 *     1 <= K <= 32; L*K <= 64; B, Q >= 0; S >= 1; M >= 1; one batch image of
 *     value (S*M*D elements) below 2^30 bytes; every element count below 2^62.
 *     Float pointers must be 16-byte aligned.  Anything else returns
 *     MSDA_ERR_UNSUPPORTED / MSDA_ERR_INVALID_DIMS / MSDA_ERR_MISALIGNED.
 *   - Trusted preconditions (device data the host cannot inspect without a
 *     sync): H_l, W_l >= 1, level_start_index is the prefix sum of H_l*W_l and
 *     S >= its last entry + H_{L-1} * W_{L-1}.  If they are violated the
 *     results are wrong, but every memory access stays inside value and
 *     grad_value (reads and atomics go through range-checked buffer
 *     descriptors).
 *   - Sampling locations may be any float, including NaN and +-Inf: a sample
 *     none of whose four corners lies inside its level contributes nothing
 *     and receives zero gradients.
 *   - Reentrant and thread-safe: no global mutable state apart from the
 *     thread-local error string (and the thread-local test hook of
 *     msda_bench.h).
 */
#ifndef MSDA_H
#define MSDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MSDA_OK = 0,
    MSDA_ERR_NULL_POINTER = 1,
    MSDA_ERR_INVALID_DIMS = 2,
    MSDA_ERR_UNSUPPORTED = 3,
    MSDA_ERR_MISALIGNED = 4,
    MSDA_ERR_WORKSPACE = 5,
    MSDA_ERR_HIP = 6
} msda_status;

typedef enum { MSDA_FP32 = 0, MSDA_BF16 = 1, MSDA_FP16 = 2 } msda_dtype;

/* Sizes of one call, in the pages' notation. */
typedef struct {
    int64_t batch;       /* B */
    int64_t num_keys;    /* S: rows of the flattened pyramid */
    int64_t num_heads;   /* M */
    int64_t head_dim;    /* D: channels per head */
    int64_t num_levels;  /* L */
    int64_t num_queries; /* Q */
    int64_t num_points;  /* K: sampling points per level */
} msda_dims;

/*
 * Forward: out = MSDA(value, spatial_shapes, level_start_index,
 * sampling_locations, attention_weights).  Accumulates in fp32 and rounds
 * once to `dtype` (round to nearest even for BF16 and FP16; FP16 overflows
 * to +-Inf past 65504).  Deterministic: the
 * same inputs give bit-identical outputs.  Q = 0 or B = 0 enqueues nothing.
 * Each block gathers the corner rows of a run of head-queries straight from
 * global memory (through the L1/L2 caches); no workspace.
 */
msda_status msda_forward(const void *value, const int64_t *spatial_shapes,
                         const int64_t *level_start_index, const void *sampling_locations,
                         const void *attention_weights, void *out, const msda_dims *dims,
                         msda_dtype dtype, void *stream);

/*
 * Forward of the "softmax" method (DeformOps page, section "Multi-scale
 * deformable attention"): as msda_forward with
 *   A[b,q,m,l,k] = exp(z[b,q,m,l,k] - max) / sum_{l',k'} exp(z[b,q,m,l',k'] - max)
 * where z = attention_logits ([B, Q, M, L, K], dtype `dtype`) and max is the
 * largest of the L*K logits of (b, q, m).  The normalisation is fused: each
 * block stages its head-queries' logits in LDS and forms A there (fp32), so
 * the call reads the logits once and writes nothing but `out`.  A NaN logit,
 * or a +Inf one, makes every weight of its head-query NaN (as exp(z - max)
 * does in exact arithmetic); all logits -Inf likewise.  Deterministic; no
 * workspace.  Errors as for msda_forward.
 */
msda_status msda_forward_softmax(const void *value, const int64_t *spatial_shapes,
                                 const int64_t *level_start_index, const void *sampling_locations,
                                 const void *attention_logits, void *out, const msda_dims *dims,
                                 msda_dtype dtype, void *stream);

/*
 * Bytes of device workspace msda_forward_binned needs for these sizes and
 * dtype (about 8 bytes per head-query plus per-block histograms), planned
 * from spatial_shapes_host ([L,2] int64 on the host, the same values as
 * spatial_shapes).  Returns SIZE_MAX when msda_forward_binned would reject
 * the call, including sizes the binned gather does not support: head rows
 * other than 64, 128 or 256 bytes, K > 8, too few queries per region of the
 * finest level, or windows that do not fit in LDS (msda_last_error() then
 * says why).
 */
size_t msda_forward_binned_workspace_bytes(const msda_dims *dims, msda_dtype dtype,
                                           const int64_t *spatial_shapes_host);

/*
 * The forward of msda_forward computed on a second schedule (equal results
 * up to the order of the fp32 additions; deterministic).  Head-queries are
 * counting-sorted by the region (bin) of the finest level their points fall
 * in; one block per bin stages, level by level, the value rows its samples
 * can reach in LDS and gathers from there; a point whose cell leaves that
 * window is gathered from global memory.  It pays off only when gathering
 * from LDS saves more than the sort and the staging cost, which this
 * library's measurements on MI355X have not shown for the encoder workloads
 * (msda_forward is faster there); it is kept for study and comparison.
 * workspace must hold at least msda_forward_binned_workspace_bytes() bytes
 * (16-byte aligned; contents on entry do not matter and are clobbered),
 * else MSDA_ERR_WORKSPACE.
 */
msda_status msda_forward_binned(const void *value, const int64_t *spatial_shapes,
                                const int64_t *level_start_index, const void *sampling_locations,
                                const void *attention_weights, void *out, const msda_dims *dims,
                                msda_dtype dtype, const int64_t *spatial_shapes_host,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * msda_forward_binned without its sort: the tile pass walks the query order
 * (head-queries sorted by region, cut into chunks) that an earlier
 * msda_forward_binned call left in `workspace`, for the inputs given now.  The
 * result is the same operator, exact for any inputs, because every point whose
 * cell leaves its region's LDS window is gathered from global memory; only
 * the speed depends on how well the old order fits the new locations.  That
 * suits calls whose reference points repeat and whose offsets move little,
 * such as an encoder layer across training steps.
 * Precondition (not checked: the order lives in device memory): the workspace
 * holds the order of an msda_forward_binned call with the same dims, dtype and
 * spatial_shapes_host, and nothing has written to it since (msda_backward does
 * not share it).  If that is violated the output is wrong, but every index
 * read from the workspace is clamped to the plan's ranges, so no access leaves
 * its buffer.  The call must fit one launch (one batch image of value below
 * 2^30 bytes for all B together), else MSDA_ERR_UNSUPPORTED.  Other arguments
 * and errors as for msda_forward_binned.
 */
msda_status msda_forward_binned_reuse(const void *value, const int64_t *spatial_shapes,
                                      const int64_t *level_start_index,
                                      const void *sampling_locations,
                                      const void *attention_weights, void *out,
                                      const msda_dims *dims, msda_dtype dtype,
                                      const int64_t *spatial_shapes_host, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* How msda_backward forms grad_value. */
typedef enum {
    /* Samples are counting-sorted by destination tile (batch, head, level,
     * 8x8 pixels); one block per tile accumulates its grad_value rows in LDS
     * and stores each row once.  No floating-point global atomics; needs a
     * workspace and a host copy of spatial_shapes.  fp32 accumulation. */
    MSDA_SCATTER_BINNED = 0,
    /* Each sample adds A * w_c * grad_out into its four corner rows with
     * device-scope atomics (fp32, or packed bf16 / fp16 for 16-bit data). */
    MSDA_SCATTER_ATOMIC = 1
} msda_scatter;

/*
 * Bytes of device workspace msda_backward needs for these sizes, dtype,
 * accumulator and scatter (the pages' own backward needs none: the DeformOps
 * page, introduction, "Zero-buffer kernels"; the binned scatter trades this
 * buffer for having no floating-point atomics):
 *   BINNED:            bin tables, sorted sample ids and tile-rim partials
 *                      (planned from spatial_shapes_host, [L,2] on the host);
 *   ATOMIC, BF16 or
 *   FP16 data, FP32
 *   accumulator:       B*S*M*D*4 (the fp32 accumulator);
 *   otherwise          0.
 * Returns SIZE_MAX when the arguments would be rejected by msda_backward
 * (msda_last_error() then says why).
 */
size_t msda_backward_workspace_bytes(const msda_dims *dims, msda_dtype dtype,
                                     msda_dtype accum_dtype, msda_scatter scatter,
                                     const int64_t *spatial_shapes_host);

/*
 * Backward of <out, grad_out>.  The gradients are those of the operator of
 * "1. Deformable attention, from scratch" (sections "The equation, term by
 * term" and "Bilinear interpolation: reading between the pixels"); the pages
 * do not print them, they follow by differentiating its sum.  grad_value is
 * the scattered accumulation "Efficient Multi-Scale Deformable Attention on
 * GPUs" describes in section "The backward pass is an atomics problem"; the
 * fp32 accumulator switch is the one of the DeformOps page, section "Backend
 * selection".  Writes (overwrites) all three gradients:
 *   grad_value[b, row, m, :] = sum over the samples whose bilinear corner is
 *                              `row` of A * corner_weight * grad_out[b,q,m,:]
 *                              (zero for rows no sample touches);
 *   grad_loc                 = d<out, grad_out> / d sampling_locations;
 *   grad_attn                = d<out, grad_out> / d attention_weights.
 * On a cell edge (an integer pixel coordinate) grad_loc is the derivative
 * from the right, the side floor() assigns the point to.  A sample with no
 * corner inside its level gets zero grad_loc and grad_attn.
 * The order in which contributions reach a grad_value row is not fixed (LDS
 * or global atomics), so its last bits may differ between runs; grad_loc and
 * grad_attn do not depend on that order.
 * scatter / accum_dtype:
 *   BINNED: accum_dtype must be FP32; spatial_shapes_host ([L,2] int64 on
 *           the host, the same values as spatial_shapes) plans the tiles.
 *           Limits (else MSDA_ERR_UNSUPPORTED): at most 12288 8x8 tiles over
 *           all levels, B*M <= 65535, B*Q*M*L*K < 2^32 - 1.
 *   ATOMIC: FP32 data -> accum FP32 (fp32 atomics into grad_value);
 *           BF16 / FP16 data -> accum FP32 (atomics into an fp32 workspace,
 *           then one rounding to the data type) or accum = the data type
 *           (packed-bf16 / packed-fp16 atomics straight into grad_value,
 *           every partial sum rounded to that type).
 *           spatial_shapes_host may be NULL.
 * workspace must hold at least msda_backward_workspace_bytes() bytes
 * (16-byte aligned; NULL when that is 0).  Its contents on entry do not
 * matter and are clobbered.
 * Device-side checks (BINNED only; the host cannot see device data without a
 * sync): the kernels compare spatial_shapes and level_start_index with the
 * plan made from spatial_shapes_host, and the plan pass bounds its waits on
 * earlier blocks.  When a check fails, all three gradients are written as NaN
 * and msda_backward_flags() reports which check failed.
 */
msda_status msda_backward(const void *value, const int64_t *spatial_shapes,
                          const int64_t *level_start_index, const void *sampling_locations,
                          const void *attention_weights, const void *grad_out, void *grad_value,
                          void *grad_loc, void *grad_attn, const msda_dims *dims,
                          msda_dtype dtype, msda_dtype accum_dtype, msda_scatter scatter,
                          const int64_t *spatial_shapes_host, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * msda_backward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and arguments without the workspace, which comes from a
 * static device array of the library instead.  That array holds
 * msda_noalloc_scratch_bytes() bytes (256 MiB) on every GPU the entry point
 * has run on, from its first call there until the process ends; calls whose
 * workspace would need more return MSDA_ERR_WORKSPACE before anything is
 * enqueued.  Every call on a GPU uses that GPU's one array, so calls whose work
 * may overlap on one GPU (other streams, other threads) race and give wrong
 * gradients: serialise them.  Each call clears what it needs cleared itself.
 * No hipMalloc / hipFree.  Errors as for msda_backward, plus MSDA_ERR_HIP when
 * the array's address cannot be looked up.
 */
msda_status msda_backward_noalloc(const void *value, const int64_t *spatial_shapes,
                                  const int64_t *level_start_index,
                                  const void *sampling_locations, const void *attention_weights,
                                  const void *grad_out, void *grad_value, void *grad_loc,
                                  void *grad_attn, const msda_dims *dims, msda_dtype dtype,
                                  msda_dtype accum_dtype, msda_scatter scatter,
                                  const int64_t *spatial_shapes_host, void *stream);

/* Bytes of the static array msda_backward_noalloc takes its workspace from. */
size_t msda_noalloc_scratch_bytes(void);

/*
 * Bytes of device workspace msda_backward_softmax needs: what
 * msda_backward_workspace_bytes() reports for the same arguments, preceded by
 * a weights image (B*Q*M*L*K elements of `dtype`, rounded up to 256 bytes)
 * unless the scatter is BINNED and L*K is a power of two (at most 64); 0 when
 * B*Q = 0.  SIZE_MAX when the call would be rejected.
 */
size_t msda_backward_softmax_workspace_bytes(const msda_dims *dims, msda_dtype dtype,
                                             msda_dtype accum_dtype, msda_scatter scatter,
                                             const int64_t *spatial_shapes_host);

/*
 * Backward of the "softmax" method (DeformOps page, section "Multi-scale
 * deformable attention"): the gradients of <out, grad_out> for the forward of
 * msda_forward_softmax, with respect to value, sampling_locations and the
 * logits.  With gA = d<out, grad_out>/dA (msda_backward's grad_attn for
 * A = softmax(z)):
 *   grad_logits[b,q,m,j] = A_j * (gA_j - sum_i A_i gA_i)   over the L*K samples.
 * Runs on `stream` as msda_backward with weights A (grad_attn written into
 * grad_logits), then an in-place pass that turns gA into grad_logits with A
 * recomputed from z in fp32.  With the BINNED scatter and L*K a power of two
 * (at most 64) the scatter pass forms A itself (fp32, from the lanes that hold
 * one head-query's logits); otherwise a first pass writes A into the head of
 * the workspace (rounded once to the data type for BF16 and FP16).  gA is
 * rounded once to the data type before the last pass.  scatter, accum_dtype,
 * spatial_shapes_host, limits and errors as for msda_backward; workspace must
 * hold msda_backward_softmax_workspace_bytes() bytes (16-byte aligned).
 */
msda_status msda_backward_softmax(const void *value, const int64_t *spatial_shapes,
                                  const int64_t *level_start_index,
                                  const void *sampling_locations, const void *attention_logits,
                                  const void *grad_out, void *grad_value, void *grad_loc,
                                  void *grad_logits, const msda_dims *dims, msda_dtype dtype,
                                  msda_dtype accum_dtype, msda_scatter scatter,
                                  const int64_t *spatial_shapes_host, void *workspace,
                                  size_t workspace_bytes, void *stream);


/* Flags of msda_backward_flags(). */
#define MSDA_BWD_SHAPES_MISMATCH 1u /* device spatial_shapes or level_start_index differ from
                                       spatial_shapes_host (or its prefix sums) */
#define MSDA_BWD_PLAN_EXPIRED 2u    /* a plan block stopped waiting for an earlier one */

/*
 * The device-side check flags a BINNED msda_backward (softmax_method = 0) or
 * msda_backward_softmax (softmax_method = 1) call left in its workspace: 0 when
 * its gradients are valid, else MSDA_BWD_* bits (its gradients are then NaN).
 * Arguments as for the call being checked (the same dims, dtypes, scatter,
 * spatial_shapes_host and workspace).  Enqueues a 4-byte copy on `stream`,
 * after the call's work, and waits for it.  With the ATOMIC scatter, or a call
 * without samples, *flags is 0 and nothing is enqueued.  Errors as for the
 * workspace-size functions, or MSDA_ERR_HIP.
 */
msda_status msda_backward_flags(const msda_dims *dims, msda_dtype dtype, msda_dtype accum_dtype,
                                msda_scatter scatter, int softmax_method,
                                const int64_t *spatial_shapes_host, const void *workspace,
                                size_t workspace_bytes, void *stream, uint32_t *flags);

/*
 * Static description of a status code.  As the DeformOps page (section
 * "Backend selection") lists every rejected candidate with its reason, every
 * rejected call here returns a status and leaves its reason for
 * msda_last_error().
 */
const char *msda_status_string(msda_status status);

/* Thread-local detail of this thread's last non-OK return ("" if none): which
 * argument or limit rejected the call (DeformOps page, "Backend selection"). */
const char *msda_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_H */
