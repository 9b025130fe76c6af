// C ABI of the MSDA library: argument validation, batch chunking and dispatch.
// Every check runs on the host before anything is enqueued; a rejected call
// leaves the stream untouched and records the reason for msda_last_error().
#include "msda.h"
#include "msda_bench.h"
#include "msda_launch.h"

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstddef>

namespace {

thread_local char g_last_error[512] = "";

msda_status fail(msda_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

constexpr int64_t kMaxElems = int64_t(1) << 62;
// Byte size of one launch's value image; keeps every corner offset (and its
// fp32-workspace double) inside 31 bits, below the "outside" sentinel.
constexpr int64_t kMaxLaunchValueBytes = (int64_t(1) << 30) - 1;

bool mul_ok(int64_t a, int64_t b, int64_t *r) {
  if (a != 0 && b > kMaxElems / a) return false;
  *r = a * b;
  return true;
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

msda::Dtype kernel_dtype(msda_dtype d) {
  return d == MSDA_FP32 ? msda::Dtype::F32 : d == MSDA_BF16 ? msda::Dtype::BF16 : msda::Dtype::F16;
}

struct Checked {
  msda_dtype dtype;      // data type of the floating tensors
  int64_t B, S, M, D, L, Q, K;
  int64_t elt;           // bytes per element of the data dtype
  int64_t value_elems;   // B*S*M*D
  int64_t batch_value_elems;
  int64_t hq_elems;      // B*Q*M
  int64_t sample_elems;  // B*Q*M*L*K
};

msda_status check_dims(const msda_dims *d, msda_dtype dtype, Checked *c) {
  if (!d) return fail(MSDA_ERR_NULL_POINTER, "dims is NULL");
  if (dtype != MSDA_FP32 && dtype != MSDA_BF16 && dtype != MSDA_FP16)
    return fail(MSDA_ERR_UNSUPPORTED, "dtype %d is not FP32 (0), BF16 (1) or FP16 (2)",
                (int)dtype);
  c->dtype = dtype;
  c->B = d->batch;
  c->S = d->num_keys;
  c->M = d->num_heads;
  c->D = d->head_dim;
  c->L = d->num_levels;
  c->Q = d->num_queries;
  c->K = d->num_points;
  if (c->B < 0 || c->Q < 0)
    return fail(MSDA_ERR_INVALID_DIMS, "batch (%lld) and num_queries (%lld) must be >= 0",
                (long long)c->B, (long long)c->Q);
  if (c->S < 1 || c->M < 1)
    return fail(MSDA_ERR_INVALID_DIMS, "num_keys (%lld) and num_heads (%lld) must be >= 1",
                (long long)c->S, (long long)c->M);
  if (c->L < 1 || c->K < 1)
    return fail(MSDA_ERR_INVALID_DIMS, "num_levels (%lld) and num_points (%lld) must be >= 1",
                (long long)c->L, (long long)c->K);
  if (c->D != 8 && c->D != 16 && c->D != 32 && c->D != 64)
    return fail(MSDA_ERR_UNSUPPORTED, "head_dim %lld not in {8, 16, 32, 64}", (long long)c->D);
  if (c->L > 16 || c->K > 32 || c->L * c->K > 64)
    return fail(MSDA_ERR_UNSUPPORTED,
                "num_levels %lld / num_points %lld outside L <= 16, K <= 32, L*K <= 64",
                (long long)c->L, (long long)c->K);
  c->elt = dtype == MSDA_FP32 ? 4 : 2;
  int64_t sm, smd, bq, bqm, lk;
  if (!mul_ok(c->S, c->M, &sm) || !mul_ok(sm, c->D, &smd) ||
      !mul_ok(smd, c->B, &c->value_elems) || !mul_ok(c->B, c->Q, &bq) ||
      !mul_ok(bq, c->M, &bqm) || !mul_ok(c->L, c->K, &lk) ||
      !mul_ok(bqm, lk * 2, &c->sample_elems))
    return fail(MSDA_ERR_INVALID_DIMS, "element counts overflow 2^62");
  c->sample_elems /= 2;
  c->batch_value_elems = smd;
  c->hq_elems = bqm;
  if (smd * c->elt > kMaxLaunchValueBytes)
    return fail(MSDA_ERR_UNSUPPORTED,
                "one batch image of value is %lld bytes; at most 2^30 - 1 are supported",
                (long long)(smd * c->elt));
  return MSDA_OK;
}

msda_status check_ptr(const void *p, const char *name, bool needed, uintptr_t align) {
  if (!needed) return MSDA_OK;
  if (!p) return fail(MSDA_ERR_NULL_POINTER, "%s is NULL", name);
  if (!aligned(p, align))
    return fail(MSDA_ERR_MISALIGNED, "%s is not %u-byte aligned", name, (unsigned)align);
  return MSDA_OK;
}

#define MSDA_TRY(expr)                     \
  do {                                     \
    msda_status _s = (expr);               \
    if (_s != MSDA_OK) return _s;          \
  } while (0)

// Batches per launch so that one launch's value image stays below 2^30 bytes.
int64_t batches_per_launch(const Checked &c) {
  const int64_t per = c.batch_value_elems * c.elt;
  int64_t nb = kMaxLaunchValueBytes / per;
  return nb < 1 ? 1 : nb;
}

msda::LaunchArgs chunk_args(const Checked &c, int64_t b0, int64_t nb, int64_t acc_elt,
                            const void *value, const int64_t *shapes, const int64_t *starts,
                            const void *loc, const void *attn) {
  msda::LaunchArgs a{};
  const int64_t per_hq = c.Q * c.M;
  a.value = static_cast<const char *>(value) + b0 * c.batch_value_elems * c.elt;
  a.shapes = shapes;
  a.starts = starts;
  a.loc = static_cast<const char *>(loc) + b0 * per_hq * c.L * c.K * 2 * c.elt;
  a.attn = static_cast<const char *>(attn) + b0 * per_hq * c.L * c.K * c.elt;
  a.nb = nb;
  a.S = c.S;
  a.M = c.M;
  a.D = c.D;
  a.L = c.L;
  a.Q = c.Q;
  a.K = c.K;
  a.value_bytes = (uint32_t)(nb * c.batch_value_elems * c.elt);
  a.acc_bytes = (uint32_t)(nb * c.batch_value_elems * acc_elt);
  return a;
}

msda_status hip_fail(hipError_t e, const char *what) {
  return fail(MSDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Plan of the query-binned forward for the largest batch chunk of a call.
msda_status forward_binned_plan(const Checked &c, const int64_t *shapes_host,
                                msda::FwdPlan *plan, size_t *ws) {
  *ws = 0;
  if (c.hq_elems == 0) return MSDA_OK;
  if (!shapes_host) return fail(MSDA_ERR_NULL_POINTER, "the binned forward needs spatial_shapes_host");
  const int64_t step = batches_per_launch(c);
  const int64_t nb = c.B < step ? c.B : step;
  if (!msda::make_fwd_plan(*plan, nb, c.Q, c.S, (int)c.M, (int)c.D, (int)c.L, (int)c.K,
                           (int)c.elt, shapes_host))
    return fail(MSDA_ERR_UNSUPPORTED,
                "the binned forward does not suit these sizes (row bytes, K, queries per "
                "region of the finest level or LDS windows)");
  *ws = msda::fwd_workspace_bytes(*plan);
  return MSDA_OK;
}

msda_status forward_checks(const void *value, const int64_t *spatial_shapes,
                           const int64_t *level_start_index, const void *sampling_locations,
                           const void *attention_weights, void *out, const msda_dims *dims,
                           msda_dtype dtype, Checked *c,
                           const char *weights_name = "attention_weights") {
  MSDA_TRY(check_dims(dims, dtype, c));
  const bool work = c->hq_elems > 0;
  MSDA_TRY(check_ptr(value, "value", true, 16));
  MSDA_TRY(check_ptr(spatial_shapes, "spatial_shapes", true, 8));
  MSDA_TRY(check_ptr(level_start_index, "level_start_index", true, 8));
  MSDA_TRY(check_ptr(sampling_locations, "sampling_locations", work, 16));
  MSDA_TRY(check_ptr(attention_weights, weights_name, work, 16));
  MSDA_TRY(check_ptr(out, "out", work, 16));
  return MSDA_OK;
}

// Direct-gather forward over batch chunks; `weights` holds attention weights,
// or raw logits when `softmax` is set.
msda_status forward_direct(const void *value, const int64_t *spatial_shapes,
                           const int64_t *level_start_index, const void *sampling_locations,
                           const void *weights, void *out, const msda_dims *dims,
                           msda_dtype dtype, bool softmax, void *stream) {
  g_last_error[0] = '\0';
  Checked c;
  MSDA_TRY(forward_checks(value, spatial_shapes, level_start_index, sampling_locations, weights,
                          out, dims, dtype, &c,
                          softmax ? "attention_logits" : "attention_weights"));
  if (c.hq_elems == 0) return MSDA_OK;
  const auto dt = kernel_dtype(dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t step = batches_per_launch(c);
  for (int64_t b0 = 0; b0 < c.B; b0 += step) {
    const int64_t nb = c.B - b0 < step ? c.B - b0 : step;
    msda::LaunchArgs a = chunk_args(c, b0, nb, c.elt, value, spatial_shapes, level_start_index,
                                    sampling_locations, weights);
    a.out = static_cast<char *>(out) + b0 * c.Q * c.M * c.D * c.elt;
    hipError_t e = msda::launch_forward(a, dt, s, softmax);
    if (e != hipSuccess) return hip_fail(e, softmax ? "softmax forward launch" : "forward launch");
  }
  return MSDA_OK;
}

}  // namespace

namespace msda {
void set_last_error(const char *msg) { snprintf(g_last_error, sizeof(g_last_error), "%s", msg); }
}  // namespace msda

extern "C" {

msda_status msda_forward(const void *value, const int64_t *spatial_shapes,
                         const int64_t *level_start_index, const void *sampling_locations,
                         const void *attention_weights, void *out, const msda_dims *dims,
                         msda_dtype dtype, void *stream) {
  return forward_direct(value, spatial_shapes, level_start_index, sampling_locations,
                        attention_weights, out, dims, dtype, false, stream);
}

msda_status msda_forward_softmax(const void *value, const int64_t *spatial_shapes,
                                 const int64_t *level_start_index, const void *sampling_locations,
                                 const void *attention_logits, void *out, const msda_dims *dims,
                                 msda_dtype dtype, void *stream) {
  return forward_direct(value, spatial_shapes, level_start_index, sampling_locations,
                        attention_logits, out, dims, dtype, true, stream);
}

size_t msda_forward_binned_workspace_bytes(const msda_dims *dims, msda_dtype dtype,
                                           const int64_t *spatial_shapes_host) {
  g_last_error[0] = '\0';
  Checked c;
  if (check_dims(dims, dtype, &c) != MSDA_OK) return SIZE_MAX;
  msda::FwdPlan plan;
  size_t ws;
  if (forward_binned_plan(c, spatial_shapes_host, &plan, &ws) != MSDA_OK) return SIZE_MAX;
  return ws;
}

}  // extern "C"

namespace {

// The query-binned forward, with or without the sort (reuse_order).
msda_status forward_binned_run(const void *value, const int64_t *spatial_shapes,
                               const int64_t *level_start_index, const void *sampling_locations,
                               const void *attention_weights, void *out, const msda_dims *dims,
                               msda_dtype dtype, const int64_t *spatial_shapes_host,
                               void *workspace, size_t workspace_bytes, bool reuse_order,
                               void *stream) {
  g_last_error[0] = '\0';
  Checked c;
  MSDA_TRY(forward_checks(value, spatial_shapes, level_start_index, sampling_locations,
                          attention_weights, out, dims, dtype, &c));
  msda::FwdPlan plan;
  size_t ws_need;
  MSDA_TRY(forward_binned_plan(c, spatial_shapes_host, &plan, &ws_need));
  if (c.hq_elems == 0) return MSDA_OK;
  if (!workspace || workspace_bytes < ws_need)
    return fail(MSDA_ERR_WORKSPACE, "this forward needs %zu bytes of workspace, got %zu%s",
                ws_need, workspace_bytes, workspace ? "" : " (NULL)");
  if (!aligned(workspace, 16)) return fail(MSDA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  const int64_t step = batches_per_launch(c);
  if (reuse_order && c.B > step)
    return fail(MSDA_ERR_UNSUPPORTED,
                "reusing the query order needs the whole call in one launch (%lld batches, at "
                "most %lld per launch here)", (long long)c.B, (long long)step);
  const auto dt = kernel_dtype(dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t b0 = 0; b0 < c.B; b0 += step) {
    const int64_t nb = c.B - b0 < step ? c.B - b0 : step;
    msda::FwdArgs fa{};
    fa.a = chunk_args(c, b0, nb, c.elt, value, spatial_shapes, level_start_index,
                      sampling_locations, attention_weights);
    fa.a.out = static_cast<char *>(out) + b0 * c.Q * c.M * c.D * c.elt;
    // the plan of a smaller last chunk needs no more workspace than the first
    if (!msda::make_fwd_plan(fa.p, nb, c.Q, c.S, (int)c.M, (int)c.D, (int)c.L, (int)c.K,
                             (int)c.elt, spatial_shapes_host))
      return fail(MSDA_ERR_UNSUPPORTED, "binned forward: no plan for %lld batches", (long long)nb);
    fa.w = msda::carve_fwd_scratch(fa.p, workspace);
    hipError_t e = msda::launch_forward_binned(fa, dt, reuse_order, s);
    if (e != hipSuccess) return hip_fail(e, "binned forward launch");
  }
  return MSDA_OK;
}

}  // namespace

extern "C" {

msda_status msda_forward_binned(const void *value, const int64_t *spatial_shapes,
                                const int64_t *level_start_index, const void *sampling_locations,
                                const void *attention_weights, void *out, const msda_dims *dims,
                                msda_dtype dtype, const int64_t *spatial_shapes_host,
                                void *workspace, size_t workspace_bytes, void *stream) {
  return forward_binned_run(value, spatial_shapes, level_start_index, sampling_locations,
                            attention_weights, out, dims, dtype, spatial_shapes_host, workspace,
                            workspace_bytes, false, stream);
}

msda_status msda_forward_binned_reuse(const void *value, const int64_t *spatial_shapes,
                                      const int64_t *level_start_index,
                                      const void *sampling_locations,
                                      const void *attention_weights, void *out,
                                      const msda_dims *dims, msda_dtype dtype,
                                      const int64_t *spatial_shapes_host, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  return forward_binned_run(value, spatial_shapes, level_start_index, sampling_locations,
                            attention_weights, out, dims, dtype, spatial_shapes_host, workspace,
                            workspace_bytes, true, stream);
}

}  // extern "C"

namespace {

struct BackwardSetup {
  Checked c;
  bool work = false;     // at least one sample
  bool binned = false;
  bool use_ws = false;   // atomic path with an fp32 workspace
  msda::BinPlan plan{};
  size_t ws_need = 0;
};

msda_status backward_setup(const msda_dims *dims, msda_dtype dtype, msda_dtype accum_dtype,
                           msda_scatter scatter, const int64_t *shapes_host, BackwardSetup *su) {
  MSDA_TRY(check_dims(dims, dtype, &su->c));
  const Checked &c = su->c;
  if (accum_dtype != MSDA_FP32 && accum_dtype != MSDA_BF16 && accum_dtype != MSDA_FP16)
    return fail(MSDA_ERR_UNSUPPORTED, "accum_dtype %d is not FP32 (0), BF16 (1) or FP16 (2)",
                (int)accum_dtype);
  if (scatter != MSDA_SCATTER_BINNED && scatter != MSDA_SCATTER_ATOMIC)
    return fail(MSDA_ERR_UNSUPPORTED, "scatter %d is not BINNED (0) or ATOMIC (1)", (int)scatter);
  su->work = c.hq_elems > 0;
  if (scatter == MSDA_SCATTER_BINNED) {
    su->binned = true;
    if (accum_dtype != MSDA_FP32)
      return fail(MSDA_ERR_UNSUPPORTED, "the binned scatter accumulates in fp32 only");
    if (su->work) {
      if (!shapes_host)
        return fail(MSDA_ERR_NULL_POINTER, "the binned scatter needs spatial_shapes_host");
      const char *why = "";
      if (!msda::make_bin_plan(su->plan, c.B, c.Q, c.S, (int)c.M, (int)c.D, (int)c.L, (int)c.K,
                               shapes_host, &why))
        return fail(MSDA_ERR_UNSUPPORTED, "binned scatter: %s", why);
      su->ws_need = msda::binned_workspace_bytes(su->plan);
    }
  } else {
    if (accum_dtype != MSDA_FP32 && accum_dtype != dtype)
      return fail(MSDA_ERR_UNSUPPORTED,
                  "the atomic scatter accumulates in FP32 or in the data type (dtype %d, "
                  "accum_dtype %d)", (int)dtype, (int)accum_dtype);
    su->use_ws = dtype != MSDA_FP32 && accum_dtype == MSDA_FP32 && su->work;
    su->ws_need = su->use_ws ? (size_t)c.value_elems * 4 : 0;
  }
  return MSDA_OK;
}

// Enqueue the backward of a validated call (backward_setup + pointer checks
// done); `workspace` is the part of the caller's workspace the scatter uses.
// softmax_logits (binned scatter only): attention_weights holds raw logits and
// the scatter pass forms the softmax weights.
msda_status backward_run(const BackwardSetup &su, msda_dtype accum_dtype, const void *value,
                         const int64_t *spatial_shapes, const int64_t *level_start_index,
                         const void *sampling_locations, const void *attention_weights,
                         const void *grad_out, void *grad_value, void *grad_loc, void *grad_attn,
                         void *workspace, hipStream_t s, bool softmax_logits = false) {
  const Checked &c = su.c;
  if (c.value_elems == 0) return MSDA_OK;
  hipError_t e;
  if (!su.work) {
    e = msda::launch_zero(grad_value, (size_t)(c.value_elems * c.elt), s);
    return e == hipSuccess ? MSDA_OK : hip_fail(e, "grad_value zero-fill launch");
  }
  const auto dt = kernel_dtype(c.dtype);
  if (su.binned) {
    msda::BinArgs a{};
    a.value = value;
    a.shapes = spatial_shapes;
    a.starts = level_start_index;
    a.loc = sampling_locations;
    a.attn = attention_weights;
    a.grad_out = grad_out;
    a.grad_value = grad_value;
    a.grad_loc = grad_loc;
    a.grad_attn = grad_attn;
    a.p = su.plan;
    a.w = msda::carve_bin_scratch(su.plan, workspace);
    a.softmax = softmax_logits;
    e = msda::launch_backward_binned(a, dt, s);
    return e == hipSuccess ? MSDA_OK : hip_fail(e, "binned backward launch");
  }
  const bool use_ws = su.use_ws;
  if (!use_ws) {
    e = msda::launch_zero(grad_value, (size_t)(c.value_elems * c.elt), s);
    if (e != hipSuccess) return hip_fail(e, "grad_value zero-fill launch");
  } else {
    e = msda::launch_zero(workspace, (size_t)c.value_elems * 4, s);
    if (e != hipSuccess) return hip_fail(e, "workspace zero-fill launch");
  }
  const auto acc = accum_dtype == MSDA_FP32 ? msda::Accum::F32 : msda::Accum::PACKED;
  const int64_t acc_elt = accum_dtype == MSDA_FP32 ? 4 : 2;
  char *acc_base = static_cast<char *>(use_ws ? workspace : grad_value);
  const int64_t step = batches_per_launch(c);
  for (int64_t b0 = 0; b0 < c.B; b0 += step) {
    const int64_t nb = c.B - b0 < step ? c.B - b0 : step;
    msda::LaunchArgs a = chunk_args(c, b0, nb, acc_elt, value, spatial_shapes, level_start_index,
                                    sampling_locations, attention_weights);
    const int64_t samples0 = b0 * c.Q * c.M * c.L * c.K;
    a.grad_out = static_cast<const char *>(grad_out) + b0 * c.Q * c.M * c.D * c.elt;
    a.grad_acc = acc_base + b0 * c.batch_value_elems * acc_elt;
    a.grad_loc = static_cast<char *>(grad_loc) + samples0 * 2 * c.elt;
    a.grad_attn = static_cast<char *>(grad_attn) + samples0 * c.elt;
    e = msda::launch_backward(a, dt, acc, s);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
  }
  if (use_ws) {
    e = msda::launch_cast_f32_to_half(static_cast<const float *>(workspace), grad_value,
                                      (size_t)c.value_elems, dt, s);
    if (e != hipSuccess) return hip_fail(e, "workspace cast launch");
  }
  return MSDA_OK;
}

msda_status backward_pointer_checks(const Checked &c, const void *value,
                                    const int64_t *spatial_shapes,
                                    const int64_t *level_start_index,
                                    const void *sampling_locations, const void *weights,
                                    const char *weights_name, const void *grad_out,
                                    void *grad_value, void *grad_loc, void *grad_weights,
                                    const char *grad_weights_name) {
  const bool work = c.hq_elems > 0;
  MSDA_TRY(check_ptr(value, "value", true, 16));
  MSDA_TRY(check_ptr(spatial_shapes, "spatial_shapes", true, 8));
  MSDA_TRY(check_ptr(level_start_index, "level_start_index", true, 8));
  MSDA_TRY(check_ptr(sampling_locations, "sampling_locations", work, 16));
  MSDA_TRY(check_ptr(weights, weights_name, work, 16));
  MSDA_TRY(check_ptr(grad_out, "grad_out", work, 16));
  MSDA_TRY(check_ptr(grad_value, "grad_value", c.value_elems > 0, 16));
  MSDA_TRY(check_ptr(grad_loc, "grad_loc", work, 16));
  MSDA_TRY(check_ptr(grad_weights, grad_weights_name, work, 16));
  return MSDA_OK;
}

msda_status workspace_check(size_t need, void *workspace, size_t workspace_bytes,
                            const char *what) {
  if (need == 0) return MSDA_OK;
  if (!workspace || workspace_bytes < need)
    return fail(MSDA_ERR_WORKSPACE, "this %s needs %zu bytes of workspace, got %zu%s", what, need,
                workspace_bytes, workspace ? "" : " (NULL)");
  if (!aligned(workspace, 16)) return fail(MSDA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  return MSDA_OK;
}

// The softmax backward forms the weights inside the binned scatter pass when a
// head-query's L*K samples fill an aligned lane group (L*K a power of two, at
// most 64); otherwise a row pass writes them to the head of the workspace.
bool softmax_in_scatter(const BackwardSetup &su) {
  const int64_t lk = su.c.L * su.c.K;
  return su.binned && lk <= 64 && (lk & (lk - 1)) == 0;
}

// Bytes of the softmax backward's weights image at the head of its workspace
// (256-byte multiple, so the scatter's part keeps its alignment); 0 when the
// scatter pass forms the weights.
size_t softmax_weights_bytes(const BackwardSetup &su) {
  if (!su.work || softmax_in_scatter(su)) return 0;
  return ((size_t)(su.c.sample_elems * su.c.elt) + 255) / 256 * 256;
}

}  // namespace

extern "C" {

size_t msda_backward_workspace_bytes(const msda_dims *dims, msda_dtype dtype,
                                     msda_dtype accum_dtype, msda_scatter scatter,
                                     const int64_t *spatial_shapes_host) {
  g_last_error[0] = '\0';
  BackwardSetup su;
  if (backward_setup(dims, dtype, accum_dtype, scatter, spatial_shapes_host, &su) != MSDA_OK)
    return SIZE_MAX;
  return su.ws_need;
}

msda_status msda_backward(const void *value, const int64_t *spatial_shapes,
                          const int64_t *level_start_index, const void *sampling_locations,
                          const void *attention_weights, const void *grad_out, void *grad_value,
                          void *grad_loc, void *grad_attn, const msda_dims *dims,
                          msda_dtype dtype, msda_dtype accum_dtype, msda_scatter scatter,
                          const int64_t *spatial_shapes_host, void *workspace,
                          size_t workspace_bytes, void *stream) {
  g_last_error[0] = '\0';
  BackwardSetup su;
  MSDA_TRY(backward_setup(dims, dtype, accum_dtype, scatter, spatial_shapes_host, &su));
  MSDA_TRY(backward_pointer_checks(su.c, value, spatial_shapes, level_start_index,
                                   sampling_locations, attention_weights, "attention_weights",
                                   grad_out, grad_value, grad_loc, grad_attn, "grad_attn"));
  MSDA_TRY(workspace_check(su.ws_need, workspace, workspace_bytes, "backward"));
  return backward_run(su, accum_dtype, value, spatial_shapes, level_start_index,
                      sampling_locations, attention_weights, grad_out, grad_value, grad_loc,
                      grad_attn, workspace, static_cast<hipStream_t>(stream));
}

size_t msda_backward_softmax_workspace_bytes(const msda_dims *dims, msda_dtype dtype,
                                             msda_dtype accum_dtype, msda_scatter scatter,
                                             const int64_t *spatial_shapes_host) {
  g_last_error[0] = '\0';
  BackwardSetup su;
  if (backward_setup(dims, dtype, accum_dtype, scatter, spatial_shapes_host, &su) != MSDA_OK)
    return SIZE_MAX;
  return su.work ? softmax_weights_bytes(su) + su.ws_need : 0;
}

msda_status msda_backward_softmax(const void *value, const int64_t *spatial_shapes,
                                  const int64_t *level_start_index,
                                  const void *sampling_locations, const void *attention_logits,
                                  const void *grad_out, void *grad_value, void *grad_loc,
                                  void *grad_logits, const msda_dims *dims, msda_dtype dtype,
                                  msda_dtype accum_dtype, msda_scatter scatter,
                                  const int64_t *spatial_shapes_host, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  g_last_error[0] = '\0';
  BackwardSetup su;
  MSDA_TRY(backward_setup(dims, dtype, accum_dtype, scatter, spatial_shapes_host, &su));
  const Checked &c = su.c;
  MSDA_TRY(backward_pointer_checks(c, value, spatial_shapes, level_start_index,
                                   sampling_locations, attention_logits, "attention_logits",
                                   grad_out, grad_value, grad_loc, grad_logits, "grad_logits"));
  const size_t wbytes = softmax_weights_bytes(su);
  MSDA_TRY(workspace_check(wbytes + su.ws_need, workspace, workspace_bytes, "softmax backward"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto dt = kernel_dtype(dtype);
  const int lk = (int)(c.L * c.K);
  const bool fused = su.work && softmax_in_scatter(su);
  const void *weights = fused ? attention_logits : workspace;
  if (su.work && !fused) {
    hipError_t e = msda::launch_softmax_rows(attention_logits, workspace, c.hq_elems, lk, dt, s);
    if (e != hipSuccess) return hip_fail(e, "softmax launch");
  }
  void *scatter_ws = wbytes ? static_cast<char *>(workspace) + wbytes : workspace;
  MSDA_TRY(backward_run(su, accum_dtype, value, spatial_shapes, level_start_index,
                        sampling_locations, weights, grad_out, grad_value, grad_loc, grad_logits,
                        scatter_ws, s, fused));
  if (su.work) {
    hipError_t e = msda::launch_softmax_grad_rows(attention_logits, grad_logits, c.hq_elems, lk,
                                                  dt, s);
    if (e != hipSuccess) return hip_fail(e, "softmax derivative launch");
  }
  return MSDA_OK;
}

msda_status msda_backward_flags(const msda_dims *dims, msda_dtype dtype, msda_dtype accum_dtype,
                                msda_scatter scatter, int softmax_method,
                                const int64_t *spatial_shapes_host, const void *workspace,
                                size_t workspace_bytes, void *stream, uint32_t *flags) {
  g_last_error[0] = '\0';
  if (!flags) return fail(MSDA_ERR_NULL_POINTER, "flags is NULL");
  *flags = 0;
  BackwardSetup su;
  MSDA_TRY(backward_setup(dims, dtype, accum_dtype, scatter, spatial_shapes_host, &su));
  if (!su.binned || !su.work) return MSDA_OK;  // only the binned scatter checks on the device
  const size_t head = softmax_method ? softmax_weights_bytes(su) : 0;
  MSDA_TRY(workspace_check(head + su.ws_need, const_cast<void *>(workspace), workspace_bytes,
                           "check"));
  const char *word = static_cast<const char *>(workspace) + head + msda::binned_error_offset(su.plan);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, word, sizeof(v), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the error word");
  *flags = v;
  return MSDA_OK;
}

void msda_test_set_plan_wait_limit(uint32_t polls) { msda::set_plan_spin_limit(polls); }

void msda_test_set_forward_schedule(int schedule) { msda::set_forward_schedule(schedule); }

void msda_test_set_tile_wide_addressing(int wide) { msda::set_tile_wide_addressing(wide != 0); }

msda_status msda_test_tile_phase_clocks(unsigned long long *out, int nblocks) {
  if (out == nullptr) return MSDA_ERR_NULL_POINTER;
  if (nblocks < 0 || nblocks > 2048) return MSDA_ERR_INVALID_DIMS;
  const hipError_t e = msda::tile_phase_clocks(out, nblocks);
  if (e == hipErrorNotSupported) return MSDA_ERR_UNSUPPORTED;
  return e == hipSuccess ? MSDA_OK : MSDA_ERR_HIP;
}

const char *msda_status_string(msda_status status) {
  switch (status) {
    case MSDA_OK: return "MSDA_OK";
    case MSDA_ERR_NULL_POINTER: return "MSDA_ERR_NULL_POINTER: a required pointer is NULL";
    case MSDA_ERR_INVALID_DIMS: return "MSDA_ERR_INVALID_DIMS: sizes are negative, zero or overflow";
    case MSDA_ERR_UNSUPPORTED: return "MSDA_ERR_UNSUPPORTED: dtype or size outside the supported set";
    case MSDA_ERR_MISALIGNED: return "MSDA_ERR_MISALIGNED: a pointer is not aligned as required";
    case MSDA_ERR_WORKSPACE: return "MSDA_ERR_WORKSPACE: workspace missing or too small";
    case MSDA_ERR_HIP: return "MSDA_ERR_HIP: a HIP launch failed";
  }
  return "unknown msda_status";
}

const char *msda_last_error(void) { return g_last_error; }

}  // extern "C"
