// C ABI of the dMoE layer: argument checks and the launch sequence of each
// entry point.  Every check here runs on the host before anything is
// enqueued; nothing is allocated and nothing waits on the device.
#include "../../include/dmoe.h"
#include "dmoe_internal.h"


namespace {

using dmoe::MetaPtrs;
using dmoe::Shape;

int check_dims(const dmoe_dims* d) {
  if (!d) return DMOE_ERR_ARG;
  if (d->T <= 0 || d->H <= 0 || d->F <= 0 || d->E <= 0 || d->k <= 0) return DMOE_ERR_ARG;
  if (d->dtype != DMOE_F32 && d->dtype != DMOE_BF16) return DMOE_ERR_UNSUPPORTED;
  if (d->E > DMOE_MAX_EXPERTS) return DMOE_ERR_UNSUPPORTED;
  if (d->k > d->E) return DMOE_ERR_ARG;
  const int64_t n = d->T * (int64_t)d->k;
  if (d->T >= (int64_t(1) << 31) || n >= (int64_t(1) << 31)) return DMOE_ERR_ARG;
  // P_max must stay below 2^31 rows: row indices are int32 on the device.
  const int64_t pmax = n + 127 * (int64_t)(d->E < n ? d->E : n);
  if (pmax >= (int64_t(1) << 31)) return DMOE_ERR_ARG;
  if (d->F % DMOE_BLOCK != 0 || d->H % DMOE_BLOCK != 0) return DMOE_ERR_SHAPE;
  if (d->H > (int64_t(1) << 24) || d->F > (int64_t(1) << 24)) return DMOE_ERR_UNSUPPORTED;
  return DMOE_OK;
}

// The row-block GEMMs put the 128-row block index on grid dimension y.
constexpr int64_t kMaxGridY = 65535;

int check_gemm_dims(const dmoe_dims* d) {
  const int rc = check_dims(d);
  if (rc != DMOE_OK) return rc;
  const int64_t n = d->T * (int64_t)d->k;
  const int64_t tiles = (n + 127 * (int64_t)(d->E < n ? d->E : n)) / DMOE_BLOCK;
  return tiles > kMaxGridY ? DMOE_ERR_UNSUPPORTED : DMOE_OK;
}

int64_t max_tiles_of(const dmoe_dims* d) {
  const int64_t n = d->T * (int64_t)d->k;
  return (n + 127 * (int64_t)(d->E < n ? d->E : n)) / DMOE_BLOCK;
}

Shape shape_of(const dmoe_dims* d) {
  return Shape{d->T, d->H, d->F, d->E, d->k, max_tiles_of(d), d->dtype == DMOE_BF16};
}

int check_meta(const dmoe_meta* m) {
  if (!m || !m->tokens_per_expert || !m->bins || !m->padded_bins || !m->indices ||
      !m->bin_ids || !m->row_of_entry || !m->tile_expert || !m->num_padded_rows ||
      !m->status || !m->pair_first || !m->num_pairs || !m->row_token ||
      !m->xcd_first)
    return DMOE_ERR_ARG;
  return DMOE_OK;
}

MetaPtrs meta_ptrs(const dmoe_meta* m) {
  return MetaPtrs{m->tokens_per_expert, m->bins, m->padded_bins, m->indices,
                  m->bin_ids, m->row_of_entry, m->tile_expert, m->num_padded_rows,
                  m->status, m->pair_first, m->num_pairs, m->row_token,
                  m->xcd_first};
}

// Records events[i] on the stream when timing is requested and the entry is
// not NULL.
struct Recorder {
  hipEvent_t* events;
  hipStream_t stream;
  hipError_t operator()(int i) const {
    return events && events[i] ? hipEventRecord(events[i], stream) : hipSuccess;
  }
};

#define DMOE_TRY(expr)                                  \
  do {                                                  \
    if ((expr) != hipSuccess) return DMOE_ERR_HIP;      \
  } while (0)

}  // namespace

extern "C" {

int64_t dmoe_max_tiles(const dmoe_dims* dims) {
  const int rc = check_dims(dims);
  return rc != DMOE_OK ? rc : max_tiles_of(dims);
}

int64_t dmoe_workspace_bytes(const dmoe_dims* dims) {
  const int rc = check_dims(dims);
  if (rc != DMOE_OK) return rc;
  return dmoe::meta_workspace_bytes(dims->T * (int64_t)dims->k, dims->E);
}

int dmoe_metadata_timed(const dmoe_dims* dims, const int32_t* top_experts,
                        const dmoe_meta* meta, void* ws, hipStream_t stream,
                        hipEvent_t* events) {
  int rc = check_dims(dims);
  if (rc != DMOE_OK) return rc;
  if ((rc = check_meta(meta)) != DMOE_OK) return rc;
  if (!top_experts || !ws) return DMOE_ERR_ARG;
  DMOE_TRY(dmoe::launch_metadata(dims->T * (int64_t)dims->k, dims->E, dims->k, max_tiles_of(dims),
                                 top_experts, meta_ptrs(meta), ws, stream, events));
  return DMOE_OK;
}

int dmoe_metadata(const dmoe_dims* dims, const int32_t* top_experts,
                  const dmoe_meta* meta, void* ws, hipStream_t stream) {
  return dmoe_metadata_timed(dims, top_experts, meta, ws, stream, nullptr);
}

}  // extern "C"

namespace {

// The gather fused into the operand loads: bf16 only, and x must stay below
// 2 GB (the records of the buffer resource its rows are read through).
int check_fused(const dmoe_dims* d) {
  if (d->dtype != DMOE_BF16) return DMOE_ERR_UNSUPPORTED;
  if (d->T * d->H * 2 >= (int64_t(1) << 31)) return DMOE_ERR_UNSUPPORTED;
  return DMOE_OK;
}

// The forward; with `fused`, no padded_gather: the up projection reads each
// padded row's token row of x directly and saved->x_perm is not used (event
// 0 then brackets the up projection).
int forward_impl(const dmoe_dims* dims, const void* x, const float* weights, const void* w1,
                 const void* w3, const void* w2, const dmoe_meta* meta,
                 const dmoe_saved* saved, void* y, hipStream_t stream, hipEvent_t* ev,
                 bool fused) {
  int rc = check_gemm_dims(dims);
  if (rc != DMOE_OK) return rc;
  if (fused && (rc = check_fused(dims)) != DMOE_OK) return rc;
  if ((rc = check_meta(meta)) != DMOE_OK) return rc;
  if (!x || !weights || !w1 || !w3 || !w2 || !saved || !y || (!fused && !saved->x_perm) ||
      !saved->h1 || !saved->h3 || !saved->act || !saved->y_perm)
    return DMOE_ERR_ARG;
  const Shape s = shape_of(dims);
  const MetaPtrs m = meta_ptrs(meta);
  Recorder rec{ev, stream};
  int i = 0;
  if (!fused) {
    DMOE_TRY(rec(i++));
    DMOE_TRY(dmoe::launch_padded_gather(s, x, m, saved->x_perm, stream));
  }
  DMOE_TRY(rec(i++));
  DMOE_TRY(dmoe::launch_gemm_up(s, fused ? nullptr : saved->x_perm, fused ? x : nullptr, w1, w3,
                                m, saved->h1, saved->h3, saved->act, stream));
  DMOE_TRY(rec(i++));
  DMOE_TRY(dmoe::launch_gemm_down(s, saved->act, w2, m, saved->y_perm, stream));
  DMOE_TRY(rec(i++));
  DMOE_TRY(dmoe::launch_padded_scatter(s, saved->y_perm, weights, m, y, stream));
  DMOE_TRY(rec(i++));
  return DMOE_OK;
}

}  // namespace

extern "C" {

int dmoe_forward_timed(const dmoe_dims* dims, const void* x, const float* weights,
                       const void* w1, const void* w3, const void* w2,
                       const dmoe_meta* meta, const dmoe_saved* saved, void* y,
                       hipStream_t stream, hipEvent_t* ev) {
  return forward_impl(dims, x, weights, w1, w3, w2, meta, saved, y, stream, ev, false);
}

int dmoe_forward_fused_gather_timed(const dmoe_dims* dims, const void* x, const float* weights,
                                    const void* w1, const void* w3, const void* w2,
                                    const dmoe_meta* meta, const dmoe_saved* saved, void* y,
                                    hipStream_t stream, hipEvent_t* ev) {
  return forward_impl(dims, x, weights, w1, w3, w2, meta, saved, y, stream, ev, true);
}

int dmoe_forward_fused_gather(const dmoe_dims* dims, const void* x, const float* weights,
                              const void* w1, const void* w3, const void* w2,
                              const dmoe_meta* meta, const dmoe_saved* saved, void* y,
                              hipStream_t stream) {
  return forward_impl(dims, x, weights, w1, w3, w2, meta, saved, y, stream, nullptr, true);
}

int dmoe_forward(const dmoe_dims* dims, const void* x, const float* weights,
                 const void* w1, const void* w3, const void* w2,
                 const dmoe_meta* meta, const dmoe_saved* saved, void* y,
                 hipStream_t stream) {
  return dmoe_forward_timed(dims, x, weights, w1, w3, w2, meta, saved, y, stream, nullptr);
}

}  // extern "C"

namespace {

// The backward of the layer; with `recompute`, act is rebuilt from h1 and h3
// first, and with a non-null x (after the fused-gather forward) x_perm is
// gathered from x before the up dgrad.  Each such kernel has an event of its
// own in launch order.
int backward_impl(const dmoe_dims* dims, const void* x, const void* dy, const float* weights,
                  const void* w1, const void* w3, const void* w2, const dmoe_meta* meta,
                  const dmoe_saved* saved, const dmoe_grad_scratch* scratch, void* dx,
                  void* dw1, void* dw3, void* dw2, float* d_weights, hipStream_t stream,
                  hipEvent_t* ev, bool recompute) {
  int rc = check_gemm_dims(dims);
  if (rc != DMOE_OK) return rc;
  if (x && (rc = check_fused(dims)) != DMOE_OK) return rc;
  if ((rc = check_meta(meta)) != DMOE_OK) return rc;
  if (!dy || !weights || !w1 || !w3 || !w2 || !saved || !scratch || !dx || !dw1 ||
      !dw3 || !dw2 || !d_weights || !saved->x_perm || !saved->h1 || !saved->h3 ||
      !saved->act || !saved->y_perm || !scratch->dy_perm || !scratch->dh1 ||
      !scratch->dh3 || !scratch->dx_perm)
    return DMOE_ERR_ARG;
  const Shape s = shape_of(dims);
  const MetaPtrs m = meta_ptrs(meta);
  Recorder rec{ev, stream};
  int i = 0;
  if (recompute) {
    // before the down dgrad, which may overwrite h1 and h3 (dh1, dh3 alias)
    DMOE_TRY(rec(i++));
    DMOE_TRY(dmoe::launch_recompute_act(s, saved->h1, saved->h3, m, saved->act, stream));
  }
  // Order matters for the permitted aliases: dy_perm is last read by the
  // down-projection weight gradient, before dx_perm is written.
  DMOE_TRY(rec(i++));
  DMOE_TRY(dmoe::launch_scatter_backward(s, dy, saved->y_perm, weights, m,
                                         scratch->dy_perm, d_weights, stream));
  DMOE_TRY(rec(i++));
  DMOE_TRY(dmoe::launch_gemm_down_dgrad_wgrad_down(s, scratch->dy_perm, w2, saved->h1,
                                                   saved->h3, saved->act, m, scratch->dh1,
                                                   scratch->dh3, dw2, stream));
  DMOE_TRY(rec(i++));
  if (x) {
    // the forward did not keep x_perm: gather it for the products that read
    // it (dw1/dw3, some of them in the up dgrad's launch)
    DMOE_TRY(dmoe::launch_padded_gather(s, x, m, saved->x_perm, stream));
    DMOE_TRY(rec(i++));
  }
  DMOE_TRY(dmoe::launch_gemm_up_dgrad(s, scratch->dh1, scratch->dh3, w1, w3, saved->x_perm, m,
                                      scratch->dx_perm, dw1, dw3, stream));
  DMOE_TRY(rec(i++));
  // the gather's backward right away, while dx_perm is still in the
  // last-level cache
  DMOE_TRY(dmoe::launch_padded_scatter(s, scratch->dx_perm, nullptr, m, dx, stream));
  DMOE_TRY(rec(i++));
  DMOE_TRY(dmoe::launch_gemm_wgrad_up(s, scratch->dh1, scratch->dh3, w1, w3, saved->x_perm, m,
                                      scratch->dx_perm, dw1, dw3, stream));
  DMOE_TRY(rec(i++));
  return DMOE_OK;
}

}  // namespace

extern "C" {

int dmoe_backward_timed(const dmoe_dims* dims, const void* dy, const float* weights,
                        const void* w1, const void* w3, const void* w2,
                        const dmoe_meta* meta, const dmoe_saved* saved,
                        const dmoe_grad_scratch* scratch, void* dx, void* dw1,
                        void* dw3, void* dw2, float* d_weights, hipStream_t stream,
                        hipEvent_t* ev) {
  return backward_impl(dims, nullptr, dy, weights, w1, w3, w2, meta, saved, scratch, dx, dw1,
                       dw3, dw2, d_weights, stream, ev, false);
}

int dmoe_backward(const dmoe_dims* dims, const void* dy, const float* weights,
                  const void* w1, const void* w3, const void* w2,
                  const dmoe_meta* meta, const dmoe_saved* saved,
                  const dmoe_grad_scratch* scratch, void* dx, void* dw1,
                  void* dw3, void* dw2, float* d_weights, hipStream_t stream) {
  return backward_impl(dims, nullptr, dy, weights, w1, w3, w2, meta, saved, scratch, dx, dw1,
                       dw3, dw2, d_weights, stream, nullptr, false);
}

int dmoe_backward_recompute_timed(const dmoe_dims* dims, const void* dy, const float* weights,
                                  const void* w1, const void* w3, const void* w2,
                                  const dmoe_meta* meta, const dmoe_saved* saved,
                                  const dmoe_grad_scratch* scratch, void* dx, void* dw1,
                                  void* dw3, void* dw2, float* d_weights, hipStream_t stream,
                                  hipEvent_t* ev) {
  return backward_impl(dims, nullptr, dy, weights, w1, w3, w2, meta, saved, scratch, dx, dw1,
                       dw3, dw2, d_weights, stream, ev, true);
}

int dmoe_backward_recompute(const dmoe_dims* dims, const void* dy, const float* weights,
                            const void* w1, const void* w3, const void* w2,
                            const dmoe_meta* meta, const dmoe_saved* saved,
                            const dmoe_grad_scratch* scratch, void* dx, void* dw1,
                            void* dw3, void* dw2, float* d_weights, hipStream_t stream) {
  return backward_impl(dims, nullptr, dy, weights, w1, w3, w2, meta, saved, scratch, dx, dw1,
                       dw3, dw2, d_weights, stream, nullptr, true);
}

int dmoe_backward_fused_gather_timed(const dmoe_dims* dims, const void* x, const void* dy,
                                     const float* weights, const void* w1, const void* w3,
                                     const void* w2, const dmoe_meta* meta,
                                     const dmoe_saved* saved, const dmoe_grad_scratch* scratch,
                                     void* dx, void* dw1, void* dw3, void* dw2, float* d_weights,
                                     hipStream_t stream, hipEvent_t* ev) {
  if (!x) return DMOE_ERR_ARG;
  return backward_impl(dims, x, dy, weights, w1, w3, w2, meta, saved, scratch, dx, dw1, dw3, dw2,
                       d_weights, stream, ev, false);
}

int dmoe_backward_fused_gather(const dmoe_dims* dims, const void* x, const void* dy,
                               const float* weights, const void* w1, const void* w3,
                               const void* w2, const dmoe_meta* meta, const dmoe_saved* saved,
                               const dmoe_grad_scratch* scratch, void* dx, void* dw1, void* dw3,
                               void* dw2, float* d_weights, hipStream_t stream) {
  return dmoe_backward_fused_gather_timed(dims, x, dy, weights, w1, w3, w2, meta, saved, scratch,
                                          dx, dw1, dw3, dw2, d_weights, stream, nullptr);
}

int dmoe_padded_gather(const dmoe_dims* dims, const void* x, const dmoe_meta* meta,
                       void* x_perm, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != DMOE_OK) return rc;
  if ((rc = check_meta(meta)) != DMOE_OK) return rc;
  if (!x || !x_perm) return DMOE_ERR_ARG;
  DMOE_TRY(dmoe::launch_padded_gather(shape_of(dims), x, meta_ptrs(meta), x_perm, stream));
  return DMOE_OK;
}

int dmoe_padded_scatter(const dmoe_dims* dims, const void* src_perm,
                        const float* weights, const dmoe_meta* meta, void* out,
                        hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != DMOE_OK) return rc;
  if ((rc = check_meta(meta)) != DMOE_OK) return rc;
  if (!src_perm || !out) return DMOE_ERR_ARG;
  DMOE_TRY(dmoe::launch_padded_scatter(shape_of(dims), src_perm, weights, meta_ptrs(meta),
                                       out, stream));
  return DMOE_OK;
}

int dmoe_router_forward(const dmoe_dims* dims, const float* logits, float zloss_coef,
                        int32_t* top_experts, float* weights, float* z, float* zloss,
                        hipStream_t stream) {
  const int rc = check_dims(dims);
  if (rc != DMOE_OK) return rc;
  if (!logits || !top_experts || !weights) return DMOE_ERR_ARG;
  if (zloss_coef != 0.0f && (!z || !zloss)) return DMOE_ERR_ARG;
  DMOE_TRY(dmoe::launch_router_forward(shape_of(dims), logits, zloss_coef, top_experts,
                                       weights, zloss_coef != 0.0f ? z : nullptr, zloss,
                                       stream));
  return DMOE_OK;
}

int dmoe_router_backward(const dmoe_dims* dims, const float* logits,
                         const int32_t* top_experts, const float* weights,
                         const float* d_weights, float zloss_coef, float* d_logits,
                         hipStream_t stream) {
  const int rc = check_dims(dims);
  if (rc != DMOE_OK) return rc;
  if (!logits || !top_experts || !weights || !d_weights || !d_logits) return DMOE_ERR_ARG;
  DMOE_TRY(dmoe::launch_router_backward(shape_of(dims), logits, top_experts, weights,
                                        d_weights, zloss_coef, d_logits, stream));
  return DMOE_OK;
}

const char* dmoe_status_string(int status) {
  switch (status) {
    case DMOE_OK: return "ok";
    case DMOE_ERR_ARG: return "invalid argument (null pointer, non-positive size, k > E or too many entries)";
    case DMOE_ERR_SHAPE: return "H and F must be multiples of 128";
    case DMOE_ERR_UNSUPPORTED: return "unsupported (E > 256, dtype, H/F too large, or more than 65535 row blocks)";
    case DMOE_ERR_HIP: return "HIP kernel launch failed";
    case DMOE_ERR_EXPERT_ID: return "an expert id is outside [0, E)";
    default: return "unknown dmoe status";
  }
}

}  // extern "C"
