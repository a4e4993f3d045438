/*
 * dmoe.h -- C ABI of the dropless mixture-of-experts (dMoE) expert layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer, as the MegaBlocks chapter "02 · dropless MoE 与 block-sparse 重构"
 * describes it: every (token, slot) entry chosen by the router is kept (no
 * capacity, no dropping, §1); the entries are sorted by expert, each
 * expert's count is rounded up to a multiple of 128 so that every 128-row
 * block belongs to one expert (§2, §4.1); token rows are copied into that
 * padded layout (padded_gather, §4.2); each expert's FFN runs on its row
 * blocks only (the sdd/dsd pair of §3, here gated SiLU as in the Fast-LLM
 * issue "[feat] Support sparse copy for a large number of experts"); the
 * results are copied back, scaled by the routing weight and summed over the
 * k slots (padded_scatter, §4.2).  The backward pairs gather with scatter
 * and adds the routing-weight gradient (§4.2).
 *
 *   y[t] = sum_j weights[t,j] * ( silu(x[t] w1[e]) * (x[t] w3[e]) ) w2[e],
 *          e = top_experts[t,j],  silu(z) = z / (1 + exp(-z)).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers.  Every array argument is a DEVICE pointer owned by the caller.
 *   The library allocates nothing, frees nothing and never synchronises
 *   the host: all work is enqueued on `stream` (a hipStream_t; NULL is the
 *   default stream).  No state is kept between calls; calls on different
 *   streams with disjoint buffers may run concurrently.
 * - Layouts.  Row-major and contiguous.  x, dy, dx, y: [T,H].
 *   top_experts: int32 [T,k].  weights, d_weights: fp32 [T,k] for every
 *   dtype.  w1, w3, dw1, dw3: [E,H,F].  w2, dw2: [E,F,H].  The floating
 *   arrays other than weights/d_weights are all of `dims->dtype`.
 * - Entry numbering.  Entry a = t*k + j is slot j of token t.
 * - Empty slots.  An expert id of -1 is an empty slot: the entry is routed
 *   nowhere (row_of_entry = -1, no padded row), adds nothing to y or dx and
 *   gets d_weights = 0, so a token may use fewer than k experts (for
 *   instance after dmoe_token_round).  The sorted arrays (indices, bin_ids)
 *   list the routed entries only and hold -1 past them, and bins[E-1] is
 *   their number.
 * - Padded rows.  P = padded_bins[E-1] is known only on the device
 *   (meta.num_padded_rows).  Buffers with padded rows are sized for
 *   P_max = 128 * dmoe_max_tiles(dims) rows.  Rows in [P, P_max) are left
 *   untouched.  Pad rows inside [0, P) are written as exact zeros.
 * - Precision.  bf16 inputs are multiplied on the matrix cores with fp32
 *   accumulation; every stored intermediate (x_perm, h1, h3, act, y_perm,
 *   dy_perm, dh1, dh3, dx_perm) and every output is rounded once to the
 *   I/O dtype (round to nearest even).  The top-k sums run in fp32 in slot
 *   order.  fp32 runs in full fp32.
 * - Determinism.  No reduction uses atomics; results are bitwise
 *   reproducible run to run.
 * - Errors.  Argument and shape errors are detected on the host before any
 *   launch and returned as a negative dmoe_status; nothing is enqueued then.
 *   An expert id outside [0,E) other than -1 is a data error found on the
 *   device:
 *   dmoe_metadata stores DMOE_ERR_EXPERT_ID in meta.status (0 otherwise),
 *   the offending entries get row_of_entry = -1 and contribute nothing;
 *   other outputs are then unspecified.  The caller reads meta.status after
 *   its own synchronisation.  A failed launch returns DMOE_ERR_HIP.
 */
#ifndef DMOE_H
#define DMOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DMOE_BLOCK 128       /* rows per padded block (MegaBlocks §2) */
#define DMOE_MAX_EXPERTS 256

typedef enum {
  DMOE_OK = 0,
  DMOE_ERR_ARG = -1,         /* null pointer, non-positive size, k > E, T*k >= 2^31 */
  DMOE_ERR_SHAPE = -2,       /* F % 128 != 0 (MegaBlocks §5) or H % 128 != 0 */
  DMOE_ERR_UNSUPPORTED = -3, /* E > 256, an unknown dtype, H or F > 2^24, or
                                (forward/backward) more than 65535 row blocks;
                                for fp32, more than 32767 row blocks or 65535
                                64-column blocks of H or F */
  DMOE_ERR_HIP = -4,         /* a kernel launch failed */
  DMOE_ERR_EXPERT_ID = -5    /* device-side: an expert id outside [0,E) */
} dmoe_status;

typedef enum { DMOE_F32 = 0, DMOE_BF16 = 1 } dmoe_dtype;

/* Problem sizes.  T tokens, hidden size H, per-expert ffn size F, E experts,
 * top-k slots per token, element type of the floating arrays. */
typedef struct {
  int64_t T, H, F;
  int32_t E, k;
  int32_t dtype;             /* a dmoe_dtype */
} dmoe_dims;

/* Routing metadata, written by dmoe_metadata and read by the other calls
 * (MegaBlocks §4.1-§4.3).  Device arrays owned by the caller.
 *   tokens_per_expert[E]  int32, histogram of the expert ids
 *   bins[E]               int32, inclusive cumsum of tokens_per_expert
 *   padded_bins[E]        int32, inclusive cumsum of round_up(tokens_per_expert, 128)
 *   indices[T*k]          int32, stable sort of the routed entries by expert:
 *                         indices[s] = a; -1 past the routed entries
 *   bin_ids[T*k]          int32, expert of the s-th sorted entry
 *   row_of_entry[T*k]     int32, padded row of entry a:
 *                         (s - bins[e-1]) + padded_bins[e-1], both starts 0 at e=0
 *   tile_expert[max_tiles] int32, expert owning 128-row block r; -1 for r >= P/128
 *   num_padded_rows[1]    int32, P = padded_bins[E-1]
 *   status[1]             int32, 0, or DMOE_ERR_EXPERT_ID
 *   row_token[max_tiles*128] int32, the token whose row padded row p holds:
 *                         a / k for the entry a placed there (the §4.2 index
 *                         rule read from the row side), -1 for a pad row
 *                         below P; rows from P on are left untouched
 *   schedule              opaque, dmoe_schedule_bytes(dims) bytes: the order
 *                         in which the grouped matrix products take their
 *                         tiles, derived from the counts by dmoe_metadata and
 *                         read by the forward and backward calls.  It is not
 *                         part of the method's result; its layout is private
 *                         to the library and may change without changing
 *                         this struct.                                         */
typedef struct {
  int32_t *tokens_per_expert, *bins, *padded_bins;
  int32_t *indices, *bin_ids, *row_of_entry;
  int32_t *tile_expert;
  int32_t *num_padded_rows;
  int32_t *status;
  int32_t *row_token;
  void *schedule;
} dmoe_meta;

/* Activations kept from forward for backward, each [P_max, H] or [P_max, F]
 * of dtype: x_perm [.,H] (padded_gather output), h1 = x_perm w1, h3 = x_perm w3,
 * act = silu(h1)*h3 [.,F], y_perm = act w2 [.,H]. */
typedef struct {
  void *x_perm, *h1, *h3, *act, *y_perm;
} dmoe_saved;

/* Backward intermediates, caller-owned: dy_perm [.,H], dh1, dh3 [.,F],
 * dx_perm [.,H], all [P_max, .] of dtype.  dh1 may alias saved.h1, dh3 may
 * alias saved.h3 and dx_perm may alias dy_perm (each element is read before
 * it is overwritten); no other aliasing is allowed. */
typedef struct {
  void *dy_perm, *dh1, *dh3, *dx_perm;
} dmoe_grad_scratch;

/* Number of 128-row blocks that bound P:
 * floor((T*k + 127*min(E, T*k)) / 128), since each non-empty expert adds at
 * most 127 pad rows (MegaBlocks §2).  Returns a negative dmoe_status on bad
 * dims. */
int64_t dmoe_max_tiles(const dmoe_dims* dims);

/* Bytes of device workspace `ws` that dmoe_metadata needs: per-chunk
 * expert histograms and error flags, scratch that is dead once the call's
 * kernels have run (the same ws may serve other work afterwards, in stream
 * order).  The forward and backward calls need no workspace: no product is
 * split along K and no reduction uses atomics, so there are no partial
 * results to keep.  At most 4 210 688 bytes (4096 chunks x (256 + 1) int32).
 * Returns a negative dmoe_status on bad dims. */
int64_t dmoe_workspace_bytes(const dmoe_dims* dims);

/* Bytes of dmoe_meta.schedule for these dims (a few KB: 4 * (max_tiles + 1)
 * rounded up to 256).  Returns a negative dmoe_status on bad dims. */
int64_t dmoe_schedule_bytes(const dmoe_dims* dims);

/* Routing metadata (MegaBlocks §4.1 sort / histogram / cumsum and round_up,
 * §4.2 padded row of each entry, §4.3 row block -> expert).
 * top_experts: int32 [T,k] device.  Writes every array of *meta.
 * ws: device scratch of dmoe_workspace_bytes(dims) bytes; contents on entry
 * are ignored.  LDS use is O(E) and independent of T. */
int dmoe_metadata(const dmoe_dims* dims, const int32_t* top_experts,
                  const dmoe_meta* meta, void* ws, hipStream_t stream);

/* dmoe_metadata without the workspace argument, for callers that cannot
 * allocate device memory at all (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same results as
 * dmoe_metadata, bit for bit.  The workspace is a 4 210 688-byte array in
 * the library's own device memory (one per GPU, held until the process
 * ends), which this call neither allocates nor frees.  Every call on one
 * GPU uses that GPU's one array: calls that may overlap in time on one GPU
 * (different streams, or different host threads without stream order
 * between them) race and give unspecified metadata; calls in the order of
 * one stream do not.  Dims whose workspace would exceed the array return
 * DMOE_ERR_UNSUPPORTED (none do under the limits DMOE_ERR_ARG enforces). */
int dmoe_metadata_noalloc(const dmoe_dims* dims, const int32_t* top_experts,
                          const dmoe_meta* meta, hipStream_t stream);

/* Forward: padded_gather (MegaBlocks §4.2) -> per-128-row-block gated-SiLU
 * up projection (the sdd of §3, GLU variant of §5) -> down projection (the
 * dsd of §3) -> padded_scatter with the routing weights and the top-k sum
 * (§4.2, §4.5).  Reads x, weights, w1, w3, w2 and *meta (from
 * dmoe_metadata); writes every buffer of *saved and y [T,H]. */
int dmoe_forward(const dmoe_dims* dims, const void* x, const float* weights,
                 const void* w1, const void* w3, const void* w2,
                 const dmoe_meta* meta, const dmoe_saved* saved, void* y,
                 hipStream_t stream);

/* Backward of dmoe_forward for upstream gradient dy [T,H] (MegaBlocks §4.2:
 * the scatter's backward is a gather of dy times the routing weight plus the
 * routing-weight gradient d_weights[a] = <dy[a/k], y_perm[row_of_entry[a]]>;
 * the gather's backward is a scatter summing the k slots).  Reads *saved
 * from the forward of the same inputs.  Writes dx [T,H], dw1, dw3 [E,H,F],
 * dw2 [E,F,H] (overwritten, not accumulated; experts with no rows get
 * zeros), d_weights fp32 [T,k] and every buffer of *scratch. */
int dmoe_backward(const dmoe_dims* dims, const void* dy, const float* weights,
                  const void* w1, const void* w3, const void* w2,
                  const dmoe_meta* meta, const dmoe_saved* saved,
                  const dmoe_grad_scratch* scratch, void* dx, void* dw1,
                  void* dw3, void* dw2, float* d_weights, hipStream_t stream);

/* dmoe_backward for callers that did not keep the activation: the
 * memory-optimized MLP of the MegaBlocks chapter (§4.4) recomputes the
 * activation in the backward instead of storing it.  saved->act is scratch
 * on entry (its contents are ignored, so its memory may serve other work
 * between forward and backward); the call first rebuilds act = silu(h1) *
 * h3 from saved->h1 and saved->h3, bit-identical to the forward's, and
 * leaves it there.  Every other buffer and every result are as for
 * dmoe_backward, bit for bit. */
int dmoe_backward_recompute(const dmoe_dims* dims, const void* dy, const float* weights,
                            const void* w1, const void* w3, const void* w2,
                            const dmoe_meta* meta, const dmoe_saved* saved,
                            const dmoe_grad_scratch* scratch, void* dx, void* dw1,
                            void* dw3, void* dw2, float* d_weights, hipStream_t stream);

/* The backward for callers that keep only y_perm of the forward's saved
 * activations: the memory-optimized MLP of the MegaBlocks chapter (§4.4)
 * taken to the whole up projection.  x is the forward's input [T,H], which
 * the caller holds anyway.  saved->x_perm, h1, h3 and act are scratch on
 * entry (their memory may serve other work between forward and backward);
 * the call first gathers x_perm from x and reruns the up projection into
 * h1, h3 and act -- the forward's kernels on the forward's input, so the
 * same bits -- then runs the backward of dmoe_backward.  saved->y_perm must
 * hold the forward's y_perm (the routing-weight gradient reads it).  Every
 * result and every buffer is then bit-identical to dmoe_forward +
 * dmoe_backward on the same inputs.  Kept between forward and backward: H
 * elements per padded row instead of 2H + 3F.  Costs one more up
 * projection (4 P H F flops) and one more gather.  Either forward may
 * precede it. */
int dmoe_backward_lean(const dmoe_dims* dims, const void* x, const void* dy,
                       const float* weights, const void* w1, const void* w3, const void* w2,
                       const dmoe_meta* meta, const dmoe_saved* saved,
                       const dmoe_grad_scratch* scratch, void* dx, void* dw1, void* dw3,
                       void* dw2, float* d_weights, hipStream_t stream);

/* The forward with the gather fused into the up projection's operand loads
 * (bf16 only), and its backward.  Fine-grained experts are bound by memory
 * IO, and overlapping that IO with the products is how the pages' own
 * design answers it ("SonicMoE: Accelerating MoE with IO and Tile-aware
 * Optimizations", abstract).  Here the up projection fetches padded row p
 * as token row meta.row_token[p] of x (zeros for a pad row) straight into
 * its tiles, so the forward writes no x_perm: the padded copy of
 * MegaBlocks §4.2 is never made in the forward and need not be kept until
 * the backward.  dmoe_backward_fused_gather takes the forward's x and
 * gathers x_perm into saved->x_perm, which is scratch on entry (its memory
 * may serve other work between forward and backward), before the products
 * that read it.  Every result and every other saved or scratch
 * buffer is bit-identical to dmoe_forward / dmoe_backward on the same
 * inputs.
 *   dmoe_forward_fused_gather: saved->x_perm may be NULL (it is not used).
 * DMOE_ERR_UNSUPPORTED for fp32 or when T*H*2 >= 2^31 (x is read through a
 * buffer resource of T*H*2 bytes). */
int dmoe_forward_fused_gather(const dmoe_dims* dims, const void* x, const float* weights,
                              const void* w1, const void* w3, const void* w2,
                              const dmoe_meta* meta, const dmoe_saved* saved, void* y,
                              hipStream_t stream);
int dmoe_backward_fused_gather(const dmoe_dims* dims, const void* x, const void* dy,
                               const float* weights, const void* w1, const void* w3,
                               const void* w2, const dmoe_meta* meta, const dmoe_saved* saved,
                               const dmoe_grad_scratch* scratch, void* dx, void* dw1, void* dw3,
                               void* dw2, float* d_weights, hipStream_t stream);

/* padded_gather alone (MegaBlocks §4.2, gather direction): for every real
 * padded row p of entry a, x_perm[p] = x[a / k]; pad rows below P are zero.
 * x [T,H], x_perm [P_max,H] of dtype; *meta from dmoe_metadata. */
int dmoe_padded_gather(const dmoe_dims* dims, const void* x, const dmoe_meta* meta,
                       void* x_perm, hipStream_t stream);

/* padded_scatter alone (MegaBlocks §4.2, scatter direction, and the top-k
 * sum of §4.5): out[t] = sum_j w[t,j] * src_perm[row_of_entry[t*k+j]], in
 * fp32 in slot order, rounded once.  weights may be NULL for unit weights
 * (the gather's backward).  src_perm [P_max,H], out [T,H] of dtype. */
int dmoe_padded_scatter(const dmoe_dims* dims, const void* src_perm,
                        const float* weights, const dmoe_meta* meta, void* out,
                        hipStream_t stream);

/* The router in front of the layer (Fast-LLM issue "[feat] Support sparse
 * copy for a large number of experts": each token goes to k of E experts,
 * with an expert z-loss coefficient; "yikangshen/megablocks" README: the
 * router z-loss of ST-MoE).
 *   logits [T,E] fp32, finite (results are unspecified for NaN or inf).
 *   top_experts [T,k] int32: the k largest logits of each token in
 *     descending order, equal logits to the lower expert id (unique).
 *   weights [T,k] fp32: the softmax over the k chosen logits.
 *   zloss_coef: the z-loss weight; 0 skips it, and z and zloss may be NULL.
 *   z [T] fp32: (log sum_e exp logits[t,e])^2 per token.
 *   zloss [1] fp32: zloss_coef * mean_t z[t], summed in a fixed order.
 * Only dims->T, E and k are used (H, F and dtype are checked as for the
 * layer).  Returns a negative dmoe_status on bad arguments; nothing is
 * enqueued then. */
int dmoe_router_forward(const dmoe_dims* dims, const float* logits, float zloss_coef,
                        int32_t* top_experts, float* weights, float* z, float* zloss,
                        hipStream_t stream);

/* Backward of dmoe_router_forward for upstream d_weights [T,k] fp32 (and
 * unit weight on zloss): the selection carries no gradient, so
 *   d_logits[t, top_experts[t,j]] = w_j (d_weights[t,j] - sum_i w_i d_weights[t,i])
 * and 0 at the other experts, plus zloss_coef * 2 / T * lse_t *
 * softmax(logits[t])_e at every expert when zloss_coef != 0.
 * logits, top_experts and weights as produced by the forward; d_logits [T,E]
 * fp32 is overwritten.  Ids outside [0, E) are ignored. */
int dmoe_router_backward(const dmoe_dims* dims, const float* logits,
                         const int32_t* top_experts, const float* weights,
                         const float* d_weights, float zloss_coef, float* d_logits,
                         hipStream_t stream);

/* Tile-aware token rounding of the router's choice ("SonicMoE: Accelerating
 * MoE with IO and Tile-aware Optimizations", abstract: round each expert's
 * token count to the grouped GEMM's tile instead of padding it).  The page
 * gives no rule; this one is taken: each token is routed to its k largest
 * logits (the order of dmoe_router_forward) and its (k+1)-th largest is
 * its candidate; an expert with c routed tokens and r = c mod tile_rows > 0
 * takes its tile_rows - r best candidates (largest logit, then lower token
 * id) when tile_rows - r < r and it has that many, and otherwise drops its
 * r worst routed tokens (smallest logit, then higher token id).
 *   logits [T,E] fp32, finite; dims->k = k routed slots, 1 <= k < E.
 *   top_experts [T,k+1] int32: slot j < k the j-th routed expert or -1 when
 *     dropped; slot k the candidate when taken, else -1.
 *   weights [T,k+1] fp32: the softmax over the logits of the occupied slots,
 *     0 in empty slots (all 0 for a token left with no expert).
 *   ws: dmoe_token_round_workspace_bytes(dims) bytes of scratch.
 * Every expert then has a multiple of tile_rows tokens; with tile_rows =
 * 128 the layer called on these slots (dims->k = k + 1) computes no pad
 * rows.  Bit-reproducible.  DMOE_ERR_ARG for k >= E, tile_rows < 1, null
 * pointers, or T*(k+1) at 2^31 or more. */
int64_t dmoe_token_round_workspace_bytes(const dmoe_dims* dims);
int dmoe_token_round(const dmoe_dims* dims, const float* logits, int32_t tile_rows,
                     int32_t* top_experts, float* weights, void* ws, hipStream_t stream);

/* The metadata, forward and backward calls with per-kernel timing.  `events`
 * is NULL or an array of n+1 hipEvent_t; event i is recorded on `stream`
 * just before kernel i and event n after the last kernel, so the elapsed
 * time between events i and i+1 is kernel i's duration on the stream plus
 * the cost of one record (about 4.4 us on MI355X: the interval between two
 * records with nothing between them).  An entry may be NULL: that record is
 * skipped (each record puts a timestamp between two kernels, so timing one
 * kernel with two records disturbs the sequence less than timing all of
 * them).
 *   metadata (n = 3): histogram, scan, placement.
 *   forward  (n = 4): padded_gather, up projection + SiLU gate, down
 *                     projection, padded_scatter.
 *   backward (n = 5): scatter backward (dy_perm, d_weights), down dgrad +
 *                     gate backward together with dw2 (one launch for
 *                     bf16), up dgrad (dx_perm; for bf16 possibly with the
 *                     first dw1/dw3 tiles), gather backward (dx), dw1 + dw3.
 *   backward_recompute (n = 6): the activation recompute, then the five
 *                     kernels of the backward.
 *   backward_lean (n = 7): padded_gather (x_perm), up projection + SiLU
 *                     gate, then the five kernels of the backward.
 *   forward_fused_gather (n = 3): the forward's kernels but padded_gather.
 *   backward_fused_gather (n = 6): scatter backward, down dgrad + dw2,
 *                     padded_gather (x_perm), up dgrad, gather backward,
 *                     dw1 + dw3.
 * Results are identical to the untimed calls. */
int dmoe_metadata_timed(const dmoe_dims* dims, const int32_t* top_experts,
                        const dmoe_meta* meta, void* ws, hipStream_t stream,
                        hipEvent_t* events);
int dmoe_forward_timed(const dmoe_dims* dims, const void* x, const float* weights,
                       const void* w1, const void* w3, const void* w2,
                       const dmoe_meta* meta, const dmoe_saved* saved, void* y,
                       hipStream_t stream, hipEvent_t* events);
int dmoe_backward_timed(const dmoe_dims* dims, const void* dy, const float* weights,
                        const void* w1, const void* w3, const void* w2,
                        const dmoe_meta* meta, const dmoe_saved* saved,
                        const dmoe_grad_scratch* scratch, void* dx, void* dw1,
                        void* dw3, void* dw2, float* d_weights, hipStream_t stream,
                        hipEvent_t* events);
int dmoe_backward_recompute_timed(const dmoe_dims* dims, const void* dy, const float* weights,
                                  const void* w1, const void* w3, const void* w2,
                                  const dmoe_meta* meta, const dmoe_saved* saved,
                                  const dmoe_grad_scratch* scratch, void* dx, void* dw1,
                                  void* dw3, void* dw2, float* d_weights, hipStream_t stream,
                                  hipEvent_t* events);

int dmoe_backward_lean_timed(const dmoe_dims* dims, const void* x, const void* dy,
                             const float* weights, const void* w1, const void* w3,
                             const void* w2, const dmoe_meta* meta, const dmoe_saved* saved,
                             const dmoe_grad_scratch* scratch, void* dx, void* dw1, void* dw3,
                             void* dw2, float* d_weights, hipStream_t stream, hipEvent_t* events);

int dmoe_forward_fused_gather_timed(const dmoe_dims* dims, const void* x, const float* weights,
                                    const void* w1, const void* w3, const void* w2,
                                    const dmoe_meta* meta, const dmoe_saved* saved, void* y,
                                    hipStream_t stream, hipEvent_t* events);
int dmoe_backward_fused_gather_timed(const dmoe_dims* dims, const void* x, const void* dy,
                                     const float* weights, const void* w1, const void* w3,
                                     const void* w2, const dmoe_meta* meta,
                                     const dmoe_saved* saved, const dmoe_grad_scratch* scratch,
                                     void* dx, void* dw1, void* dw3, void* dw2, float* d_weights,
                                     hipStream_t stream, hipEvent_t* events);

/* ---- dMoA: the map / reduce pair of mixture of attention heads ---------------
 *
 * "yikangshen/megablocks" README (the dMoA example): a causal self-attention
 * whose query projection is a dMoA layer built from the plain MLP expert
 * with no activation and no bias.  map(x) gives each token k query vectors,
 * one per routed expert; attention (not part of this library) turns them
 * into k outputs; reduce(y) projects each output with its expert and sums
 * the k slots with the routing weights.  Reading taken (the README prints no
 * formula): expert e is w1[e] [H, F] and w2[e] [F, H];
 *     map:    q[t*k + j]  = x[t] w1[e(t, j)]                   (no weight)
 *     reduce: out[t]      = sum_j weights[t*k + j] * y[t*k + j] w2[e(t, j)]
 * An empty slot (id -1) maps to a zero row and adds nothing.  The routing
 * and its metadata are the dMoE layer's (dmoe_metadata), so the pages'
 * padded layout and grouped products serve both.  The README's example has
 * F = H.
 *
 * bf16 only (DMOE_ERR_UNSUPPORTED for fp32); the dims rules of
 * dmoe_forward otherwise.  All pointers are device memory owned by the
 * caller; P_max = 128 * dmoe_max_tiles(dims).  Slot-order arrays have
 * T*k rows in entry order a = t*k + j.  Nothing is allocated, nothing
 * waits on the host, and argument errors return before any launch.  No two
 * array arguments of one call may overlap (each backward call computes its
 * dgrad and its weight gradient in one launch, so a scratch array that
 * aliased an input would be overwritten while it is read).
 *
 * dmoe_moa_map:     x [T, H] -> q [T*k, F].  x_perm [P_max, H] is written
 *                   (the padded copy of x, saved for dmoe_moa_map_backward);
 *                   q_perm [P_max, F] is scratch.
 * dmoe_moa_reduce:  y [T*k, F], weights fp32 [T*k] -> out [T, H].
 *                   y_perm [P_max, F] and o_perm [P_max, H] are written and
 *                   saved for dmoe_moa_reduce_backward.
 * dmoe_moa_reduce_backward: dout [T, H] -> dy [T*k, F] (zero rows for empty
 *                   slots), dw2 [E, F, H] (zero for an empty expert),
 *                   d_weights fp32 [T*k] (<dout[t], y[t*k+j] w2[e]>, 0 for
 *                   an empty slot).  do_perm [P_max, H] and dy_perm
 *                   [P_max, F] are scratch.
 * dmoe_moa_map_backward: dq [T*k, F] -> dx [T, H], dw1 [E, H, F].
 *                   x_perm is the one dmoe_moa_map wrote; dq_perm [P_max, F]
 *                   and dx_perm [P_max, H] are scratch. */
int dmoe_moa_map(const dmoe_dims* dims, const void* x, const void* w1, const dmoe_meta* meta,
                 void* x_perm, void* q_perm, void* q, hipStream_t stream);
int dmoe_moa_reduce(const dmoe_dims* dims, const void* y, const float* weights, const void* w2,
                    const dmoe_meta* meta, void* y_perm, void* o_perm, void* out,
                    hipStream_t stream);
int dmoe_moa_reduce_backward(const dmoe_dims* dims, const void* dout, const float* weights,
                             const void* w2, const dmoe_meta* meta, const void* y_perm,
                             const void* o_perm, void* do_perm, void* dy_perm, void* dy,
                             void* dw2, float* d_weights, hipStream_t stream);
int dmoe_moa_map_backward(const dmoe_dims* dims, const void* dq, const void* w1,
                          const dmoe_meta* meta, const void* x_perm, void* dq_perm,
                          void* dx_perm, void* dx, void* dw1, hipStream_t stream);

/* Static text for a dmoe_status value. */
const char* dmoe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DMOE_H */
