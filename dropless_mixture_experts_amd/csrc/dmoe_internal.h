// Host-side declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmoe {

constexpr int kMaxExperts = 256;
constexpr int kErrExpertId = -5;   // matches DMOE_ERR_EXPERT_ID

// The metadata arrays, and the two tables of the opaque schedule buffer
// (dmoe_meta.schedule), which holds, as int32:
//   [0, max_tiles)              pair_first: group s of row blocks starts at
//                               block pair_first[s] and also takes the next
//                               block when it belongs to the same expert
//                               (each expert's blocks paired in order, an
//                               odd last one single); -1 past the last group
//   [max_tiles]                 num_pairs: the number of groups
struct MetaPtrs {
  int32_t *tokens_per_expert, *bins, *padded_bins;
  int32_t *indices, *bin_ids, *row_of_entry;
  int32_t *tile_expert, *num_padded_rows, *status;
  int32_t *pair_first, *num_pairs;
  int32_t *row_token;
};

// Bytes of the schedule buffer for max_tiles 128-row blocks.
inline int64_t schedule_bytes(int64_t max_tiles) {
  return ((max_tiles + 1) * 4 + 255) / 256 * 256;
}

struct Shape {
  int64_t T, H, F;
  int E, k;
  int64_t max_tiles;
  bool bf16;
};

// meta.hip
int64_t meta_chunk(int64_t n, int E);
int meta_nchunks(int64_t n, int E);
int64_t meta_workspace_bytes(int64_t n, int E);
hipError_t launch_metadata(int64_t n, int E, int k, int64_t max_tiles,
                           const int32_t* ids, const MetaPtrs& m, void* ws,
                           hipStream_t stream, hipEvent_t* ev);

// permute.hip
hipError_t launch_padded_gather(const Shape& s, const void* x, const MetaPtrs& m,
                                void* x_perm, hipStream_t stream);
hipError_t launch_padded_scatter(const Shape& s, const void* src_perm,
                                 const float* weights, const MetaPtrs& m,
                                 void* out, hipStream_t stream);
hipError_t launch_scatter_backward(const Shape& s, const void* dy,
                                   const void* y_perm, const float* weights,
                                   const MetaPtrs& m, void* dy_perm,
                                   float* d_weights, hipStream_t stream);
// Slot order (T*k rows of W elements) <-> padded order: out[a] = src_perm[row(a)]
// (zeros for an empty slot); dst_perm[row(a)] = src[a] with the pad rows zeroed.
hipError_t launch_slot_unpermute(const Shape& s, int64_t W, const void* src_perm,
                                 const MetaPtrs& m, void* out, hipStream_t stream);
hipError_t launch_slot_permute(const Shape& s, int64_t W, const void* src, const MetaPtrs& m,
                               void* dst_perm, hipStream_t stream);

// token_round.hip: tile-aware token rounding of the router's top-k (s.k
// routed slots, outputs [T, s.k + 1]); M rows per tile.
int64_t token_round_workspace_bytes(int64_t T, int E, int k);
hipError_t launch_token_round(const Shape& s, const float* logits, int M, int32_t* out_ids,
                              float* out_w, void* ws, hipStream_t stream);

// activation.hip: act = silu(h1) * h3 over rows [0, P) (backward recompute)
hipError_t launch_recompute_act(const Shape& s, const void* h1, const void* h3,
                                const MetaPtrs& m, void* act, hipStream_t stream);

// router.hip
hipError_t launch_router_forward(const Shape& s, const float* logits, float coef,
                                 int32_t* ids, float* weights, float* z, float* loss,
                                 hipStream_t stream);
hipError_t launch_router_backward(const Shape& s, const float* logits, const int32_t* ids,
                                  const float* weights, const float* d_weights, float coef,
                                  float* d_logits, hipStream_t stream);

// gemm.hip: the products of the layer.  bf16 runs on the engine in
// gemm_bf16.hip; fp32 on the tiled kernels of gemm.hip.  In the up
// projection, a non-null x (bf16 only) makes it read each padded row's token
// row of x through m.row_token (zeros for a pad row) instead of x_perm.
hipError_t launch_gemm_up(const Shape& s, const void* x_perm, const void* x, const void* w1,
                          const void* w3, const MetaPtrs& m, void* h1, void* h3,
                          void* act, hipStream_t stream);
hipError_t launch_gemm_down(const Shape& s, const void* act, const void* w2,
                            const MetaPtrs& m, void* y_perm, hipStream_t stream);
// down dgrad + gate backward (dh1, dh3) and dw2; one launch for bf16
hipError_t launch_gemm_down_dgrad_wgrad_down(const Shape& s, const void* dy_perm,
                                             const void* w2, const void* h1, const void* h3,
                                             const void* act, const MetaPtrs& m, void* dh1,
                                             void* dh3, void* dw2, hipStream_t stream);
// up dgrad (dx_perm) and dw1/dw3 as two calls, with the gather's backward
// between them: for bf16 the first also computes the dw1/dw3 tiles that
// fill its last round, the second the others.  Both take every operand.
hipError_t launch_gemm_up_dgrad(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const void* x_perm,
                                const MetaPtrs& m, void* dx_perm, void* dw1, void* dw3,
                                hipStream_t stream);
hipError_t launch_gemm_wgrad_up(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const void* x_perm,
                                const MetaPtrs& m, void* dx_perm, void* dw1, void* dw3,
                                hipStream_t stream);

// gemm_bf16.hip
hipError_t launch_bf16_up(const Shape& s, const void* x_perm, const void* x, const void* w1,
                          const void* w3, const MetaPtrs& m, void* h1, void* h3, void* act,
                          hipStream_t stream);
hipError_t launch_bf16_down(const Shape& s, const void* act, const void* w2,
                            const MetaPtrs& m, void* y_perm, hipStream_t stream);
hipError_t launch_bf16_down_dgrad_wgrad_down(const Shape& s, const void* dy_perm,
                                             const void* w2, const void* h1, const void* h3,
                                             const void* act, const MetaPtrs& m, void* dh1,
                                             void* dh3, void* dw2, hipStream_t stream);
hipError_t launch_bf16_up_dgrad(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const void* x_perm,
                                const MetaPtrs& m, void* dx_perm, void* dw1, void* dw3,
                                hipStream_t stream);
hipError_t launch_bf16_wgrad_up(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const void* x_perm,
                                const MetaPtrs& m, void* dx_perm, void* dw1, void* dw3,
                                hipStream_t stream);
// A single grouped linear map y = x w[e] (w [E, H, F]): its dgrad
// dx_perm [P, H] = dy_perm [P, F] w[e]^T and its weight gradient
// dw [E, H, F] = x_perm [P, H]^T dy_perm [P, F], in one launch.
hipError_t launch_bf16_dgrad_wgrad(const Shape& s, const void* dy_perm, const void* w,
                                   const void* x_perm, const MetaPtrs& m, void* dx_perm,
                                   void* dw, hipStream_t stream);

}  // namespace dmoe
