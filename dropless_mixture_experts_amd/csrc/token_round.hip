// Tile-aware token rounding (gfx950).
//
// "SonicMoE: Accelerating MoE with IO and Tile-aware Optimizations"
// (abstract) rounds the number of tokens each expert receives to the grouped
// GEMM's tile, so that the padding MegaBlocks §2 adds to every expert is not
// computed.  The page gives no rule; the one taken here:
//   * every token is routed to its k largest logits (the router's order:
//     descending, equal logits to the lower expert id); its (k+1)-th is its
//     candidate expert;
//   * an expert with c routed tokens and r = c mod M != 0 takes its M - r
//     best candidates (largest logit, then lower token id) when M - r < r
//     and it has that many; otherwise it drops its r worst routed tokens
//     (smallest logit, then higher token id);
//   * the result has k + 1 slots per token: slot j < k the j-th routed
//     expert or -1 when dropped, slot k the candidate when taken or -1; the
//     weights are the softmax over the occupied slots' logits (0 elsewhere).
// Every expert then holds a multiple of M tokens, so with M = 128 the padded
// layout of the layer has no pad rows.
//
// Four launches: the router's top-(k+1) selection, the layer's metadata on
// the k+1 slots (which groups each expert's routed tokens and candidates,
// stably), one workgroup per expert that decides and selects by a radix
// select on unique 64-bit keys (logit order, then token), and one thread per
// token that writes the slots and weights.  No atomics on global memory;
// the LDS histogram counts are integers, so results are bit-reproducible.
#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {

constexpr int kTrThreads = 256;

// The order of finite floats as unsigned keys (-0 taken as +0), as the
// router compares logits.
__device__ __forceinline__ uint32_t tr_order(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Entry key of token t for one expert: its logit, then the lower token id
// ranking higher.  Keys of one expert's entries are unique (a token lists
// an expert at most once among its k + 1 choices).  Taking: the largest
// keys; dropping: the smallest.
__device__ __forceinline__ uint64_t tr_key(float logit, int64_t t) {
  return ((uint64_t)tr_order(logit) << 32) | (uint64_t)(~(uint32_t)t);
}

// Inclusive sum over the 256 threads of the workgroup, in thread order: a
// shuffle scan inside each wave, then the totals of the waves before.
__device__ __forceinline__ int tr_block_scan(int v, int32_t* wave_tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) wave_tot[w] = v;
  __syncthreads();
  for (int i = 0; i < w; ++i) v += wave_tot[i];
  return v;
}

// Keys of one expert's selected entries kept in LDS across the radix
// passes when they fit; beyond that each pass recomputes them from global
// memory (same keys, same result).
constexpr int kTrCache = 4096;

// One workgroup per expert e.  Its entries (from every one of the k1 = k + 1
// slots) are indices[bins[e] - cnt, bins[e]); slot j = a % k1 < k is routed,
// j = k the candidate.  active[a] is written for every entry of e, so for
// every entry overall.
__global__ void __launch_bounds__(kTrThreads)
tr_select_kernel(const float* __restrict__ logits, int E, int k1, int M,
                 const int32_t* __restrict__ tpe, const int32_t* __restrict__ bins,
                 const int32_t* __restrict__ indices, int32_t* __restrict__ active) {
  __shared__ int32_t cnt_s[3];
  __shared__ int32_t hist[256];
  __shared__ int32_t wave_tot[kTrThreads / 64];
  __shared__ uint64_t prefix_s;
  __shared__ int32_t rank_s;
  __shared__ uint64_t keys_s[kTrCache];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int cnt = tpe[e];
  const int start = bins[e] - cnt;
  const int k = k1 - 1;
  if (tid < 3) cnt_s[tid] = 0;
  __syncthreads();
  int cr = 0, cc = 0;
  for (int s = tid; s < cnt; s += kTrThreads) {
    const int a = indices[start + s];
    if (a % k1 < k) ++cr; else ++cc;
  }
  atomicAdd(&cnt_s[0], cr);     // integer counts: the order does not matter
  atomicAdd(&cnt_s[1], cc);
  __syncthreads();
  const int routed = cnt_s[0], cands = cnt_s[1];
  const int r = routed % M, up = M - r;
  // 0: keep, 1: take `up` candidates, 2: drop `r` routed
  const int mode = r == 0 ? 0 : (up < r && cands >= up ? 1 : 2);
  uint64_t thr = 0;
  if (mode != 0) {
    // the q-th smallest key (from 0) of the set: the r-th smallest routed
    // key (drop those up to it), or the up-th largest candidate key (take
    // those from it)
    const bool want_cand = mode == 1;
    const int nsel = want_cand ? cands : routed;
    const bool cached = nsel <= kTrCache;
    if (cached) {
      // the selected keys, compacted in any order (a selection does not
      // depend on it)
      for (int s = tid; s < cnt; s += kTrThreads) {
        const int a = indices[start + s];
        if ((a % k1 == k) != want_cand) continue;
        const int64_t t = a / k1;
        keys_s[atomicAdd(&cnt_s[2], 1)] = tr_key(logits[t * E + e], t);
      }
    }
    if (tid == 0) {
      prefix_s = 0;
      rank_s = mode == 2 ? r - 1 : cands - up;
    }
    uint64_t mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      const uint64_t prefix = prefix_s;
      const int q = rank_s;
      if (cached) {
        for (int s = tid; s < nsel; s += kTrThreads) {
          const uint64_t key = keys_s[s];
          if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
      } else {
        for (int s = tid; s < cnt; s += kTrThreads) {
          const int a = indices[start + s];
          if ((a % k1 == k) != want_cand) continue;
          const int64_t t = a / k1;
          const uint64_t key = tr_key(logits[t * E + e], t);
          if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
      }
      __syncthreads();
      // digit d holds rank q when the counts below it sum to at most q and
      // with it to more than q (the last digit takes any remainder)
      const int v = hist[tid];
      const int incl = tr_block_scan(v, wave_tot);
      const int excl = incl - v;
      __syncthreads();                    // every thread has read prefix_s and rank_s
      if (excl <= q && (q < incl || tid == 255)) {
        rank_s = q - excl;
        prefix_s = prefix | ((uint64_t)tid << shift);
      }
      mask |= (uint64_t)255 << shift;
      __syncthreads();
    }
    thr = prefix_s;
  }
  for (int s = tid; s < cnt; s += kTrThreads) {
    const int a = indices[start + s];
    const bool is_cand = a % k1 == k;
    int on;
    if (mode == 0) {
      on = !is_cand;
    } else {
      const int64_t t = a / k1;
      const uint64_t key = tr_key(logits[t * E + e], t);
      on = mode == 1 ? (!is_cand || key >= thr) : (!is_cand && key > thr);
    }
    active[a] = on;
  }
}

// One thread per token: the k + 1 slots and the softmax over the occupied
// ones (zeros for a token left with none).
__global__ void __launch_bounds__(kTrThreads)
tr_output_kernel(const float* __restrict__ logits, int64_t T, int E, int k1,
                 const int32_t* __restrict__ ids1, const int32_t* __restrict__ active,
                 int32_t* __restrict__ out_ids, float* __restrict__ out_w) {
  const int64_t t = (int64_t)blockIdx.x * kTrThreads + threadIdx.x;
  if (t >= T) return;
  const int64_t a0 = t * k1;
  float m = 0.f;
  bool any = false;
  for (int j = 0; j < k1; ++j)
    if (active[a0 + j]) {
      const float z = logits[t * E + ids1[a0 + j]];
      m = any ? fmaxf(m, z) : z;
      any = true;
    }
  float s = 0.f;
  for (int j = 0; j < k1; ++j)
    if (active[a0 + j]) s += __expf(logits[t * E + ids1[a0 + j]] - m);
  for (int j = 0; j < k1; ++j) {
    const bool on = active[a0 + j] != 0;
    out_ids[a0 + j] = on ? ids1[a0 + j] : -1;
    out_w[a0 + j] = on ? __expf(logits[t * E + ids1[a0 + j]] - m) / s : 0.f;
  }
}

namespace {

int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

// The workspace: the top-(k+1) ids and weights, the metadata of the k + 1
// slots with its schedule and scratch, and the per-entry flags.
struct TrLayout {
  int64_t n1, mt;
  int64_t off[16];
  int64_t total;
  TrLayout(int64_t T, int E, int k) {
    n1 = T * (k + 1);
    mt = (n1 + 127 * (E < n1 ? E : n1)) / kBlock;
    const int64_t sizes[] = {
        4 * n1, 4 * n1, 4 * n1,                       // ids1, w1, active
        4 * E, 4 * E, 4 * E,                          // tokens_per_expert, bins, padded_bins
        4 * n1, 4 * n1, 4 * n1,                       // indices, bin_ids, row_of_entry
        4 * mt, 4, 4,                                 // tile_expert, num_padded_rows, status
        4 * mt * kBlock,                              // row_token
        schedule_bytes(mt), meta_workspace_bytes(n1, E)};
    int64_t o = 0;
    for (int i = 0; i < 15; ++i) {
      off[i] = o;
      o += align256(sizes[i]);
    }
    total = o;
  }
};

}  // namespace

int64_t token_round_workspace_bytes(int64_t T, int E, int k) { return TrLayout(T, E, k).total; }

hipError_t launch_token_round(const Shape& s, const float* logits, int M, int32_t* out_ids,
                              float* out_w, void* ws, hipStream_t stream) {
  const TrLayout L(s.T, s.E, s.k);
  char* base = static_cast<char*>(ws);
  const auto i32 = [&](int i) { return reinterpret_cast<int32_t*>(base + L.off[i]); };
  int32_t* ids1 = i32(0);
  float* w1 = reinterpret_cast<float*>(base + L.off[1]);
  int32_t* active = i32(2);
  int32_t* sched = i32(13);
  const MetaPtrs m{i32(3), i32(4), i32(5), i32(6), i32(7), i32(8), i32(9), i32(10), i32(11),
                   sched, sched + L.mt, i32(12)};
  Shape s1 = s;
  s1.k = s.k + 1;
  hipError_t err = launch_router_forward(s1, logits, 0.0f, ids1, w1, nullptr, nullptr, stream);
  if (err != hipSuccess) return err;
  err = launch_metadata(L.n1, s.E, s.k + 1, L.mt, ids1, m, base + L.off[14], stream, nullptr);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(tr_select_kernel, dim3(s.E), dim3(kTrThreads), 0, stream, logits, s.E,
                     s.k + 1, M, m.tokens_per_expert, m.bins, m.indices, active);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(tr_output_kernel, dim3((unsigned)((s.T + kTrThreads - 1) / kTrThreads)),
                     dim3(kTrThreads), 0, stream, logits, s.T, s.E, s.k + 1, ids1, active,
                     out_ids, out_w);
  return hipGetLastError();
}

}  // namespace dmoe
