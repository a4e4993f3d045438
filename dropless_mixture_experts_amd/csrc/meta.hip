// Routing metadata for the dropless MoE layer (gfx950).
//
// MegaBlocks chapter "02 · dropless MoE 与 block-sparse 重构": §4.1 asks for a
// sort of the (token, expert) entries by expert, a histogram, its inclusive
// cumsum `bins`, the counts rounded up to 128 and their inclusive cumsum
// `padded_bins`; §4.2 places sorted entry s of expert e on padded row
// (s - bins[e-1]) + padded_bins[e-1]; §2/§4.3 give each 128-row block one
// expert.  The Fast-LLM issue "[feat] Support sparse copy for a large number
// of experts" reports a metadata kernel whose on-chip footprint grew with the
// token count and overflowed shared memory at 64 experts; here on-chip memory
// is O(E) (at most ~5 KB at E = 256) whatever T is.
//
// Three launches, stream-ordered, no host synchronisation:
//   meta_hist   one wave per chunk of entries: expert histogram of the chunk
//               (LDS counters) and an invalid-id flag.
//   meta_scan   one workgroup: per-expert totals, bins / padded_bins / P,
//               each chunk's starting sorted position per expert, the
//               block -> expert table, the pairs of row blocks that the
//               matrix products process together, the status word.
//   meta_place  one wave per chunk: stable rank of every entry among the
//               chunk's entries of the same expert (64-lane ballots on the
//               bits of the id + mbcnt), then writes indices, bin_ids,
//               row_of_entry and the token of the entry's padded row
//               (row_token; meta_scan marks the pad rows -1).  Ties keep
//               ascending entry order, so the result is unique and
//               bit-identical on every run.
#include <algorithm>
#include <cmath>

#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {

constexpr int kMetaWaves = 4;  // waves (chunks) per workgroup
constexpr int kScanThreads = 1024;
constexpr int kScanBatch = 8;   // chunk counts a scan thread loads at once

__global__ void __launch_bounds__(kMetaWaves * kWave)
meta_hist_kernel(const int32_t* __restrict__ ids, int64_t n, int64_t chunk,
                 int nchunks, int E, int32_t* __restrict__ hist,
                 int32_t* __restrict__ err) {
  __shared__ int32_t cnt[kMetaWaves][kMaxExperts];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int c = blockIdx.x * kMetaWaves + w;
  for (int i = lane; i < E; i += kWave) cnt[w][i] = 0;
  __syncthreads();
  int bad = 0;
  if (c < nchunks) {
    const int64_t beg = c * chunk;
    const int64_t end = min(n, beg + chunk);
    for (int64_t a = beg + lane; a < end; a += kWave) {
      const int e = ids[a];
      if (e >= 0 && e < E)
        atomicAdd(&cnt[w][e], 1);   // integer count: order does not matter
      else
        bad = 1;
    }
  }
  __syncthreads();
  if (c < nchunks) {
    for (int i = lane; i < E; i += kWave) hist[(int64_t)c * E + i] = cnt[w][i];
    const unsigned long long any_bad = __ballot(bad);
    if (lane == 0) err[c] = any_bad ? 1 : 0;
  }
}

// One workgroup of 1024 threads.  Thread (e, seg) owns expert e over the
// seg-th range of chunks; Ecap (a power of two >= E) experts x S segments.
__global__ void __launch_bounds__(kScanThreads)
meta_scan_kernel(int32_t* __restrict__ hist, const int32_t* __restrict__ err,
                 int nchunks, int E, int Ecap, int max_tiles,
                 int32_t* __restrict__ tokens_per_expert,
                 int32_t* __restrict__ bins, int32_t* __restrict__ padded_bins,
                 int32_t* __restrict__ tile_expert,
                 int32_t* __restrict__ num_padded_rows,
                 int32_t* __restrict__ status,
                 int32_t* __restrict__ pair_first,
                 int32_t* __restrict__ num_pairs,
                 int32_t* __restrict__ row_token,
                 int32_t* __restrict__ xcd_first) {
  __shared__ int32_t seg_tot[kScanThreads];
  __shared__ int32_t nxt_s[kMaxExperts + 1];
  __shared__ int32_t maxb_s, feas_s;
  __shared__ int32_t count_s[kMaxExperts];
  __shared__ int32_t start_s[kMaxExperts];
  __shared__ int32_t pend_s[kMaxExperts];
  __shared__ int32_t pair_s[kMaxExperts];   // first group of each expert
  __shared__ int32_t P_s, S_s, bad_s;
  const int tid = threadIdx.x;
  const int S = kScanThreads / Ecap;
  const int e = tid % Ecap, seg = tid / Ecap;
  const int seg_len = (nchunks + S - 1) / S;
  const int c0 = min(nchunks, seg * seg_len);
  const int c1 = min(nchunks, c0 + seg_len);

  // Batches of kScanBatch independent loads, so a thread waits for memory
  // once per batch rather than once per chunk.
  int sum = 0;
  if (e < E)
    for (int cb = c0; cb < c1; cb += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        v[i] = cb + i < c1 ? hist[(int64_t)(cb + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) sum += v[i];
    }
  seg_tot[tid] = sum;
  if (tid == 0) bad_s = 0;
  __syncthreads();
  for (int c = tid; c < nchunks; c += kScanThreads)
    if (err[c]) bad_s = 1;                 // every writer stores the same 1
  if (tid < E) {
    int tot = 0;
    for (int s = 0; s < S; ++s) tot += seg_tot[s * Ecap + tid];
    count_s[tid] = tot;
  }
  __syncthreads();

  // Inclusive scans over experts of the counts and the rounded-up counts:
  // wave 0, four consecutive experts per lane, then a 64-lane shuffle scan.
  // The same scan also numbers the groups of (at most) two row blocks of one
  // expert that the matrix products work on: ceil(blocks / 2) per expert.
  if (tid < kWave) {
    int c[4], pc[4], gp[4], cs = 0, ps = 0, gs = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = tid * 4 + i;
      c[i] = ee < E ? count_s[ee] : 0;
      pc[i] = round_up_block(c[i]);
      gp[i] = (pc[i] / kBlock + 1) / 2;
      cs += c[i];
      ps += pc[i];
      gs += gp[i];
    }
    int ci = cs, pi = ps, gi = gs;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int cu = __shfl_up(ci, off, kWave);
      const int pu = __shfl_up(pi, off, kWave);
      const int gu = __shfl_up(gi, off, kWave);
      if (tid >= off) { ci += cu; pi += pu; gi += gu; }
    }
    int crun = ci - cs, prun = pi - ps, grun = gi - gs;   // exclusive starts
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = tid * 4 + i;
      if (ee < E) {
        start_s[ee] = crun;
        pair_s[ee] = grun;
        crun += c[i];
        prun += pc[i];
        grun += gp[i];
        pend_s[ee] = prun;
        tokens_per_expert[ee] = c[i];
        bins[ee] = crun;
        padded_bins[ee] = prun;
      }
    }
    if (tid == kWave - 1) {
      P_s = pi;
      S_s = gi;
      *num_padded_rows = pi;
      *num_pairs = gi;
    }
  }
  __syncthreads();

  // Each chunk's first sorted position per expert (exclusive, global).
  if (e < E) {
    int run = start_s[e];
    for (int s = 0; s < seg; ++s) run += seg_tot[s * Ecap + e];
    for (int cb = c0; cb < c1; cb += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        v[i] = cb + i < c1 ? hist[(int64_t)(cb + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (cb + i < c1) {
          hist[(int64_t)(cb + i) * E + e] = run;
          run += v[i];
        }
    }
  }
  // 128-row block r -> its expert: the first e with padded_bins[e] > 128 r.
  const int P = P_s;
  for (int r = tid; r < max_tiles; r += kScanThreads) {
    const int row = r * kBlock;
    int owner = -1;
    if (row < P) {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (pend_s[mid] > row) hi = mid; else lo = mid + 1;
      }
      owner = lo;
    }
    tile_expert[r] = owner;
  }
  // Groups of expert e start at block (pend - pc) / 128 and step by two.
  if (tid < E) {
    const int pc = round_up_block(count_s[tid]);
    const int t0 = (pend_s[tid] - pc) / kBlock;
    const int ng = (pc / kBlock + 1) / 2;
    const int g0 = pair_s[tid];
    for (int q = 0; q < ng; ++q) pair_first[g0 + q] = t0 + 2 * q;
  }
  for (int r = S_s + tid; r < max_tiles; r += kScanThreads) pair_first[r] = -1;
  // Pad rows hold no token: rows [pend - pc + c, pend) of each expert (at
  // most 127 per expert, MegaBlocks §2).
  for (int q = tid; q < E * (kBlock - 1); q += kScanThreads) {
    const int ee = q / (kBlock - 1), i = q - ee * (kBlock - 1);
    const int c = count_s[ee], pc = round_up_block(c);
    if (i < pc - c) row_token[pend_s[ee] - pc + c + i] = -1;
  }
  if (tid == 0) *status = bad_s ? kErrExpertId : 0;

  // The experts whose weight-gradient tiles each XCD computes: 8 contiguous
  // ranges with the least possible largest cost.  A tile of those products
  // has K = its expert's padded rows plus an epilogue of about two K steps
  // of 64, so an expert costs its 128-row blocks + 1 (an empty expert's
  // tiles still write zeros).  Balancing rows alone measured worse than
  // balancing this cost under skewed routing.  With total cost W and the
  // largest expert cost M, the least maximum lies in [max(ceil(W / 8), M),
  // ceil(W / 8) + M]: at the upper cap a greedy range that stops before E
  // costs more than cap - M = ceil(W / 8), so 8 of them reach E.  Binary
  // search on the cap; a cap is feasible when 8 greedy ranges reach E.
  // nxt_s[s] is the greedy end of a range starting at expert s: the largest
  // b with cost(s, b) <= cap, one binary search per thread.
  if (tid == 0) maxb_s = 0;
  __syncthreads();
  if (tid < E) atomicMax(&maxb_s, round_up_block(count_s[tid]) / kBlock + 1);
  __syncthreads();
  const auto pre = [&](int b) { return b == 0 ? 0 : pend_s[b - 1] / kBlock + b; };
  const int eighth = (P / kBlock + E + 7) / 8;
  const auto greedy_ends = [&](int cap) {
    for (int s0 = tid; s0 <= E; s0 += kScanThreads) {
      const int lim = pre(s0) + cap;
      int a = s0, z = E;
      while (a < z) {
        const int mid = (a + z + 1) >> 1;
        if (pre(mid) <= lim) a = mid; else z = mid - 1;
      }
      nxt_s[s0] = a;
    }
  };
  int lo = max(eighth, maxb_s), hi = eighth + maxb_s;
  while (lo < hi) {                      // lo, hi are the same in every thread
    const int cap = (lo + hi) >> 1;
    greedy_ends(cap);
    __syncthreads();
    if (tid == 0) {
      int b = 0;
      for (int x = 0; x < 8 && b < E; ++x) b = nxt_s[b];
      feas_s = b >= E;
    }
    __syncthreads();
    if (feas_s) hi = cap; else lo = cap + 1;
    __syncthreads();                     // nxt_s and feas_s are rewritten
  }
  greedy_ends(lo);
  __syncthreads();
  if (tid == 0) {
    int b = 0;
    xcd_first[0] = 0;
    for (int x = 1; x < 8; ++x) {
      b = b < E ? nxt_s[b] : E;
      xcd_first[x] = b;
    }
    xcd_first[8] = E;
  }
}

__global__ void __launch_bounds__(kMetaWaves * kWave)
meta_place_kernel(const int32_t* __restrict__ ids, int64_t n, int64_t chunk,
                  int nchunks, int E, int k, int nbits,
                  const int32_t* __restrict__ chunk_start,
                  const int32_t* __restrict__ tokens_per_expert,
                  const int32_t* __restrict__ bins,
                  const int32_t* __restrict__ padded_bins,
                  int32_t* __restrict__ indices, int32_t* __restrict__ bin_ids,
                  int32_t* __restrict__ row_of_entry, int32_t* __restrict__ row_token) {
  __shared__ int32_t run[kMetaWaves][kMaxExperts];
  __shared__ int32_t shift_s[kMaxExperts];   // padded start - sorted start
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int c = blockIdx.x * kMetaWaves + w;
  for (int i = threadIdx.x; i < E; i += blockDim.x) {
    const int cnt = tokens_per_expert[i];
    shift_s[i] = (padded_bins[i] - round_up_block(cnt)) - (bins[i] - cnt);
  }
  if (c < nchunks)
    for (int i = lane; i < E; i += kWave) run[w][i] = chunk_start[(int64_t)c * E + i];
  __syncthreads();
  if (c >= nchunks) return;

  const int64_t beg = c * chunk;
  const int64_t end = min(n, beg + chunk);
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int64_t base = beg; base < end; base += kWave) {
    const int64_t a = base + lane;
    const bool in = a < end;
    const int e = in ? ids[a] : -1;
    const bool ok = in && e >= 0 && e < E;
    // Lanes holding the same expert id: intersect ballots over its bits.
    unsigned long long same = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const unsigned long long on = __ballot(bit);
      same &= ((e >> b) & 1) ? on : ~on;
    }
    if (ok) {
      const int rank = __popcll(same & lt);
      const int pos = run[w][e] + rank;
      indices[pos] = (int32_t)a;
      bin_ids[pos] = e;
      row_of_entry[a] = pos + shift_s[e];
      row_token[pos + shift_s[e]] = (int32_t)(a / k);
      if ((same & lt) == 0ull) run[w][e] = pos + __popcll(same);  // group leader
    } else if (in) {
      row_of_entry[a] = -1;
    }
  }
}

static int expert_cap(int E) {
  int Ecap = 1;
  while (Ecap < E) Ecap <<= 1;
  return Ecap;
}

int64_t meta_chunk(int64_t n, int E) {
  // A multiple of 64 entries per wave.  meta_hist and meta_place walk a chunk
  // per wave (n / chunks entries, 64 at a time); each thread of meta_scan
  // walks chunks / S chunks of one expert (S = 1024 / Ecap threads per
  // expert).  About sqrt(n S / 16) chunks balances the two, counting a
  // 64-entry step of the placement as 4 scan loads; at most 4096 chunks.
  const double S = (double)(kScanThreads / expert_cap(E));
  const int64_t target =
      std::max<int64_t>(1, std::min<int64_t>(4096, (int64_t)std::sqrt((double)n * S / 16.0)));
  int64_t c = (n + target - 1) / target;
  c = ((c + kWave - 1) / kWave) * kWave;
  c = std::max<int64_t>(c, kWave);
  while ((n + c - 1) / c > 4096) c += kWave;
  return c;
}

int meta_nchunks(int64_t n, int E) {
  return (int)((n + meta_chunk(n, E) - 1) / meta_chunk(n, E));
}

int64_t meta_workspace_bytes(int64_t n, int E) {
  const int64_t nc = meta_nchunks(n, E);
  return ((nc * E + nc) * (int64_t)sizeof(int32_t) + 255) / 256 * 256;
}

hipError_t launch_metadata(int64_t n, int E, int k, int64_t max_tiles,
                           const int32_t* ids, const MetaPtrs& m, void* ws,
                           hipStream_t stream, hipEvent_t* ev) {
  const int64_t chunk = meta_chunk(n, E);
  const int nchunks = meta_nchunks(n, E);
  int32_t* hist = static_cast<int32_t*>(ws);
  int32_t* err = hist + (int64_t)nchunks * E;
  int Ecap = 1;
  while (Ecap < E) Ecap <<= 1;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int blocks = (nchunks + kMetaWaves - 1) / kMetaWaves;
  hipError_t rc = hipSuccess;
  if (ev && ev[0] && (rc = hipEventRecord(ev[0], stream)) != hipSuccess) return rc;
  hipLaunchKernelGGL(meta_hist_kernel, dim3(blocks), dim3(kMetaWaves * kWave), 0,
                     stream, ids, n, chunk, nchunks, E, hist, err);
  if (ev && ev[1] && (rc = hipEventRecord(ev[1], stream)) != hipSuccess) return rc;
  hipLaunchKernelGGL(meta_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream,
                     hist, err, nchunks, E, Ecap, (int)max_tiles,
                     m.tokens_per_expert, m.bins, m.padded_bins, m.tile_expert,
                     m.num_padded_rows, m.status, m.pair_first, m.num_pairs, m.row_token,
                     m.xcd_first);
  if (ev && ev[2] && (rc = hipEventRecord(ev[2], stream)) != hipSuccess) return rc;
  hipLaunchKernelGGL(meta_place_kernel, dim3(blocks), dim3(kMetaWaves * kWave), 0,
                     stream, ids, n, chunk, nchunks, E, k, nbits, hist,
                     m.tokens_per_expert, m.bins, m.padded_bins, m.indices,
                     m.bin_ids, m.row_of_entry, m.row_token);
  if (ev && ev[3] && (rc = hipEventRecord(ev[3], stream)) != hipSuccess) return rc;
  return hipGetLastError();
}

}  // namespace dmoe
