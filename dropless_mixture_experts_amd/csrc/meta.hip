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
// Three or four launches, stream-ordered, no host synchronisation:
//   meta_hist   one wave per chunk of entries: expert histogram of the chunk
//               (LDS counters) and an invalid-id flag (-1 is no error: an
//               empty slot, routed nowhere).
//   meta_count  kCountExperts experts per workgroup: each expert's total and
//               each chunk's first position among that expert's entries
//               (a scan over the chunks, independent per expert).  Skipped
//               when one workgroup covers every expert with one batch of
//               loads per thread: meta_scan then does these scans itself.
//   meta_scan   one workgroup: bins / padded_bins / P from the totals, the
//               block -> expert table, the pairs of row blocks that the
//               matrix products process together, the status word.
//   meta_place  one wave per chunk: stable rank of every entry among the
//               chunk's entries of the same expert (64-lane ballots on the
//               bits of the id + mbcnt), then writes indices, bin_ids,
//               row_of_entry and the token of the entry's padded row
//               (row_token).  Ties keep ascending entry order, so the
//               result is unique and bit-identical on every run.  Its
//               workgroups also mark the pad rows of row_token -1 and fill
//               the sorted arrays past the routed entries with -1: spread
//               over the grid, not left to meta_scan's single workgroup.
#include <algorithm>
#include <cmath>

#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {

constexpr int kMetaWaves = 4;  // waves (chunks) per workgroup
constexpr int kScanThreads = 1024;
constexpr int kScanBatch = 32;  // chunk counts a scan thread loads at once
constexpr int kCountExperts = 8;  // experts per meta_count workgroup

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
      else if (e != -1)             // -1: an empty slot, routed nowhere
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

// The chunk scan of experts [e0, e0 + ne) by one workgroup of 1024 threads
// (ne <= 256): thread (el, seg) owns expert e0 + el over the seg-th of S =
// 1024 / ne ranges of chunks (threads past S ne only join the barriers).  It
// sums its range, the workgroup scans the S range sums of each expert
// (Hillis-Steele in LDS, `seg_tot` of 1024 entries), and the thread writes
// each chunk's first position among the expert's entries over the chunk's
// count in hist; the last range writes the expert's total to
// tokens_per_expert and, when `tot` is given, to tot[e0 + el] in LDS.
// Ends with a barrier.
__device__ __forceinline__ void scan_chunks(int32_t* __restrict__ hist, int nchunks, int E,
                                            int e0, int ne, int32_t* seg_tot,
                                            int32_t* __restrict__ tokens_per_expert,
                                            int32_t* tot) {
  const int S = kScanThreads / ne;
  const int tid = threadIdx.x;
  const int el = tid % ne, seg = tid / ne;
  const int e = e0 + el;
  const bool mine = seg < S;
  const int seg_len = (nchunks + S - 1) / S;
  const int c0 = min(nchunks, seg * seg_len);
  const int c1 = mine ? min(nchunks, c0 + seg_len) : c0;
  // batches of kScanBatch independent loads: one wait for memory per batch;
  // a range of one batch (the usual case) keeps its counts in registers for
  // the second pass
  int sum = 0;
  int v[kScanBatch];
  for (int cb = c0; cb < c1; cb += kScanBatch) {
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      v[i] = cb + i < c1 ? hist[(int64_t)(cb + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) sum += v[i];
  }
  seg_tot[tid] = sum;
  __syncthreads();
  for (int off = 1; off < S; off <<= 1) {
    const int u = seg >= off ? seg_tot[tid - off * ne] : 0;
    __syncthreads();
    seg_tot[tid] += u;
    __syncthreads();
  }
  if (mine) {
    int run = seg_tot[tid] - sum;            // entries of e in ranges 0..seg-1
    const bool reload = c1 - c0 > kScanBatch;
    for (int cb = c0; cb < c1; cb += kScanBatch) {
      if (reload)
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
    if (seg == S - 1) {
      tokens_per_expert[e] = run;
      if (tot) tot[e] = run;
    }
  }
  __syncthreads();
}

// kCountExperts experts per workgroup; the chunk scans of different experts
// are independent, so E / kCountExperts workgroups share them.
__global__ void __launch_bounds__(kScanThreads)
meta_count_kernel(int32_t* __restrict__ hist, int nchunks, int E,
                  int32_t* __restrict__ tokens_per_expert) {
  __shared__ int32_t seg_tot[kScanThreads];
  const int e0 = blockIdx.x * kCountExperts;
  scan_chunks(hist, nchunks, E, e0, min(kCountExperts, E - e0), seg_tot, tokens_per_expert,
              nullptr);
}

// One workgroup of 1024 threads, from the expert totals of meta_count, or
// (fuse_count) doing meta_count's chunk scans of all E experts itself first.
__global__ void __launch_bounds__(kScanThreads)
meta_scan_kernel(int32_t* __restrict__ hist, const int32_t* __restrict__ err, int nchunks,
                 int E, int max_tiles, int fuse_count,
                 int32_t* __restrict__ tokens_per_expert,
                 int32_t* __restrict__ bins, int32_t* __restrict__ padded_bins,
                 int32_t* __restrict__ tile_expert,
                 int32_t* __restrict__ num_padded_rows,
                 int32_t* __restrict__ status,
                 int32_t* __restrict__ pair_first,
                 int32_t* __restrict__ num_pairs) {
  __shared__ int32_t count_s[kMaxExperts];
  __shared__ int32_t pend_s[kMaxExperts];
  __shared__ int32_t pair_s[kMaxExperts];   // first group of each expert
  __shared__ int32_t P_s, S_s, bad_s;
  __shared__ int32_t seg_tot[kScanThreads];
  const int tid = threadIdx.x;
  if (tid == 0) bad_s = 0;
  if (fuse_count) scan_chunks(hist, nchunks, E, 0, E, seg_tot, tokens_per_expert, count_s);
  else __syncthreads();
  for (int c = tid; c < nchunks; c += kScanThreads)
    if (err[c]) bad_s = 1;                 // every writer stores the same 1
  if (!fuse_count && tid < E) count_s[tid] = tokens_per_expert[tid];
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
        pair_s[ee] = grun;
        crun += c[i];
        prun += pc[i];
        grun += gp[i];
        pend_s[ee] = prun;
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
  if (tid == 0) *status = bad_s ? kErrExpertId : 0;
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
  if (c < nchunks)   // the chunk's first position among expert i's entries, made global
    for (int i = lane; i < E; i += kWave)
      run[w][i] = chunk_start[(int64_t)c * E + i] + (bins[i] - tokens_per_expert[i]);
  // Pad rows hold no token: rows [padded_bins[e] - pc + cnt, padded_bins[e])
  // of expert e, at most 127 (MegaBlocks §2); workgroup b takes experts b,
  // b + gridDim.x, ...
  for (int e = blockIdx.x; e < E; e += gridDim.x) {
    const int cnt = tokens_per_expert[e], pc = round_up_block(cnt);
    for (int i = threadIdx.x; i < pc - cnt; i += blockDim.x)
      row_token[padded_bins[e] - pc + cnt + i] = -1;
  }
  // The sorted arrays list the routed entries only: past their total (less
  // than n when some slots are empty or invalid) they hold -1.
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = bins[E - 1] + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += stride) {
    indices[i] = -1;
    bin_ids[i] = -1;
  }
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

int64_t meta_chunk(int64_t n, int E) {
  // A multiple of 64 entries per wave.  meta_hist and meta_place walk a chunk
  // per wave (n / chunks entries, 64 at a time); each thread of meta_count
  // walks chunks / S chunks of one expert (S = 1024 / kCountExperts threads
  // per expert).  About sqrt(n S / 16) chunks balances the two, counting a
  // 64-entry step of the placement as 4 loads of the count; at most 4096
  // chunks.  E only bounds the workspace (chunks x E counts).
  (void)E;
  const double S = (double)(kScanThreads / kCountExperts);
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
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int blocks = (nchunks + kMetaWaves - 1) / kMetaWaves;
  hipError_t rc = hipSuccess;
  if (ev && ev[0] && (rc = hipEventRecord(ev[0], stream)) != hipSuccess) return rc;
  hipLaunchKernelGGL(meta_hist_kernel, dim3(blocks), dim3(kMetaWaves * kWave), 0,
                     stream, ids, n, chunk, nchunks, E, hist, err);
  if (ev && ev[1] && (rc = hipEventRecord(ev[1], stream)) != hipSuccess) return rc;
  // When one workgroup covers every expert with one batch of loads per
  // thread, the scan kernel takes the chunk scans too: one launch fewer.
  const int segs = kScanThreads / E;
  const bool fuse = (nchunks + segs - 1) / segs <= kScanBatch;
  if (!fuse)
    hipLaunchKernelGGL(meta_count_kernel, dim3((E + kCountExperts - 1) / kCountExperts),
                       dim3(kScanThreads), 0, stream, hist, nchunks, E, m.tokens_per_expert);
  hipLaunchKernelGGL(meta_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream,
                     hist, err, nchunks, E, (int)max_tiles, fuse ? 1 : 0,
                     m.tokens_per_expert, m.bins, m.padded_bins, m.tile_expert,
                     m.num_padded_rows, m.status, m.pair_first, m.num_pairs);
  if (ev && ev[2] && (rc = hipEventRecord(ev[2], stream)) != hipSuccess) return rc;
  hipLaunchKernelGGL(meta_place_kernel, dim3(blocks), dim3(kMetaWaves * kWave), 0,
                     stream, ids, n, chunk, nchunks, E, k, nbits, hist,
                     m.tokens_per_expert, m.bins, m.padded_bins, m.indices,
                     m.bin_ids, m.row_of_entry, m.row_token);
  if (ev && ev[3] && (rc = hipEventRecord(ev[3], stream)) != hipSuccess) return rc;
  return hipGetLastError();
}

}  // namespace dmoe
