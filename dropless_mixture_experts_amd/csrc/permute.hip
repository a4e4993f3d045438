// padded_gather / padded_scatter and their backward (gfx950).
//
// MegaBlocks chapter "02 · dropless MoE 与 block-sparse 重构" §4.2: one index
// rule serves both directions.  Gather copies token row a / k (a = t*k + j)
// to the entry's padded row; scatter reads the entry's padded row back,
// multiplies by the routing weight and sums the k slots of a token.  The
// scatter's backward is a gather of dy times the routing weight plus the
// routing-weight gradient; the gather's backward is a scatter with unit
// weights.  §5: pad rows hold zeros and the scatter reads only real rows.
//
// These kernels move bytes and do almost no arithmetic, so they are bound by
// HBM.  One wave owns one token: it reads the token's row once and reaches
// its k padded rows through row_of_entry; extra waves zero the pad rows.
// Each lane moves 16 bytes per access, so a 4 KB bf16 row (H = 2048) is four
// fully coalesced 1 KB wave transactions.  No atomics: each output row is
// written by exactly one wave, and the top-k sum runs in fp32 in slot order
// with one final rounding.  Every store is non-temporal: each output is read
// by the next kernel, not by this one, and without the hint the lines this
// kernel leaves dirty in L2 are written back under the next kernel's loads
// (measured: the scatter backward's output then cost the down-projection
// dgrad 44 us on the 256-expert layer).
#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {

constexpr int kRowsPerBlock = 4;   // one wave per row (or token)
constexpr int kUnroll = 4;         // 16-byte accesses in flight per lane
constexpr int kPadWaves = kBlock - 1;   // an expert has at most 127 pad rows

// Wave index of this lane's wave, the same in every lane.
__device__ __forceinline__ int64_t wave_index() {
  return (int64_t)blockIdx.x * kRowsPerBlock +
         __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

// Pad row i of expert e for the wave q = e * 127 + i after the token waves, or
// -1 if expert e has at most i pad rows (MegaBlocks §2: rows
// [start_e + c_e, start_e + round_up(c_e)) of expert e are padding).
__device__ __forceinline__ int64_t pad_row(int64_t q, const int32_t* tpe,
                                           const int32_t* padded_bins) {
  const int e = (int)(q / kPadWaves), i = (int)(q - (int64_t)e * kPadWaves);
  const int c = tpe[e], pc = round_up_block(c);
  return i < pc - c ? (int64_t)padded_bins[e] - pc + c + i : -1;
}

__device__ __forceinline__ void zero_row(char* dst, int64_t vecs, int lane) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t v = lane; v < vecs; v += kWave) st16_nt(dst + v * 16, z);
}

// Waves [0, ntok): token t copies its row of x to the padded rows of its k
// entries (the row is read once, written k times).  Waves [ntok, ntok + 127 E):
// zero the pad rows.
template <typename T>
__global__ void __launch_bounds__(kRowsPerBlock * kWave)
padded_gather_kernel(const T* __restrict__ x, int64_t ntok, int64_t H, int k, int E,
                     const int32_t* __restrict__ row_of_entry,
                     const int32_t* __restrict__ tpe,
                     const int32_t* __restrict__ padded_bins, T* __restrict__ x_perm) {
  const int lane = threadIdx.x % kWave;
  const int64_t q = wave_index();
  const int64_t vecs = H * (int64_t)sizeof(T) / 16;
  const int64_t rowb = H * (int64_t)sizeof(T);
  char* out = reinterpret_cast<char*>(x_perm);
  if (q >= ntok) {
    if (q - ntok >= (int64_t)E * kPadWaves) return;
    const int64_t p = pad_row(q - ntok, tpe, padded_bins);
    if (p >= 0) zero_row(out + p * rowb, vecs, lane);
    return;
  }
  const char* src = reinterpret_cast<const char*>(x) + q * rowb;
  const int32_t* rows = row_of_entry + q * k;
  for (int64_t v0 = lane; v0 < vecs; v0 += kWave * kUnroll) {
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + u * kWave;
      if (v < vecs) r[u] = ld16_nt(src + v * 16);
    }
    for (int j = 0; j < k; ++j) {
      const int row = rows[j];
      if (row < 0) continue;     // an empty slot (or an invalid id): no row
      char* dst = out + (int64_t)row * rowb;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t v = v0 + u * kWave;
        if (v < vecs) st16_nt(dst + v * 16, r[u]);
      }
    }
  }
}

// out[t] = sum_j w[t,j] * src_perm[row_of_entry[t*k+j]]  (w = 1 if null).
// Four 16-byte columns per lane and pass (a whole 4 KB bf16 row per wave) and
// rows in groups of four, so 16 loads are in flight and each row is read in
// one pass rather than in halves.
template <typename T>
__global__ void __launch_bounds__(kRowsPerBlock * kWave)
padded_scatter_kernel(const T* __restrict__ src_perm,
                      const float* __restrict__ weights,
                      const int32_t* __restrict__ row_of_entry, int64_t ntok,
                      int64_t H, int k, T* __restrict__ out) {
  using V = Vec16<T>;
  const int lane = threadIdx.x % kWave;
  const int64_t t = wave_index();
  if (t >= ntok) return;
  const int64_t vecs = H * (int64_t)sizeof(T) / 16;
  const int64_t rowb = H * (int64_t)sizeof(T);
  const char* src = reinterpret_cast<const char*>(src_perm);
  const int32_t* rows = row_of_entry + t * k;
  const float* wts = weights ? weights + t * k : nullptr;
  char* dst = reinterpret_cast<char*>(out + t * H);
  for (int64_t v0 = lane; v0 < vecs; v0 += 4 * kWave) {
    bool has[4];
    float acc[4][V::N];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      has[c] = v0 + c * kWave < vecs;
#pragma unroll
      for (int i = 0; i < V::N; ++i) acc[c][i] = 0.f;
    }
    for (int j0 = 0; j0 < k; j0 += 4) {
      u32x4 d[4][4];
      float wj[4];
      bool live[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u;
        const int r = j < k ? rows[j] : -1;
        live[u] = r >= 0;
        wj[u] = wts && live[u] ? wts[j] : 1.f;
        const char* row = src + (int64_t)(live[u] ? r : 0) * rowb;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          d[u][c] = live[u] && has[c] ? ld16_nt(row + (v0 + c * kWave) * 16) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (live[u]) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            float f[V::N];
            V::unpack(d[u][c], f);
#pragma unroll
            for (int i = 0; i < V::N; ++i) acc[c][i] = __builtin_fmaf(wj[u], f[i], acc[c][i]);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (has[c]) st16_nt(dst + (v0 + c * kWave) * 16, V::pack(acc[c]));
  }
}

// The scatter's backward, in two launches that share no output: one writes,
// one reads.  Measured against a single kernel doing both per token (56.4
// against 60.2 us on fine_e64, 171 against 181 us on sparse_e256): dy is read
// twice, but each stream runs in one direction.
//
// scatter_backward_rows: waves [0, ntok): token t reads dy[t] once and writes
// dy_perm[p] = w[a] * dy[t] to the padded row p of each entry a = t*k + j;
// waves [ntok, ntok + 127 E): zero the pad rows of dy_perm.
template <typename T>
__global__ void __launch_bounds__(kRowsPerBlock * kWave)
scatter_backward_rows_kernel(const T* __restrict__ dy, const float* __restrict__ weights,
                             int64_t ntok, int64_t H, int k, int E,
                             const int32_t* __restrict__ row_of_entry,
                             const int32_t* __restrict__ tpe,
                             const int32_t* __restrict__ padded_bins,
                             T* __restrict__ dy_perm) {
  using V = Vec16<T>;
  const int lane = threadIdx.x % kWave;
  const int64_t q = wave_index();
  const int64_t vecs = H * (int64_t)sizeof(T) / 16;
  const int64_t rowb = H * (int64_t)sizeof(T);
  char* out = reinterpret_cast<char*>(dy_perm);
  if (q >= ntok) {
    if (q - ntok >= (int64_t)E * kPadWaves) return;
    const int64_t p = pad_row(q - ntok, tpe, padded_bins);
    if (p >= 0) zero_row(out + p * rowb, vecs, lane);
    return;
  }
  const char* src = reinterpret_cast<const char*>(dy) + q * rowb;
  const int32_t* rows = row_of_entry + q * k;
  for (int64_t v0 = lane; v0 < vecs; v0 += kWave * kUnroll) {
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + u * kWave;
      if (v < vecs) r[u] = ld16_nt(src + v * 16);
    }
    for (int j = 0; j < k; ++j) {
      const int row = rows[j];
      if (row < 0) continue;     // an empty slot: no row
      const float wt = weights[q * k + j];
      char* dst = out + (int64_t)row * rowb;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t v = v0 + u * kWave;
        if (v < vecs) {
          float f[V::N];
          V::unpack(r[u], f);
#pragma unroll
          for (int i = 0; i < V::N; ++i) f[i] = wt * f[i];
          st16_nt(dst + v * 16, V::pack(f));
        }
      }
    }
  }
}

// scatter_backward_dot: waves [0, ntok): d_weights[a] = <dy[t], y_perm[p]>
// for each entry a = t*k + j on padded row p (0 for an empty slot).  The
// entries go four at a time; per pass a lane holds four 16-byte columns of
// dy[t] and of the four y_perm rows (20 loads in flight).  Each dot
// accumulates a lane's columns in ascending order and is summed over the wave
// in a fixed order (run-to-run identical).
template <typename T>
__global__ void __launch_bounds__(kRowsPerBlock * kWave)
scatter_backward_dot_kernel(const T* __restrict__ dy, const T* __restrict__ y_perm,
                            int64_t ntok, int64_t H, int k,
                            const int32_t* __restrict__ row_of_entry,
                            float* __restrict__ d_weights) {
  using V = Vec16<T>;
  const int lane = threadIdx.x % kWave;
  const int64_t t = wave_index();
  if (t >= ntok) return;
  const int64_t vecs = H * (int64_t)sizeof(T) / 16;
  const int64_t rowb = H * (int64_t)sizeof(T);
  const char* g = reinterpret_cast<const char*>(dy) + t * rowb;
  const char* yp = reinterpret_cast<const char*>(y_perm);
  const int32_t* rows = row_of_entry + t * k;
  for (int j0 = 0; j0 < k; j0 += 4) {
    int row[4];
    float dot[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u;
      row[u] = j < k ? rows[j] : -1;     // -1: past k, or an empty slot
      dot[u] = 0.f;
    }
    for (int64_t v0 = lane; v0 < vecs; v0 += 4 * kWave) {
      u32x4 gd[4], yd[4][4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        gd[c] = v0 + c * kWave < vecs ? ld16(g + (v0 + c * kWave) * 16) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const char* src = yp + (int64_t)(row[u] >= 0 ? row[u] : 0) * rowb;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          yd[u][c] = row[u] >= 0 && v0 + c * kWave < vecs ? ld16_nt(src + (v0 + c * kWave) * 16)
                                                          : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (v0 + c * kWave >= vecs) break;
        float gf[V::N];
        V::unpack(gd[c], gf);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (row[u] < 0) continue;
          float yf[V::N];
          V::unpack(yd[u][c], yf);
#pragma unroll
          for (int i = 0; i < V::N; ++i) dot[u] = __builtin_fmaf(gf[i], yf[i], dot[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float d = wave_sum(dot[u]);
      if (lane == 0 && j0 + u < k) d_weights[t * k + j0 + u] = row[u] >= 0 ? d : 0.f;
    }
  }
}

// Slot order <-> padded order, one row per entry, no weights and no sum
// (the map / reduce pair of mixture of attention heads: the
// "yikangshen/megablocks" README feeds attention with k queries per token
// and reduces the k attention outputs).  Rows are W elements wide.
//
// slot_unpermute: waves [0, nent): out[a] = src_perm[row_of_entry[a]], zeros
// for an empty slot (row -1).
template <typename T>
__global__ void __launch_bounds__(kRowsPerBlock * kWave)
slot_unpermute_kernel(const T* __restrict__ src_perm, int64_t nent, int64_t W,
                      const int32_t* __restrict__ row_of_entry, T* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int64_t a = wave_index();
  if (a >= nent) return;
  const int64_t vecs = W * (int64_t)sizeof(T) / 16;
  const int64_t rowb = W * (int64_t)sizeof(T);
  char* dst = reinterpret_cast<char*>(out) + a * rowb;
  const int row = row_of_entry[a];
  if (row < 0) {
    zero_row(dst, vecs, lane);
    return;
  }
  const char* src = reinterpret_cast<const char*>(src_perm) + (int64_t)row * rowb;
  for (int64_t v0 = lane; v0 < vecs; v0 += kWave * kUnroll) {
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + u * kWave;
      if (v < vecs) r[u] = ld16_nt(src + v * 16);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + u * kWave;
      if (v < vecs) st16_nt(dst + v * 16, r[u]);
    }
  }
}

// slot_permute: waves [0, nent): dst_perm[row_of_entry[a]] = src[a] (nothing
// for an empty slot); waves [nent, nent + 127 E): zero the pad rows.
template <typename T>
__global__ void __launch_bounds__(kRowsPerBlock * kWave)
slot_permute_kernel(const T* __restrict__ src, int64_t nent, int64_t W, int E,
                    const int32_t* __restrict__ row_of_entry,
                    const int32_t* __restrict__ tpe,
                    const int32_t* __restrict__ padded_bins, T* __restrict__ dst_perm) {
  const int lane = threadIdx.x % kWave;
  const int64_t a = wave_index();
  const int64_t vecs = W * (int64_t)sizeof(T) / 16;
  const int64_t rowb = W * (int64_t)sizeof(T);
  char* out = reinterpret_cast<char*>(dst_perm);
  if (a >= nent) {
    if (a - nent >= (int64_t)E * kPadWaves) return;
    const int64_t p = pad_row(a - nent, tpe, padded_bins);
    if (p >= 0) zero_row(out + p * rowb, vecs, lane);
    return;
  }
  const int row = row_of_entry[a];
  if (row < 0) return;
  const char* s = reinterpret_cast<const char*>(src) + a * rowb;
  char* d = out + (int64_t)row * rowb;
  for (int64_t v0 = lane; v0 < vecs; v0 += kWave * kUnroll) {
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + u * kWave;
      if (v < vecs) r[u] = ld16_nt(s + v * 16);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + u * kWave;
      if (v < vecs) st16_nt(d + v * 16, r[u]);
    }
  }
}

static unsigned blocks_for(int64_t rows) {
  return (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
}

// Waves for the tokens plus 127 per expert for the pad rows.
static unsigned permute_blocks(const Shape& s) {
  return blocks_for(s.T + (int64_t)s.E * kPadWaves);
}

hipError_t launch_padded_gather(const Shape& s, const void* x, const MetaPtrs& m,
                                void* x_perm, hipStream_t stream) {
  const dim3 grid(permute_blocks(s)), block(kRowsPerBlock * kWave);
  if (s.bf16)
    hipLaunchKernelGGL(padded_gather_kernel<bf16>, grid, block, 0, stream,
                       static_cast<const bf16*>(x), s.T, s.H, s.k, s.E, m.row_of_entry,
                       m.tokens_per_expert, m.padded_bins, static_cast<bf16*>(x_perm));
  else
    hipLaunchKernelGGL(padded_gather_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(x), s.T, s.H, s.k, s.E, m.row_of_entry,
                       m.tokens_per_expert, m.padded_bins, static_cast<float*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_padded_scatter(const Shape& s, const void* src_perm,
                                 const float* weights, const MetaPtrs& m,
                                 void* out, hipStream_t stream) {
  const dim3 grid(blocks_for(s.T)), block(kRowsPerBlock * kWave);
  if (s.bf16)
    hipLaunchKernelGGL(padded_scatter_kernel<bf16>, grid, block, 0, stream,
                       static_cast<const bf16*>(src_perm), weights,
                       m.row_of_entry, s.T, s.H, s.k, static_cast<bf16*>(out));
  else
    hipLaunchKernelGGL(padded_scatter_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(src_perm), weights,
                       m.row_of_entry, s.T, s.H, s.k, static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_scatter_backward(const Shape& s, const void* dy,
                                   const void* y_perm, const float* weights,
                                   const MetaPtrs& m, void* dy_perm,
                                   float* d_weights, hipStream_t stream) {
  const dim3 block(kRowsPerBlock * kWave);
  const dim3 rows_grid(permute_blocks(s)), dot_grid(blocks_for(s.T));
  if (s.bf16) {
    hipLaunchKernelGGL(scatter_backward_rows_kernel<bf16>, rows_grid, block, 0, stream,
                       static_cast<const bf16*>(dy), weights, s.T, s.H, s.k, s.E,
                       m.row_of_entry, m.tokens_per_expert, m.padded_bins,
                       static_cast<bf16*>(dy_perm));
    hipLaunchKernelGGL(scatter_backward_dot_kernel<bf16>, dot_grid, block, 0, stream,
                       static_cast<const bf16*>(dy), static_cast<const bf16*>(y_perm), s.T,
                       s.H, s.k, m.row_of_entry, d_weights);
  } else {
    hipLaunchKernelGGL(scatter_backward_rows_kernel<float>, rows_grid, block, 0, stream,
                       static_cast<const float*>(dy), weights, s.T, s.H, s.k, s.E,
                       m.row_of_entry, m.tokens_per_expert, m.padded_bins,
                       static_cast<float*>(dy_perm));
    hipLaunchKernelGGL(scatter_backward_dot_kernel<float>, dot_grid, block, 0, stream,
                       static_cast<const float*>(dy), static_cast<const float*>(y_perm), s.T,
                       s.H, s.k, m.row_of_entry, d_weights);
  }
  return hipGetLastError();
}

hipError_t launch_slot_unpermute(const Shape& s, int64_t W, const void* src_perm,
                                 const MetaPtrs& m, void* out, hipStream_t stream) {
  const int64_t n = s.T * s.k;
  const dim3 grid(blocks_for(n)), block(kRowsPerBlock * kWave);
  if (s.bf16)
    hipLaunchKernelGGL(slot_unpermute_kernel<bf16>, grid, block, 0, stream,
                       static_cast<const bf16*>(src_perm), n, W, m.row_of_entry,
                       static_cast<bf16*>(out));
  else
    hipLaunchKernelGGL(slot_unpermute_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(src_perm), n, W, m.row_of_entry,
                       static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_slot_permute(const Shape& s, int64_t W, const void* src, const MetaPtrs& m,
                               void* dst_perm, hipStream_t stream) {
  const int64_t n = s.T * s.k;
  const dim3 grid(blocks_for(n + (int64_t)s.E * kPadWaves)), block(kRowsPerBlock * kWave);
  if (s.bf16)
    hipLaunchKernelGGL(slot_permute_kernel<bf16>, grid, block, 0, stream,
                       static_cast<const bf16*>(src), n, W, s.E, m.row_of_entry,
                       m.tokens_per_expert, m.padded_bins, static_cast<bf16*>(dst_perm));
  else
    hipLaunchKernelGGL(slot_permute_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(src), n, W, s.E, m.row_of_entry,
                       m.tokens_per_expert, m.padded_bins, static_cast<float*>(dst_perm));
  return hipGetLastError();
}

}  // namespace dmoe
