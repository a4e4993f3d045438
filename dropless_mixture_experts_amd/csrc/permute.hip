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
// HBM.  One wave owns one row; each lane moves 16 bytes per access, so a
// 4 KB bf16 row (H = 2048) is four fully coalesced 1 KB wave transactions.
// No atomics: each output row is written by exactly one wave, and the top-k
// sum runs in fp32 in slot order with one final rounding.
#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {

constexpr int kRowsPerBlock = 4;   // one wave per row
constexpr int kUnroll = 4;         // 16-byte accesses in flight per lane

// Real row p of expert e holds sorted entry s = bins[e] - count[e] + offset;
// pad rows get -1.
__device__ __forceinline__ int source_entry(int64_t p, const int32_t* tile_expert,
                                            const int32_t* tpe, const int32_t* bins,
                                            const int32_t* padded_bins,
                                            const int32_t* indices) {
  const int e = tile_expert[p / kBlock];
  const int cnt = tpe[e];
  const int off = (int)(p - (padded_bins[e] - round_up_block(cnt)));
  return off < cnt ? indices[bins[e] - cnt + off] : -1;
}

template <typename T>
__global__ void __launch_bounds__(kRowsPerBlock * kWave)
padded_gather_kernel(const T* __restrict__ x, int64_t H, int k,
                     const int32_t* __restrict__ tile_expert,
                     const int32_t* __restrict__ tpe,
                     const int32_t* __restrict__ bins,
                     const int32_t* __restrict__ padded_bins,
                     const int32_t* __restrict__ indices,
                     const int32_t* __restrict__ num_padded_rows,
                     T* __restrict__ x_perm) {
  const int lane = threadIdx.x % kWave;
  const int64_t p = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (p >= *num_padded_rows) return;
  const int a = source_entry(p, tile_expert, tpe, bins, padded_bins, indices);
  const int64_t vecs = H * (int64_t)sizeof(T) / 16;
  char* dst = reinterpret_cast<char*>(x_perm + p * H);
  if (a >= 0) {
    const char* src = reinterpret_cast<const char*>(x + (int64_t)(a / k) * H);
    for (int64_t v0 = lane; v0 < vecs; v0 += kWave * kUnroll) {
      u32x4 r[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t v = v0 + u * kWave;
        if (v < vecs) r[u] = ld16(src + v * 16);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t v = v0 + u * kWave;
        if (v < vecs) st16(dst + v * 16, r[u]);
      }
    }
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t v = lane; v < vecs; v += kWave) st16(dst + v * 16, z);
  }
}

// out[t] = sum_j w[t,j] * src_perm[row_of_entry[t*k+j]]  (w = 1 if null).
template <typename T>
__global__ void __launch_bounds__(kRowsPerBlock * kWave)
padded_scatter_kernel(const T* __restrict__ src_perm,
                      const float* __restrict__ weights,
                      const int32_t* __restrict__ row_of_entry, int64_t ntok,
                      int64_t H, int k, T* __restrict__ out) {
  using V = Vec16<T>;
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (t >= ntok) return;
  const int64_t vecs = H * (int64_t)sizeof(T) / 16;
  const int64_t rowb = H * (int64_t)sizeof(T);
  const char* src = reinterpret_cast<const char*>(src_perm);
  const int32_t* rows = row_of_entry + t * k;
  const float* wts = weights ? weights + t * k : nullptr;
  char* dst = reinterpret_cast<char*>(out + t * H);
  for (int64_t v = lane; v < vecs; v += kWave) {
    float acc[V::N];
#pragma unroll
    for (int i = 0; i < V::N; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += 8) {
      u32x4 d[8];
      float wj[8];
      bool live[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        const int r = j < k ? rows[j] : -1;
        live[u] = r >= 0;          // -1: padding of the unrolled loop, or an invalid id
        wj[u] = wts && live[u] ? wts[j] : 1.f;
        if (live[u]) d[u] = ld16(src + (int64_t)r * rowb + v * 16);
        else d[u] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (live[u]) {
          float f[V::N];
          V::unpack(d[u], f);
#pragma unroll
          for (int i = 0; i < V::N; ++i) acc[i] = __builtin_fmaf(wj[u], f[i], acc[i]);
        }
      }
    }
    st16(dst + v * 16, V::pack(acc));
  }
}

// dy_perm[p] = w[a] * dy[a / k] (pad rows 0) and
// d_weights[a] = <dy[a / k], y_perm[p]> for the entry a on real row p.
template <typename T>
__global__ void __launch_bounds__(kRowsPerBlock * kWave)
scatter_backward_kernel(const T* __restrict__ dy, const T* __restrict__ y_perm,
                        const float* __restrict__ weights, int64_t H, int k,
                        const int32_t* __restrict__ tile_expert,
                        const int32_t* __restrict__ tpe,
                        const int32_t* __restrict__ bins,
                        const int32_t* __restrict__ padded_bins,
                        const int32_t* __restrict__ indices,
                        const int32_t* __restrict__ num_padded_rows,
                        T* __restrict__ dy_perm, float* __restrict__ d_weights) {
  using V = Vec16<T>;
  const int lane = threadIdx.x % kWave;
  const int64_t p = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (p >= *num_padded_rows) return;
  const int a = source_entry(p, tile_expert, tpe, bins, padded_bins, indices);
  const int64_t vecs = H * (int64_t)sizeof(T) / 16;
  char* dst = reinterpret_cast<char*>(dy_perm + p * H);
  if (a < 0) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t v = lane; v < vecs; v += kWave) st16(dst + v * 16, z);
    return;
  }
  const char* g = reinterpret_cast<const char*>(dy + (int64_t)(a / k) * H);
  const char* yp = reinterpret_cast<const char*>(y_perm + p * H);
  const float wt = weights[a];
  float dot = 0.f;
  for (int64_t v = lane; v < vecs; v += kWave) {
    float gf[V::N], yf[V::N], o[V::N];
    V::unpack(ld16(g + v * 16), gf);
    V::unpack(ld16(yp + v * 16), yf);
#pragma unroll
    for (int i = 0; i < V::N; ++i) {
      o[i] = wt * gf[i];
      dot = __builtin_fmaf(gf[i], yf[i], dot);
    }
    st16(dst + v * 16, V::pack(o));
  }
  dot = wave_sum(dot);
  if (lane == 0) d_weights[a] = dot;
}

static unsigned blocks_for(int64_t rows) {
  return (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
}

hipError_t launch_padded_gather(const Shape& s, const void* x, const MetaPtrs& m,
                                void* x_perm, hipStream_t stream) {
  const dim3 grid(blocks_for(s.max_tiles * kBlock)), block(kRowsPerBlock * kWave);
  if (s.bf16)
    hipLaunchKernelGGL(padded_gather_kernel<bf16>, grid, block, 0, stream,
                       static_cast<const bf16*>(x), s.H, s.k, m.tile_expert,
                       m.tokens_per_expert, m.bins, m.padded_bins, m.indices,
                       m.num_padded_rows, static_cast<bf16*>(x_perm));
  else
    hipLaunchKernelGGL(padded_gather_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(x), s.H, s.k, m.tile_expert,
                       m.tokens_per_expert, m.bins, m.padded_bins, m.indices,
                       m.num_padded_rows, static_cast<float*>(x_perm));
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
  const dim3 grid(blocks_for(s.max_tiles * kBlock)), block(kRowsPerBlock * kWave);
  if (s.bf16)
    hipLaunchKernelGGL(scatter_backward_kernel<bf16>, grid, block, 0, stream,
                       static_cast<const bf16*>(dy), static_cast<const bf16*>(y_perm),
                       weights, s.H, s.k, m.tile_expert, m.tokens_per_expert,
                       m.bins, m.padded_bins, m.indices, m.num_padded_rows,
                       static_cast<bf16*>(dy_perm), d_weights);
  else
    hipLaunchKernelGGL(scatter_backward_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(dy), static_cast<const float*>(y_perm),
                       weights, s.H, s.k, m.tile_expert, m.tokens_per_expert,
                       m.bins, m.padded_bins, m.indices, m.num_padded_rows,
                       static_cast<float*>(dy_perm), d_weights);
  return hipGetLastError();
}

}  // namespace dmoe
