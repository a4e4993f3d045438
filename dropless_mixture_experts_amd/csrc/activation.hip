// The expert FFN's activation recomputed from its stored pre-activations:
// act = silu(h1) * h3 over the padded rows [0, P).  The memory-optimized
// MLP of the MegaBlocks chapter (§4.4) recomputes the activation in the
// backward instead of keeping it from the forward; with this kernel the
// caller may reuse act's memory between the two.  gated_silu is the
// definition the forward epilogue uses, on the same stored values, so the
// result is bit-identical to the forward's act.
//
// HBM-bound: 3 P F s bytes (h1 and h3 in, act out), 16 bytes per lane.
#include <algorithm>

#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {

constexpr int kActThreads = 256;
constexpr int64_t kActMaxBlocks = 8192;

template <typename T>
__global__ void __launch_bounds__(kActThreads)
recompute_act_kernel(const T* __restrict__ h1, const T* __restrict__ h3, int64_t F,
                     const int32_t* __restrict__ num_padded_rows, T* __restrict__ act) {
  using V = Vec16<T>;
  // F is a multiple of 128, so rows are whole 16-byte chunks
  const int64_t n = (int64_t)(*num_padded_rows) * F / V::N;
  const int64_t stride = (int64_t)gridDim.x * kActThreads;
  for (int64_t i = (int64_t)blockIdx.x * kActThreads + threadIdx.x; i < n; i += stride) {
    float a[V::N], b[V::N];
    V::unpack(ld16(h1 + i * V::N), a);
    V::unpack(ld16(h3 + i * V::N), b);
#pragma unroll
    for (int r = 0; r < V::N; ++r) a[r] = gated_silu(a[r], b[r]);
    st16_nt(act + i * V::N, V::pack(a));
  }
}

hipError_t launch_recompute_act(const Shape& s, const void* h1, const void* h3,
                                const MetaPtrs& m, void* act, hipStream_t stream) {
  const int64_t chunks = s.max_tiles * kBlock * s.F / (s.bf16 ? 8 : 4);
  const unsigned grid = (unsigned)std::min<int64_t>(
      kActMaxBlocks, std::max<int64_t>(1, (chunks + kActThreads - 1) / kActThreads));
  if (s.bf16)
    hipLaunchKernelGGL(recompute_act_kernel<bf16>, dim3(grid), dim3(kActThreads), 0, stream,
                       static_cast<const bf16*>(h1), static_cast<const bf16*>(h3), s.F,
                       m.num_padded_rows, static_cast<bf16*>(act));
  else
    hipLaunchKernelGGL(recompute_act_kernel<float>, dim3(grid), dim3(kActThreads), 0, stream,
                       static_cast<const float*>(h1), static_cast<const float*>(h3), s.F,
                       m.num_padded_rows, static_cast<float*>(act));
  return hipGetLastError();
}

}  // namespace dmoe
