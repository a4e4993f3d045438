// The router in front of the dropless MoE layer (gfx950): top-k of each
// token's expert logits, the softmax over the chosen k, the router z-loss,
// and their backward.
//
// The Fast-LLM issue "[feat] Support sparse copy for a large number of
// experts" routes each token to num_experts_per_token experts and sets an
// expert_z_loss_coefficient; the "yikangshen/megablocks" README names the
// z-loss of ST-MoE.  Here: the k largest logits in descending order, equal
// logits to the lower expert id; weights = softmax over those k logits;
// z-loss = coef * mean_t (log sum_e exp l[t, e])^2.  The selection carries no
// gradient; the softmax's flows to the chosen logits, the z-loss's to all.
//
// One wave per token (E <= 256: four logits per lane).  Logits must be
// finite.  No atomics: every output is written by one lane, and the z-loss mean is summed by one
// workgroup in a fixed order, so results are bit-reproducible.
#include <float.h>

#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {

constexpr int kRouterWaves = 4;                    // tokens per workgroup
constexpr int kPerLane = kMaxExperts / kWave;      // logits per lane
constexpr int kSumThreads = 1024;

// A finite float as an unsigned key with the same order (negative values
// flipped whole, positive ones above them; -0 taken as +0, the two being
// one value in a comparison); 0 is below every key.  Bitwise, so subnormal
// logits keep their order whatever the float mode.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Maximum of v over the wave, in every lane.  Cross-lane moves by DPP (an
// inclusive max-scan inside each row of 16 lanes by shifts of 1, 2, 4 and
// 8, then row 15 to row 1 and 3, lane 31 to rows 2 and 3), so lane 63 ends
// with the maximum; no LDS traffic.  Lanes whose source is outside the row
// read 0, the identity.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  const auto step = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// ids [T,k], weights [T,k]; z [T] = (log sum_e exp l)^2 when z is not null.
// Lane (j mod 64) keeps the j-th chosen logit in slot j / 64 of sel.
__global__ void __launch_bounds__(kRouterWaves * kWave)
router_forward_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                      int32_t* __restrict__ ids, float* __restrict__ weights,
                      float* __restrict__ z) {
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kRouterWaves + w;
  if (t >= T) return;                    // the whole wave leaves together
  const float* row = logits + t * E;
  float v[kPerLane], sel[kPerLane];
  bool live[kPerLane];
#pragma unroll
  for (int q = 0; q < kPerLane; ++q) {
    const int e = q * kWave + lane;
    live[q] = e < E;
    v[q] = live[q] ? row[e] : -FLT_MAX;
    sel[q] = 0.f;
  }
  uint32_t key[kPerLane];
#pragma unroll
  for (int q = 0; q < kPerLane; ++q) key[q] = live[q] ? order_key(v[q]) : 0u;
  for (int j = 0; j < k; ++j) {
    // the largest remaining logit, then the lowest expert id holding it
    // (expert q * 64 + lane: the first slot q with a holder, its lowest lane)
    uint32_t lk = 0u;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) lk = key[q] > lk ? key[q] : lk;
    const uint32_t best = wave_umax(lk);
    int bi = INT32_MAX;
#pragma unroll
    for (int q = kPerLane - 1; q >= 0; --q) {
      const unsigned long long hold = __ballot(key[q] == best && best != 0u);
      if (hold) bi = q * kWave + (__ffsll((long long)hold) - 1);
    }
    const float bv = key_value(best);
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
      if (q * kWave + lane == bi) key[q] = 0u;
      if (q * kWave + lane == bi) live[q] = false;
      if (q == j / kWave && lane == j % kWave) sel[q] = bv;
    }
    if (lane == 0) ids[t * k + j] = bi;
  }
  // The first chosen logit is the largest of the row.
  const float m = __shfl(sel[0], 0, kWave);
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < kPerLane; ++q)
    if (q * kWave + lane < k) s += __expf(sel[q] - m);
  s = wave_sum(s);
#pragma unroll
  for (int q = 0; q < kPerLane; ++q) {
    const int j = q * kWave + lane;
    if (j < k) weights[t * k + j] = __expf(sel[q] - m) / s;
  }
  if (z) {
    float se = 0.f;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q)
      if (q * kWave + lane < E) se += __expf(v[q] - m);
    se = wave_sum(se);
    const float lse = m + __logf(se);
    if (lane == 0) z[t] = lse * lse;
  }
}

// loss[0] = coef * mean(z): one workgroup, fixed order.
__global__ void __launch_bounds__(kSumThreads)
zloss_mean_kernel(const float* __restrict__ z, int64_t T, float coef, float* __restrict__ loss) {
  __shared__ double part[kSumThreads];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < T; i += kSumThreads) acc += z[i];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int n = kSumThreads / 2; n > 0; n >>= 1) {
    if ((int)threadIdx.x < n) part[threadIdx.x] += part[threadIdx.x + n];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)(coef * part[0] / (double)T);
}

// d_logits [T,E]: w_j (g_j - sum_i w_i g_i) at the chosen experts, 0
// elsewhere, plus coef * 2 / T * lse * softmax(l) when coef != 0.
__global__ void __launch_bounds__(kRouterWaves * kWave)
router_backward_kernel(const float* __restrict__ logits, const int32_t* __restrict__ ids,
                       const float* __restrict__ weights, const float* __restrict__ d_weights,
                       int64_t T, int E, int k, float coef, float* __restrict__ d_logits) {
  __shared__ int pos[kRouterWaves][kMaxExperts];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kRouterWaves + w;
  const bool active = t < T;             // no early return: the block syncs twice
#pragma unroll
  for (int q = 0; q < kPerLane; ++q) pos[w][q * kWave + lane] = -1;
  __syncthreads();
  float dot = 0.f;
  if (active)
    for (int j = lane; j < k; j += kWave) {
      const int e = ids[t * k + j];
      if (e >= 0 && e < E) pos[w][e] = j;
      dot += weights[t * k + j] * d_weights[t * k + j];
    }
  __syncthreads();
  if (!active) return;
  dot = wave_sum(dot);
  const float* row = logits + t * E;
  float v[kPerLane];
#pragma unroll
  for (int q = 0; q < kPerLane; ++q) {
    const int e = q * kWave + lane;
    v[q] = e < E ? row[e] : -FLT_MAX;
  }
  float m = 0.f, zscale = 0.f;
  if (coef != 0.f) {
    float lm = -FLT_MAX;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) lm = fmaxf(lm, v[q]);
    m = wave_max(lm);
    float se = 0.f;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q)
      if (q * kWave + lane < E) se += __expf(v[q] - m);
    se = wave_sum(se);
    const float lse = m + __logf(se);
    zscale = coef * 2.0f / (float)T * lse / se;   // times exp(l - m) = softmax * se
  }
#pragma unroll
  for (int q = 0; q < kPerLane; ++q) {
    const int e = q * kWave + lane;
    if (e >= E) continue;
    const int j = pos[w][e];
    float out = 0.f;
    if (j >= 0) out = weights[t * k + j] * (d_weights[t * k + j] - dot);
    if (coef != 0.f) out += zscale * __expf(v[q] - m);
    d_logits[t * E + e] = out;
  }
}

static unsigned router_blocks(int64_t T) {
  return (unsigned)((T + kRouterWaves - 1) / kRouterWaves);
}

hipError_t launch_router_forward(const Shape& s, const float* logits, float coef,
                                 int32_t* ids, float* weights, float* z, float* loss,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(router_forward_kernel, dim3(router_blocks(s.T)), dim3(kRouterWaves * kWave),
                     0, stream, logits, s.T, s.E, s.k, ids, weights, z);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !z) return err;
  hipLaunchKernelGGL(zloss_mean_kernel, dim3(1), dim3(kSumThreads), 0, stream, z, s.T, coef,
                     loss);
  return hipGetLastError();
}

hipError_t launch_router_backward(const Shape& s, const float* logits, const int32_t* ids,
                                  const float* weights, const float* d_weights, float coef,
                                  float* d_logits, hipStream_t stream) {
  hipLaunchKernelGGL(router_backward_kernel, dim3(router_blocks(s.T)),
                     dim3(kRouterWaves * kWave), 0, stream, logits, ids, weights, d_weights, s.T,
                     s.E, s.k, coef, d_logits);
  return hipGetLastError();
}

}  // namespace dmoe
