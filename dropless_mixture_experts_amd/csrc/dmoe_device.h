// Device-side helpers shared by the dMoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmoe {

constexpr int kBlock = 128;          // rows per padded block (MegaBlocks §2)
constexpr int kWave = 64;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) {
  return static_cast<bf16>(v);
}

// 16 bytes as 8 bf16 or 4 fp32, converted to fp32 lanes.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const u32x4& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
  }
  __device__ __forceinline__ static u32x4 pack(const float* in) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(in[i]);
    return v;
  }
};
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const u32x4& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static u32x4 pack(const float* in) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = __builtin_bit_cast(uint16_t, from_f32<bf16>(in[2 * i]));
      uint32_t hi = __builtin_bit_cast(uint16_t, from_f32<bf16>(in[2 * i + 1]));
      v[i] = lo | (hi << 16);
    }
    return v;
  }
};

// 16-byte global loads and store.  ld16_nt marks the line for early eviction:
// for rows that one wave reads once and nothing reads again soon (the
// scatter's inputs), where it also lets the memory system stream them faster.
// Every store of the row kernels is non-temporal (st16_nt): the next kernel,
// not this one, reads what it writes, and without the hint the dirty lines
// are written back under that kernel's loads.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Sum of v over the wave, in every lane, in a fixed order.  Cross-lane moves
// by DPP, with no LDS traffic: an inclusive sum-scan inside each row of 16
// lanes by shifts of 1, 2, 4 and 8 (a lane outside the row adds 0), then row
// 0's lane 15 into row 1 and row 2's into row 3, then lane 31 into rows 2
// and 3, so lane 63 holds the total.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// The logistic function 1 / (1 + exp(-z)), with the hardware reciprocal
// (v_rcp_f32, about 1 ulp) in place of an IEEE division, which costs about
// ten instructions per element in the epilogues that apply the gate.  For
// z -> -inf it gives 0, for z -> +inf 1, and NaN stays NaN.
__device__ __forceinline__ float sigmoid(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}
// The gated SiLU of the expert FFN, silu(h1) * h3 with silu(z) = z
// sigmoid(z), on the stored (layer-dtype) values of h1 and h3.  The forward
// epilogues and the activation recompute all call this one definition, so a
// recomputed activation is bit-identical to the forward's.
__device__ __forceinline__ float silu(float z) { return z * sigmoid(z); }
__device__ __forceinline__ float gated_silu(float h1, float h3) { return silu(h1) * h3; }

__device__ __forceinline__ int round_up_block(int c) {
  return ((c + kBlock - 1) / kBlock) * kBlock;
}

}  // namespace dmoe
