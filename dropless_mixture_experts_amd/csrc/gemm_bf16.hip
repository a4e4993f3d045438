// bf16 grouped GEMM over expert-tagged 128-row tiles (gfx950 MFMA).
//
// The products are those of the MegaBlocks chapter "02 · dropless MoE 与
// block-sparse 重构" §3 (sdd: x_perm w1 / x_perm w3, dsd: act w2, on the row
// blocks of each expert only) and their backward, exactly as in the generic
// engine of gemm.hip; this file is the bf16 fast path.
//
// Engine
//   * 256 threads = 4 waves (2 x 2); block tile 256 "A rows" (the output's
//     contiguous dimension, weights side) x 128 "B rows" (token rows, or the
//     m dimension of a weight gradient); each wave owns 128 x 64 as 8 x 4
//     v_mfma_f32_16x16x32_bf16 tiles (128 fp32 accumulators in AGPRs).
//   * K step 64 (128 bytes per LDS row); two LDS stages of 48 KB.  The next
//     step's global loads are issued right after the current step's LDS
//     store, so their latency hides behind a whole step of MFMAs.
//   * LDS rows are unpadded; the 16-byte chunk c of row r lives at chunk
//     c ^ ((r & 7) ^ ((r >> 3) & 1)), so the 16 rows read by one quarter of a
//     wave hit distinct banks whether the LDS serves 8 or 16 lanes per cycle.
//   * Global reads are buffer loads: the tile base is in SGPRs, each lane
//     keeps a 32-bit offset that never changes, and the K step advances the
//     scalar offset.
//   * Row-contiguous sources ([K][N] weights, and both operands of the weight
//     gradients) are read in 8 x 8 (or 8 x 4) micro-blocks and transposed in
//     registers with v_perm before the LDS store.
//   * A tile that has only 128 A rows (a dimension that is an odd multiple
//     of 128) runs the same code with the second half compiled out.
#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {
namespace bfk {

constexpr int kThreads = 256;
constexpr int kRowB = 128;                    // bytes of K per LDS row per step
constexpr int kKStep = kRowB / 2;             // 64 bf16
constexpr int kStageA = 256 * kRowB;          // 32 KB
constexpr int kStageB = 128 * kRowB;          // 16 KB
constexpr int kStage = kStageA + kStageB;     // 48 KB
constexpr int kLds = 2 * kStage;              // 96 KB

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p) {
  // raw buffer, no stride; the range is not used for bounds (every access
  // is in bounds by construction), so take the largest positive size.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ u32x2 bload8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowB + ((chunk ^ swz(row)) << 4);
}
__device__ __forceinline__ void lds_st16(char* lds, int off, const u32x4& v) {
  *reinterpret_cast<u32x4*>(lds + off) = v;
}

// One operand.  Tile rows [0,128) come from r0 and rows [128,256) from r1
// (A side only).  ld: bytes between consecutive source rows.
struct Op {
  rsrc_t r0, r1;
  uint32_t ld;
};

// ---- K-contiguous source (rows of the tile are rows of the source) -------
// ROWS/32 slots of 16 bytes per thread: slot q covers tile row
// (tid >> 3) + 32 q, chunk tid & 7.
template <int ROWS>
struct DirectLoader {
  static constexpr int kSlots = ROWS / 32;
  u32x4 v[kSlots];
  uint32_t voff;      // (tid >> 3) * ld + (tid & 7) * 16
  uint32_t ld32;      // 32 * ld
  int lds0;           // LDS offset of slot 0
  __device__ __forceinline__ void init(const Op& op, int tid) {
    voff = (uint32_t)(tid >> 3) * op.ld + (uint32_t)(tid & 7) * 16u;
    ld32 = 32u * op.ld;
    lds0 = lds_off(tid >> 3, tid & 7);
  }
  template <bool FULL>
  __device__ __forceinline__ void load(const Op& op, int ks) {
    const uint32_t soff = (uint32_t)ks * kRowB;
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
      if (!FULL && q >= 4) break;
      const rsrc_t r = q < 4 ? op.r0 : op.r1;
      v[q] = bload16(r, voff + (uint32_t)(q & 3) * ld32, soff);
    }
  }
  template <bool FULL>
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
      if (!FULL && q >= 4) break;
      lds_st16(lds, lds0 + q * 32 * kRowB, v[q]);
    }
  }
};

// ---- Row-contiguous source, 256-row A tile --------------------------------
// Thread: half = tid >> 7 (one per pair of waves), kblk = (tid & 127) >> 4
// (8 source rows), nblk = tid & 15 (8 source columns = 16 bytes).  Eight
// 16-byte loads, an 8 x 8 transpose, eight 16-byte LDS stores.
struct TransLoaderA {
  u32x4 v[8];
  uint32_t voff;
  int half, kblk, nblk;
  __device__ __forceinline__ void init(const Op& op, int tid) {
    half = __builtin_amdgcn_readfirstlane(tid >> 7);   // uniform per wave
    kblk = (tid & 127) >> 4;
    nblk = tid & 15;
    voff = (uint32_t)(kblk * 8) * op.ld + (uint32_t)nblk * 16u;
  }
  template <bool FULL>
  __device__ __forceinline__ void load(const Op& op, int ks) {
    if (!FULL && half) return;
    const uint32_t soff = (uint32_t)ks * kKStep * op.ld;
    const rsrc_t r = half ? op.r1 : op.r0;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = bload16(r, voff + (uint32_t)i * op.ld, soff);
  }
  template <bool FULL>
  __device__ __forceinline__ void store(char* lds) const {
    if (!FULL && half) return;
    const int row0 = half * 128 + nblk * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int dw = c >> 1;
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = __builtin_amdgcn_perm(v[2 * q + 1][dw], v[2 * q][dw], sel);
      lds_st16(lds, lds_off(row0 + c, kblk), o);
    }
  }
};

// ---- Row-contiguous source, 128-row B tile --------------------------------
// Thread: kblk = tid >> 5 (8 source rows), nblk = tid & 31 (4 columns = 8
// bytes).  Eight 8-byte loads, an 8 x 4 transpose, four 16-byte LDS stores.
struct TransLoaderB {
  u32x2 v[8];
  uint32_t voff;
  int kblk, nblk;
  __device__ __forceinline__ void init(const Op& op, int tid) {
    kblk = tid >> 5;
    nblk = tid & 31;
    voff = (uint32_t)(kblk * 8) * op.ld + (uint32_t)nblk * 8u;
  }
  template <bool FULL>
  __device__ __forceinline__ void load(const Op& op, int ks) {
    const uint32_t soff = (uint32_t)ks * kKStep * op.ld;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = bload8(op.r0, voff + (uint32_t)i * op.ld, soff);
  }
  template <bool FULL>
  __device__ __forceinline__ void store(char* lds) const {
    const int row0 = nblk * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int dw = c >> 1;
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = __builtin_amdgcn_perm(v[2 * q + 1][dw], v[2 * q][dw], sel);
      lds_st16(lds, lds_off(row0 + c, kblk), o);
    }
  }
};

typedef f32x4 Acc[8][4];

__device__ __forceinline__ int a_row(int i, int wm) { return (i >> 2) * 128 + wm * 64 + (i & 3) * 16; }
__device__ __forceinline__ int b_row(int j, int wn) { return wn * 64 + j * 16; }

// acc += A . B^T over one 64-wide K step held in one LDS stage.
template <bool FULL>
__device__ __forceinline__ void mma_step(Acc& acc, const char* lds, int wm, int wn, int lane) {
  const char* la = lds;
  const char* lb = lds + kStageA;
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int kf = 0; kf < 2; ++kf) {
    const int chunk = kf * 4 + lq;
    bf16x8 b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(lb + lds_off(b_row(j, wn) + lr, chunk));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!FULL && i >= 4) break;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(la + lds_off(a_row(i, wm) + lr, chunk));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i][j], 0, 0, 0);
    }
  }
}

template <class LA, class LB, bool FULL>
__device__ __forceinline__ void mainloop(Acc& acc, const Op& A, const Op& B, int nk, char* lds) {
  if (nk <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  LA la;
  LB lb;
  la.init(A, tid);
  lb.init(B, tid);
  la.template load<FULL>(A, 0);
  lb.template load<FULL>(B, 0);
  la.template store<FULL>(lds);
  lb.template store<FULL>(lds + kStageA);
  if (nk > 1) {
    la.template load<FULL>(A, 1);
    lb.template load<FULL>(B, 1);
  }
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    mma_step<FULL>(acc, lds + (ks & 1) * kStage, wm, wn, lane);
    if (ks + 1 < nk) {
      char* nxt = lds + ((ks + 1) & 1) * kStage;
      la.template store<FULL>(nxt);
      lb.template store<FULL>(nxt + kStageA);
      if (ks + 2 < nk) {
        la.template load<FULL>(A, ks + 2);
        lb.template load<FULL>(B, ks + 2);
      }
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void zero(Acc& acc) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ void store4(bf16* p, const f32x4& v) {
  const uint32_t a = __builtin_bit_cast(uint16_t, from_f32<bf16>(v[0])) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(v[1])) << 16);
  const uint32_t b = __builtin_bit_cast(uint16_t, from_f32<bf16>(v[2])) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(v[3])) << 16);
  *reinterpret_cast<u32x2*>(p) = u32x2{a, b};
}
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  const u32x2 u = *reinterpret_cast<const u32x2*>(p);
  return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

#define BF_PROLOGUE                                                   \
  __shared__ __attribute__((aligned(16))) char lds[kLds];             \
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;         \
  const int wm = w >> 1, wn = w & 1;                                  \
  const int lr = (lane >> 4) * 4, lc = lane & 15;

// h1 = x_perm w1[e], h3 = x_perm w3[e], act = silu(h1) * h3.
// grid = (F/128, max_tiles).
__global__ void __launch_bounds__(kThreads)
up_kernel(const bf16* __restrict__ x_perm, const bf16* __restrict__ w1,
          const bf16* __restrict__ w3, int64_t H, int64_t F,
          const int32_t* __restrict__ tile_expert, bf16* __restrict__ h1,
          bf16* __restrict__ h3, bf16* __restrict__ act) {
  BF_PROLOGUE
  const int64_t mt = blockIdx.y, f0 = (int64_t)blockIdx.x * 128;
  const int e = tile_expert[mt];
  if (e < 0) return;
  const int64_t wofs = (int64_t)e * H * F + f0;
  const Op A{make_rsrc(w1 + wofs), make_rsrc(w3 + wofs), (uint32_t)(F * 2)};
  const Op B{make_rsrc(x_perm + mt * kBlock * H), make_rsrc(x_perm), (uint32_t)(H * 2)};
  Acc acc;
  zero(acc);
  mainloop<TransLoaderA, DirectLoader<128>, true>(acc, A, B, (int)(H / kKStep), lds);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = mt * kBlock + b_row(j, wn) + lc;
      const int64_t f = f0 + a_row(i, wm) + lr;
      const f32x4 v1 = acc[i][j], v3 = acc[i + 4][j];
      f32x4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = silu(v1[r]) * v3[r];
      store4(h1 + p * F + f, v1);
      store4(h3 + p * F + f, v3);
      store4(act + p * F + f, a);
    }
}

// y_perm = act w2[e].  grid = (ceil(H/256), max_tiles).
template <bool FULL>
__device__ __forceinline__ void down_body(const bf16* act, const bf16* w2, int64_t H,
                                          int64_t F, int64_t mt, int64_t h0, int e,
                                          bf16* y_perm, char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int lr = (lane >> 4) * 4, lc = lane & 15;
  const bf16* wb = w2 + (int64_t)e * F * H + h0;
  const Op A{make_rsrc(wb), make_rsrc(wb + 128), (uint32_t)(H * 2)};
  const Op B{make_rsrc(act + mt * kBlock * F), make_rsrc(act), (uint32_t)(F * 2)};
  Acc acc;
  zero(acc);
  mainloop<TransLoaderA, DirectLoader<128>, FULL>(acc, A, B, (int)(F / kKStep), lds);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (!FULL && i >= 4) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = mt * kBlock + b_row(j, wn) + lc;
      store4(y_perm + p * H + h0 + a_row(i, wm) + lr, acc[i][j]);
    }
  }
}

__global__ void __launch_bounds__(kThreads)
down_kernel(const bf16* __restrict__ act, const bf16* __restrict__ w2, int64_t H,
            int64_t F, const int32_t* __restrict__ tile_expert, bf16* __restrict__ y_perm) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  const int64_t mt = blockIdx.y, h0 = (int64_t)blockIdx.x * 256;
  const int e = tile_expert[mt];
  if (e < 0) return;
  if (h0 + 256 <= H)
    down_body<true>(act, w2, H, F, mt, h0, e, y_perm, lds);
  else
    down_body<false>(act, w2, H, F, mt, h0, e, y_perm, lds);
}

// dA = dy_perm w2[e]^T, then the gate's backward.  grid = (ceil(F/256), max_tiles).
template <bool FULL>
__device__ __forceinline__ void down_dgrad_body(const bf16* dy_perm, const bf16* w2,
                                                const bf16* h1, const bf16* h3, int64_t H,
                                                int64_t F, int64_t mt, int64_t fb, int e,
                                                bf16* dh1, bf16* dh3, char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int lr = (lane >> 4) * 4, lc = lane & 15;
  const bf16* wb = w2 + (int64_t)e * F * H + fb * H;
  const Op A{make_rsrc(wb), make_rsrc(wb + 128 * H), (uint32_t)(H * 2)};
  const Op B{make_rsrc(dy_perm + mt * kBlock * H), make_rsrc(dy_perm), (uint32_t)(H * 2)};
  Acc acc;
  zero(acc);
  mainloop<DirectLoader<256>, DirectLoader<128>, FULL>(acc, A, B, (int)(H / kKStep), lds);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (!FULL && i >= 4) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = mt * kBlock + b_row(j, wn) + lc;
      const int64_t o = p * F + fb + a_row(i, wm) + lr;
      const f32x4 g1 = load4(h1 + o), g3 = load4(h3 + o);
      f32x4 d1, d3;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float da = acc[i][j][r];
        const float s = 1.0f / (1.0f + __expf(-g1[r]));
        d3[r] = da * g1[r] * s;
        d1[r] = da * g3[r] * s * (1.0f + g1[r] * (1.0f - s));
      }
      store4(dh1 + o, d1);
      store4(dh3 + o, d3);
    }
  }
}

__global__ void __launch_bounds__(kThreads)
down_dgrad_kernel(const bf16* __restrict__ dy_perm, const bf16* __restrict__ w2,
                  const bf16* h1, const bf16* h3, int64_t H, int64_t F,
                  const int32_t* __restrict__ tile_expert, bf16* dh1, bf16* dh3) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  const int64_t mt = blockIdx.y, fb = (int64_t)blockIdx.x * 256;
  const int e = tile_expert[mt];
  if (e < 0) return;
  if (fb + 256 <= F)
    down_dgrad_body<true>(dy_perm, w2, h1, h3, H, F, mt, fb, e, dh1, dh3, lds);
  else
    down_dgrad_body<false>(dy_perm, w2, h1, h3, H, F, mt, fb, e, dh1, dh3, lds);
}

// dx_perm = dh1 w1[e]^T + dh3 w3[e]^T.  grid = (ceil(H/256), max_tiles).
template <bool FULL>
__device__ __forceinline__ void up_dgrad_body(const bf16* dh1, const bf16* dh3,
                                              const bf16* w1, const bf16* w3, int64_t H,
                                              int64_t F, int64_t mt, int64_t h0, int e,
                                              bf16* dx_perm, char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int lr = (lane >> 4) * 4, lc = lane & 15;
  const int64_t wofs = (int64_t)e * H * F + h0 * F;
  const int nk = (int)(F / kKStep);
  Acc acc;
  zero(acc);
  {
    const Op A{make_rsrc(w1 + wofs), make_rsrc(w1 + wofs + 128 * F), (uint32_t)(F * 2)};
    const Op B{make_rsrc(dh1 + mt * kBlock * F), make_rsrc(dh1), (uint32_t)(F * 2)};
    mainloop<DirectLoader<256>, DirectLoader<128>, FULL>(acc, A, B, nk, lds);
  }
  {
    const Op A{make_rsrc(w3 + wofs), make_rsrc(w3 + wofs + 128 * F), (uint32_t)(F * 2)};
    const Op B{make_rsrc(dh3 + mt * kBlock * F), make_rsrc(dh3), (uint32_t)(F * 2)};
    mainloop<DirectLoader<256>, DirectLoader<128>, FULL>(acc, A, B, nk, lds);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (!FULL && i >= 4) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = mt * kBlock + b_row(j, wn) + lc;
      store4(dx_perm + p * H + h0 + a_row(i, wm) + lr, acc[i][j]);
    }
  }
}

__global__ void __launch_bounds__(kThreads)
up_dgrad_kernel(const bf16* __restrict__ dh1, const bf16* __restrict__ dh3,
                const bf16* __restrict__ w1, const bf16* __restrict__ w3, int64_t H,
                int64_t F, const int32_t* __restrict__ tile_expert, bf16* dx_perm) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  const int64_t mt = blockIdx.y, h0 = (int64_t)blockIdx.x * 256;
  const int e = tile_expert[mt];
  if (e < 0) return;
  if (h0 + 256 <= H)
    up_dgrad_body<true>(dh1, dh3, w1, w3, H, F, mt, h0, e, dx_perm, lds);
  else
    up_dgrad_body<false>(dh1, dh3, w1, w3, H, F, mt, h0, e, dx_perm, lds);
}

// dw2[e] = act[rows_e]^T dy_perm[rows_e] ([F,H]).  grid = (ceil(H/256), F/128, E).
template <bool FULL>
__device__ __forceinline__ void wgrad_down_body(const bf16* act, const bf16* dy_perm,
                                                int64_t H, int64_t F, int64_t start, int n,
                                                int64_t h0, int64_t f0, int e, bf16* dw2,
                                                char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int lr = (lane >> 4) * 4, lc = lane & 15;
  const bf16* ab = dy_perm + start * H + h0;
  const Op A{make_rsrc(ab), make_rsrc(ab + 128), (uint32_t)(H * 2)};
  const Op B{make_rsrc(act + start * F + f0), make_rsrc(act), (uint32_t)(F * 2)};
  Acc acc;
  zero(acc);
  mainloop<TransLoaderA, TransLoaderB, FULL>(acc, A, B, n / kKStep, lds);
  bf16* out = dw2 + (int64_t)e * F * H;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (!FULL && i >= 4) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t f = f0 + b_row(j, wn) + lc;
      store4(out + f * H + h0 + a_row(i, wm) + lr, acc[i][j]);
    }
  }
}

__global__ void __launch_bounds__(kThreads)
wgrad_down_kernel(const bf16* __restrict__ act, const bf16* __restrict__ dy_perm,
                  int64_t H, int64_t F, const int32_t* __restrict__ tpe,
                  const int32_t* __restrict__ padded_bins, bf16* __restrict__ dw2) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  const int64_t h0 = (int64_t)blockIdx.x * 256, f0 = (int64_t)blockIdx.y * 128;
  const int e = blockIdx.z;
  const int n = round_up_block(tpe[e]);
  const int64_t start = padded_bins[e] - n;
  if (h0 + 256 <= H)
    wgrad_down_body<true>(act, dy_perm, H, F, start, n, h0, f0, e, dw2, lds);
  else
    wgrad_down_body<false>(act, dy_perm, H, F, start, n, h0, f0, e, dw2, lds);
}

// dw1[e] = x_perm[rows_e]^T dh1[rows_e], dw3[e] = x_perm[rows_e]^T dh3[rows_e].
// grid = (F/128, H/128, E).
__global__ void __launch_bounds__(kThreads)
wgrad_up_kernel(const bf16* __restrict__ x_perm, const bf16* __restrict__ dh1,
                const bf16* __restrict__ dh3, int64_t H, int64_t F,
                const int32_t* __restrict__ tpe, const int32_t* __restrict__ padded_bins,
                bf16* __restrict__ dw1, bf16* __restrict__ dw3) {
  BF_PROLOGUE
  const int64_t f0 = (int64_t)blockIdx.x * 128, h0 = (int64_t)blockIdx.y * 128;
  const int e = blockIdx.z;
  const int n = round_up_block(tpe[e]);
  const int64_t start = padded_bins[e] - n;
  const Op A{make_rsrc(dh1 + start * F + f0), make_rsrc(dh3 + start * F + f0), (uint32_t)(F * 2)};
  const Op B{make_rsrc(x_perm + start * H + h0), make_rsrc(x_perm), (uint32_t)(H * 2)};
  Acc acc;
  zero(acc);
  mainloop<TransLoaderA, TransLoaderB, true>(acc, A, B, n / kKStep, lds);
  const int64_t eo = (int64_t)e * H * F;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t h = h0 + b_row(j, wn) + lc;
      const int64_t f = f0 + a_row(i & 3, wm) + lr;
      store4((i < 4 ? dw1 : dw3) + eo + h * F + f, acc[i][j]);
    }
}

}  // namespace bfk

static unsigned cdiv_u(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

hipError_t launch_bf16_up(const Shape& s, const void* x_perm, const void* w1, const void* w3,
                          const MetaPtrs& m, void* h1, void* h3, void* act,
                          hipStream_t stream) {
  hipLaunchKernelGGL(bfk::up_kernel, dim3(cdiv_u(s.F, 128), (unsigned)s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(x_perm),
                     static_cast<const bf16*>(w1), static_cast<const bf16*>(w3), s.H, s.F,
                     m.tile_expert, static_cast<bf16*>(h1), static_cast<bf16*>(h3),
                     static_cast<bf16*>(act));
  return hipGetLastError();
}

hipError_t launch_bf16_down(const Shape& s, const void* act, const void* w2,
                            const MetaPtrs& m, void* y_perm, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::down_kernel, dim3(cdiv_u(s.H, 256), (unsigned)s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(act),
                     static_cast<const bf16*>(w2), s.H, s.F, m.tile_expert,
                     static_cast<bf16*>(y_perm));
  return hipGetLastError();
}

hipError_t launch_bf16_down_dgrad(const Shape& s, const void* dy_perm, const void* w2,
                                  const void* h1, const void* h3, const MetaPtrs& m,
                                  void* dh1, void* dh3, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::down_dgrad_kernel, dim3(cdiv_u(s.F, 256), (unsigned)s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(dy_perm),
                     static_cast<const bf16*>(w2), static_cast<const bf16*>(h1),
                     static_cast<const bf16*>(h3), s.H, s.F, m.tile_expert,
                     static_cast<bf16*>(dh1), static_cast<bf16*>(dh3));
  return hipGetLastError();
}

hipError_t launch_bf16_up_dgrad(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const MetaPtrs& m,
                                void* dx_perm, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::up_dgrad_kernel, dim3(cdiv_u(s.H, 256), (unsigned)s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(dh1),
                     static_cast<const bf16*>(dh3), static_cast<const bf16*>(w1),
                     static_cast<const bf16*>(w3), s.H, s.F, m.tile_expert,
                     static_cast<bf16*>(dx_perm));
  return hipGetLastError();
}

hipError_t launch_bf16_wgrad_down(const Shape& s, const void* act, const void* dy_perm,
                                  const MetaPtrs& m, void* dw2, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::wgrad_down_kernel,
                     dim3(cdiv_u(s.H, 256), cdiv_u(s.F, 128), (unsigned)s.E),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(act),
                     static_cast<const bf16*>(dy_perm), s.H, s.F, m.tokens_per_expert,
                     m.padded_bins, static_cast<bf16*>(dw2));
  return hipGetLastError();
}

hipError_t launch_bf16_wgrad_up(const Shape& s, const void* x_perm, const void* dh1,
                                const void* dh3, const MetaPtrs& m, void* dw1, void* dw3,
                                hipStream_t stream) {
  hipLaunchKernelGGL(bfk::wgrad_up_kernel,
                     dim3(cdiv_u(s.F, 128), cdiv_u(s.H, 128), (unsigned)s.E),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(x_perm),
                     static_cast<const bf16*>(dh1), static_cast<const bf16*>(dh3), s.H,
                     s.F, m.tokens_per_expert, m.padded_bins, static_cast<bf16*>(dw1),
                     static_cast<bf16*>(dw3));
  return hipGetLastError();
}

}  // namespace dmoe
