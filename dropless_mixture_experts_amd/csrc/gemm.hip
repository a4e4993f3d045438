// Grouped GEMM over expert-tagged 128-row tiles (gfx950 MFMA), fp32.  The
// launch_gemm_* entry points below route bf16 to the engine of
// gemm_bf16.hip; the kernels of this file run the fp32 layer.
//
// MegaBlocks chapter "02 · dropless MoE 与 block-sparse 重构" §2-§3: once each
// expert's rows are padded to a multiple of 128, every 128-row block of the
// padded token matrix belongs to one expert, so the expert FFN is a block-
// sparse product whose non-zero blocks are exactly (row block r, the columns
// of expert tile_expert[r]).  The sdd product (x_perm w1, x_perm w3) and the
// dsd product (act w2) are computed here as one launch each over all row
// blocks, each block reading its own expert's weights; §5's GLU variant
// shares the row-block -> expert map.  The backward products (dgrad of both
// projections and the per-expert weight gradients, whose contraction runs
// over the expert's padded row range) use the same tile engine.
//
// Tile engine
//   * 256 threads = 4 waves (2 x 2).  A block computes a 256 x 128 output
//     tile: 256 "A rows" along the output's contiguous dimension (weights
//     side) x 128 "B rows" (token rows, or the m dimension of a weight
//     gradient).  Each wave owns 128 x 64 = 8 x 4 MFMA 16x16 tiles.
//   * LDS holds both operands K-contiguous, 64 bytes of K per row per stage
//     (16 fp32) plus 16 bytes of padding, which spreads the eight
//     rows read by consecutive lanes over distinct banks.  Two stages: the
//     next K slice is fetched into registers while the MFMAs consume the
//     current one, then stored into the other stage (one barrier per step).
//   * An operand whose source has K contiguous is copied 16 bytes per lane.
//     One whose source has the row dimension contiguous ([K][N] weights,
//     and both operands of the weight gradients) is read in 4x4 micro-blocks
//     and transposed in registers before the LDS store, so every MFMA
//     operand is one 16-byte LDS read per lane.
//   * Four v_mfma_f32_16x16x4_f32 per 16x16 tile and 64-byte K slice (full
//     fp32 products).
//     Lane l of a 16x16 accumulator holds 4 consecutive A rows
//     (4*(l/16) + 0..3) of B row l%16, so the output's contiguous
//     dimension sits on the A side and each lane stores 4 adjacent elements.
//   * The up projection puts w1 columns [f0, f0+128) in A rows 0..127 and the
//     same w3 columns in A rows 128..255, so each lane holds matching h1 and
//     h3 values and the SiLU gate is applied in the epilogue.
#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {

constexpr int kGemmThreads = 256;
constexpr int kTileA = 256;
constexpr int kTileB = 128;
constexpr int kKBytes = 64;
constexpr int kLdsRow = kKBytes + 16;
constexpr int kLdsA = kTileA * kLdsRow;
constexpr int kLdsB = kTileB * kLdsRow;
constexpr int kLdsStage = kLdsA + kLdsB;

template <typename T> struct KStep { static constexpr int elems = kKBytes / (int)sizeof(T); };

// One operand's source: tile rows [0,128) start at p0 and rows [128,256) at
// p1 (A side only).  `ld` is the byte distance between consecutive source
// rows.  For a K-contiguous source a tile row is a source row; for a
// transposed source a tile row is a source column and K runs down the rows.
struct Operand {
  const char* p0;
  const char* p1;
  int64_t ld;
  bool has1;
};

template <typename T, bool TRANS, int ROWS> struct Loader;

// K-contiguous source: 16 bytes per lane, 4 lanes per 64-byte row slice.
template <typename T, int ROWS> struct Loader<T, false, ROWS> {
  static constexpr int kChunks = ROWS * (kKBytes / 16) / kGemmThreads;
  u32x4 r[kChunks];
  __device__ __forceinline__ void load(const Operand& op, int ks, int tid) {
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
      const int c = tid + q * kGemmThreads;
      const int row = c >> 2, seg = c & 3;
      const bool hi = row >= 128;
      if (hi && !op.has1) continue;
      const char* base = hi ? op.p1 : op.p0;
      r[q] = ld16(base + (int64_t)(row & 127) * op.ld + (int64_t)ks * kKBytes + seg * 16);
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid, bool has1) const {
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
      const int c = tid + q * kGemmThreads;
      const int row = c >> 2, seg = c & 3;
      if (row >= 128 && !has1) continue;
      *reinterpret_cast<u32x4*>(lds + row * kLdsRow + seg * 16) = r[q];
    }
  }
};

// Row-contiguous fp32 source: 4 K-rows x 4 columns per thread.
template <int ROWS> struct Loader<float, true, ROWS> {
  u32x4 v[4];
  __device__ __forceinline__ bool active(bool has1, int tid) const {
    return (ROWS == 256 || tid < 128) && (tid < 128 || has1);
  }
  __device__ __forceinline__ void load(const Operand& op, int ks, int tid) {
    if (!active(op.has1, tid)) return;
    const int half = tid >> 7, mb = tid & 127, kblk = mb >> 5, nblk = mb & 31;
    const char* base = (half ? op.p1 : op.p0) +
                       (int64_t)(ks * KStep<float>::elems + kblk * 4) * op.ld + nblk * 16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) v[kk] = ld16(base + (int64_t)kk * op.ld);
  }
  __device__ __forceinline__ void store(char* lds, int tid, bool has1) const {
    if (!active(has1, tid)) return;
    const int half = tid >> 7, mb = tid & 127, kblk = mb >> 5, nblk = mb & 31;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 o = {v[0][c], v[1][c], v[2][c], v[3][c]};
      *reinterpret_cast<u32x4*>(lds + (half * 128 + nblk * 4 + c) * kLdsRow + kblk * 16) = o;
    }
  }
};

typedef f32x4 Acc[8][4];

__device__ __forceinline__ int a_row(int i, int wm) { return (i >> 2) * 128 + wm * 64 + (i & 3) * 16; }
__device__ __forceinline__ int b_row(int j, int wn) { return wn * 64 + j * 16; }

template <typename T> struct Mma;
template <> struct Mma<float> {
  __device__ __forceinline__ static void stage(Acc& acc, const char* lds, int wm, int wn,
                                               int lane, bool has1) {
    const char* la = lds;
    const char* lb = lds + kLdsA;
    const int lrow = lane & 15, lk = (lane >> 4) * 16;
    f32x4 b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const f32x4*>(lb + (b_row(j, wn) + lrow) * kLdsRow + lk);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i >= 4 && !has1) break;
      const f32x4 a = *reinterpret_cast<const f32x4*>(la + (a_row(i, wm) + lrow) * kLdsRow + lk);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[j][s], acc[i][j], 0, 0, 0);
    }
  }
};

// acc += A_tile . B_tile^T over `ksteps` 64-byte K slices.
template <typename T, bool ATR, bool BTR>
__device__ __forceinline__ void mainloop(Acc& acc, const Operand& A, const Operand& B,
                                         int ksteps, char* lds) {
  if (ksteps <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  Loader<T, ATR, kTileA> la;
  Loader<T, BTR, kTileB> lb;
  la.load(A, 0, tid);
  lb.load(B, 0, tid);
  la.store(lds, tid, A.has1);
  lb.store(lds + kLdsA, tid, false);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    char* cur = lds + (ks & 1) * kLdsStage;
    char* nxt = lds + ((ks + 1) & 1) * kLdsStage;
    const bool more = ks + 1 < ksteps;
    if (more) {
      la.load(A, ks + 1, tid);
      lb.load(B, ks + 1, tid);
    }
    Mma<T>::stage(acc, cur, wm, wn, lane, A.has1);
    if (more) {
      la.store(nxt, tid, A.has1);
      lb.store(nxt + kLdsA, tid, false);
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

template <typename T> __device__ __forceinline__ void store4(T* p, const f32x4& v);
template <> __device__ __forceinline__ void store4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <typename T> __device__ __forceinline__ f32x4 load4(const T* p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}


#define GEMM_PROLOGUE                                        \
  __shared__ __attribute__((aligned(16))) char lds[2 * kLdsStage]; \
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6; \
  const int wm = w >> 1, wn = w & 1;                         \
  const int lr = (lane >> 4) * 4, lc = lane & 15;            \
  (void)lr; (void)lc;

// h1 = x_perm w1[e], h3 = x_perm w3[e], act = silu(h1) * h3 for one 128-row
// block and 128 ffn columns.  grid = (F/128, max_tiles).
template <typename T>
__global__ void __launch_bounds__(kGemmThreads)
gemm_up_kernel(const T* __restrict__ x_perm, const T* __restrict__ w1,
               const T* __restrict__ w3, int64_t H, int64_t F,
               const int32_t* __restrict__ tile_expert, T* __restrict__ h1,
               T* __restrict__ h3, T* __restrict__ act) {
  GEMM_PROLOGUE
  const int64_t mt = blockIdx.y, f0 = (int64_t)blockIdx.x * 128;
  const int e = tile_expert[mt];
  if (e < 0) return;
  const int64_t wofs = (int64_t)e * H * F + f0;
  const Operand A{reinterpret_cast<const char*>(w1 + wofs),
                  reinterpret_cast<const char*>(w3 + wofs), F * (int64_t)sizeof(T), true};
  const Operand B{reinterpret_cast<const char*>(x_perm + mt * kBlock * H), nullptr,
                  H * (int64_t)sizeof(T), false};
  Acc acc;
  zero(acc);
  mainloop<T, true, false>(acc, A, B, (int)(H / KStep<T>::elems), lds);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = mt * kBlock + b_row(j, wn) + lc;
      const int64_t f = f0 + a_row(i, wm) + lr;
      const f32x4 v1 = acc[i][j], v3 = acc[i + 4][j];
      f32x4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = gated_silu(v1[r], v3[r]);
      store4(h1 + p * F + f, v1);
      store4(h3 + p * F + f, v3);
      store4(act + p * F + f, a);
    }
}

// y_perm = act w2[e].  grid = (ceil(H/256), max_tiles).
template <typename T>
__global__ void __launch_bounds__(kGemmThreads)
gemm_down_kernel(const T* __restrict__ act, const T* __restrict__ w2, int64_t H,
                 int64_t F, const int32_t* __restrict__ tile_expert,
                 T* __restrict__ y_perm) {
  GEMM_PROLOGUE
  const int64_t mt = blockIdx.y, h0 = (int64_t)blockIdx.x * kTileA;
  const int e = tile_expert[mt];
  if (e < 0) return;
  const T* wb = w2 + (int64_t)e * F * H + h0;
  const Operand A{reinterpret_cast<const char*>(wb), reinterpret_cast<const char*>(wb + 128),
                  H * (int64_t)sizeof(T), h0 + 128 < H};
  const Operand B{reinterpret_cast<const char*>(act + mt * kBlock * F), nullptr,
                  F * (int64_t)sizeof(T), false};
  Acc acc;
  zero(acc);
  mainloop<T, true, false>(acc, A, B, (int)(F / KStep<T>::elems), lds);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i >= 4 && !A.has1) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = mt * kBlock + b_row(j, wn) + lc;
      store4(y_perm + p * H + h0 + a_row(i, wm) + lr, acc[i][j]);
    }
  }
}

// dA = dy_perm w2[e]^T, then the gate's backward:
// dh3 = dA * silu(h1), dh1 = dA * h3 * s * (1 + h1 (1 - s)), s = sigmoid(h1).
// grid = (ceil(F/256), max_tiles).
template <typename T>
__global__ void __launch_bounds__(kGemmThreads)
gemm_down_dgrad_kernel(const T* __restrict__ dy_perm, const T* __restrict__ w2,
                       const T* h1, const T* h3, int64_t H, int64_t F,
                       const int32_t* __restrict__ tile_expert, T* dh1, T* dh3) {
  GEMM_PROLOGUE
  const int64_t mt = blockIdx.y, fb = (int64_t)blockIdx.x * kTileA;
  const int e = tile_expert[mt];
  if (e < 0) return;
  const T* wb = w2 + (int64_t)e * F * H + fb * H;
  const Operand A{reinterpret_cast<const char*>(wb), reinterpret_cast<const char*>(wb + 128 * H),
                  H * (int64_t)sizeof(T), fb + 128 < F};
  const Operand B{reinterpret_cast<const char*>(dy_perm + mt * kBlock * H), nullptr,
                  H * (int64_t)sizeof(T), false};
  Acc acc;
  zero(acc);
  mainloop<T, false, false>(acc, A, B, (int)(H / KStep<T>::elems), lds);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i >= 4 && !A.has1) break;
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

// dx_perm = dh1 w1[e]^T + dh3 w3[e]^T.  grid = (ceil(H/256), max_tiles).
template <typename T>
__global__ void __launch_bounds__(kGemmThreads)
gemm_up_dgrad_kernel(const T* __restrict__ dh1, const T* __restrict__ dh3,
                     const T* __restrict__ w1, const T* __restrict__ w3, int64_t H,
                     int64_t F, const int32_t* __restrict__ tile_expert,
                     T* dx_perm) {
  GEMM_PROLOGUE
  const int64_t mt = blockIdx.y, h0 = (int64_t)blockIdx.x * kTileA;
  const int e = tile_expert[mt];
  if (e < 0) return;
  const int64_t wofs = (int64_t)e * H * F + h0 * F;
  const bool has1 = h0 + 128 < H;
  const int ks = (int)(F / KStep<T>::elems);
  Acc acc;
  zero(acc);
  {
    const Operand A{reinterpret_cast<const char*>(w1 + wofs),
                    reinterpret_cast<const char*>(w1 + wofs + 128 * F), F * (int64_t)sizeof(T), has1};
    const Operand B{reinterpret_cast<const char*>(dh1 + mt * kBlock * F), nullptr,
                    F * (int64_t)sizeof(T), false};
    mainloop<T, false, false>(acc, A, B, ks, lds);
  }
  {
    const Operand A{reinterpret_cast<const char*>(w3 + wofs),
                    reinterpret_cast<const char*>(w3 + wofs + 128 * F), F * (int64_t)sizeof(T), has1};
    const Operand B{reinterpret_cast<const char*>(dh3 + mt * kBlock * F), nullptr,
                    F * (int64_t)sizeof(T), false};
    mainloop<T, false, false>(acc, A, B, ks, lds);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i >= 4 && !has1) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = mt * kBlock + b_row(j, wn) + lc;
      store4(dx_perm + p * H + h0 + a_row(i, wm) + lr, acc[i][j]);
    }
  }
}

__device__ __forceinline__ void expert_rows(int e, const int32_t* tpe,
                                            const int32_t* padded_bins,
                                            int64_t& start, int& n) {
  n = round_up_block(tpe[e]);
  start = padded_bins[e] - n;
}

// dw2[e] = act[rows_e]^T dy_perm[rows_e]  ([F,H]); zero for an empty expert.
// grid = (ceil(H/256), F/128, E).
template <typename T>
__global__ void __launch_bounds__(kGemmThreads)
gemm_wgrad_down_kernel(const T* __restrict__ act, const T* __restrict__ dy_perm,
                       int64_t H, int64_t F, const int32_t* __restrict__ tpe,
                       const int32_t* __restrict__ padded_bins, T* __restrict__ dw2) {
  GEMM_PROLOGUE
  const int64_t h0 = (int64_t)blockIdx.x * kTileA, f0 = (int64_t)blockIdx.y * 128;
  const int e = blockIdx.z;
  int64_t start;
  int n;
  expert_rows(e, tpe, padded_bins, start, n);
  const T* ab = dy_perm + start * H + h0;
  const Operand A{reinterpret_cast<const char*>(ab), reinterpret_cast<const char*>(ab + 128),
                  H * (int64_t)sizeof(T), h0 + 128 < H};
  const Operand B{reinterpret_cast<const char*>(act + start * F + f0), nullptr,
                  F * (int64_t)sizeof(T), false};
  Acc acc;
  zero(acc);
  mainloop<T, true, true>(acc, A, B, n / KStep<T>::elems, lds);
  T* out = dw2 + (int64_t)e * F * H;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i >= 4 && !A.has1) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t f = f0 + b_row(j, wn) + lc;
      store4(out + f * H + h0 + a_row(i, wm) + lr, acc[i][j]);
    }
  }
}

// dw1[e] = x_perm[rows_e]^T dh1[rows_e], dw3[e] = x_perm[rows_e]^T dh3[rows_e]
// ([H,F] each); zero for an empty expert.  grid = (F/128, H/128, E).
template <typename T>
__global__ void __launch_bounds__(kGemmThreads)
gemm_wgrad_up_kernel(const T* __restrict__ x_perm, const T* __restrict__ dh1,
                     const T* __restrict__ dh3, int64_t H, int64_t F,
                     const int32_t* __restrict__ tpe,
                     const int32_t* __restrict__ padded_bins, T* __restrict__ dw1,
                     T* __restrict__ dw3) {
  GEMM_PROLOGUE
  const int64_t f0 = (int64_t)blockIdx.x * 128, h0 = (int64_t)blockIdx.y * 128;
  const int e = blockIdx.z;
  int64_t start;
  int n;
  expert_rows(e, tpe, padded_bins, start, n);
  const Operand A{reinterpret_cast<const char*>(dh1 + start * F + f0),
                  reinterpret_cast<const char*>(dh3 + start * F + f0), F * (int64_t)sizeof(T), true};
  const Operand B{reinterpret_cast<const char*>(x_perm + start * H + h0), nullptr,
                  H * (int64_t)sizeof(T), false};
  Acc acc;
  zero(acc);
  mainloop<T, true, true>(acc, A, B, n / KStep<T>::elems, lds);
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

static unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

template <typename T> static const T* cp(const void* p) { return static_cast<const T*>(p); }
template <typename T> static T* mp(void* p) { return static_cast<T*>(p); }

hipError_t launch_gemm_up(const Shape& s, const void* x_perm, const void* x, const void* w1,
                          const void* w3, const MetaPtrs& m, void* h1, void* h3,
                          void* act, hipStream_t stream) {
  const dim3 grid(cdiv(s.F, 128), (unsigned)s.max_tiles);
  if (s.bf16) return launch_bf16_up(s, x_perm, x, w1, w3, m, h1, h3, act, stream);
  if (x) return hipErrorNotSupported;   // rows from x: bf16 engine only
  hipLaunchKernelGGL(gemm_up_kernel<float>, grid, dim3(kGemmThreads), 0, stream,
                     cp<float>(x_perm), cp<float>(w1), cp<float>(w3), s.H, s.F,
                     m.tile_expert, mp<float>(h1), mp<float>(h3), mp<float>(act));
  return hipGetLastError();
}

hipError_t launch_gemm_down(const Shape& s, const void* act, const void* w2,
                            const MetaPtrs& m, void* y_perm, hipStream_t stream) {
  const dim3 grid(cdiv(s.H, kTileA), (unsigned)s.max_tiles);
  if (s.bf16) return launch_bf16_down(s, act, w2, m, y_perm, stream);
  hipLaunchKernelGGL(gemm_down_kernel<float>, grid, dim3(kGemmThreads), 0, stream,
                     cp<float>(act), cp<float>(w2), s.H, s.F, m.tile_expert,
                     mp<float>(y_perm));
  return hipGetLastError();
}

static hipError_t f32_down_dgrad(const Shape& s, const void* dy_perm, const void* w2,
                                 const void* h1, const void* h3, const MetaPtrs& m, void* dh1,
                                 void* dh3, hipStream_t stream) {
  const dim3 grid(cdiv(s.F, kTileA), (unsigned)s.max_tiles);
  hipLaunchKernelGGL(gemm_down_dgrad_kernel<float>, grid, dim3(kGemmThreads), 0, stream,
                     cp<float>(dy_perm), cp<float>(w2), cp<float>(h1), cp<float>(h3),
                     s.H, s.F, m.tile_expert, mp<float>(dh1), mp<float>(dh3));
  return hipGetLastError();
}

static hipError_t f32_wgrad_down(const Shape& s, const void* act, const void* dy_perm,
                                 const MetaPtrs& m, void* dw2, hipStream_t stream) {
  const dim3 grid(cdiv(s.H, kTileA), cdiv(s.F, 128), (unsigned)s.E);
  hipLaunchKernelGGL(gemm_wgrad_down_kernel<float>, grid, dim3(kGemmThreads), 0, stream,
                     cp<float>(act), cp<float>(dy_perm), s.H, s.F, m.tokens_per_expert,
                     m.padded_bins, mp<float>(dw2));
  return hipGetLastError();
}

hipError_t launch_gemm_down_dgrad_wgrad_down(const Shape& s, const void* dy_perm,
                                             const void* w2, const void* h1, const void* h3,
                                             const void* act, const MetaPtrs& m, void* dh1,
                                             void* dh3, void* dw2, hipStream_t stream) {
  if (s.bf16)
    return launch_bf16_down_dgrad_wgrad_down(s, dy_perm, w2, h1, h3, act, m, dh1, dh3, dw2,
                                             stream);
  const hipError_t err = f32_down_dgrad(s, dy_perm, w2, h1, h3, m, dh1, dh3, stream);
  if (err != hipSuccess) return err;
  return f32_wgrad_down(s, act, dy_perm, m, dw2, stream);
}

hipError_t launch_gemm_up_dgrad(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const void* x_perm,
                                const MetaPtrs& m, void* dx_perm, void* dw1, void* dw3,
                                hipStream_t stream) {
  if (s.bf16)
    return launch_bf16_up_dgrad(s, dh1, dh3, w1, w3, x_perm, m, dx_perm, dw1, dw3, stream);
  const dim3 grid(cdiv(s.H, kTileA), (unsigned)s.max_tiles);
  hipLaunchKernelGGL(gemm_up_dgrad_kernel<float>, grid, dim3(kGemmThreads), 0, stream,
                     cp<float>(dh1), cp<float>(dh3), cp<float>(w1), cp<float>(w3), s.H,
                     s.F, m.tile_expert, mp<float>(dx_perm));
  return hipGetLastError();
}

hipError_t launch_gemm_wgrad_up(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const void* x_perm,
                                const MetaPtrs& m, void* dx_perm, void* dw1, void* dw3,
                                hipStream_t stream) {
  if (s.bf16)
    return launch_bf16_wgrad_up(s, dh1, dh3, w1, w3, x_perm, m, dx_perm, dw1, dw3, stream);
  const dim3 grid(cdiv(s.F, 128), cdiv(s.H, 128), (unsigned)s.E);
  hipLaunchKernelGGL(gemm_wgrad_up_kernel<float>, grid, dim3(kGemmThreads), 0, stream,
                     cp<float>(x_perm), cp<float>(dh1), cp<float>(dh3), s.H, s.F,
                     m.tokens_per_expert, m.padded_bins, mp<float>(dw1), mp<float>(dw3));
  return hipGetLastError();
}

}  // namespace dmoe
