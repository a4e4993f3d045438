// Grouped GEMM over expert-tagged 128-row blocks (gfx950 MFMA), fp32.  The
// launch_gemm_* entry points below route bf16 to the engine of
// gemm_bf16.hip; the kernels of this file run the fp32 layer.
//
// MegaBlocks chapter "02 · dropless MoE 与 block-sparse 重构" §2-§3: once each
// expert's rows are padded to a multiple of 128, every 128-row block of the
// padded token matrix belongs to one expert, so the expert FFN is a block-
// sparse product whose non-zero blocks are exactly (row block r, the columns
// of expert tile_expert[r]).  The sdd product (x_perm w1, x_perm w3) and the
// dsd product (act w2) are computed here as one launch each over all row
// blocks, each tile reading its own expert's weights; §5's GLU variant
// shares the row-block -> expert map.  The backward products (dgrad of both
// projections and the per-expert weight gradients, whose contraction runs
// over the expert's padded row range) use the same tile engine.
//
// Tile engine.  The fp32 layer is small (its products are a few hundred
// MFLOP), so tiles are small too, to spread one product over many CUs:
//   * 256 threads = 4 waves (2 x 2).  A block computes a 64 x 64 output
//     tile: 64 "A rows" along the output's contiguous dimension (weights
//     side) x 64 "B rows" (token rows, or the m dimension of a weight
//     gradient).  The A rows are two halves of 32 from two sources (w1 and
//     w3 columns in the up projection, so the SiLU gate pairs them in
//     registers; consecutive columns elsewhere).  Each wave owns 16 rows of
//     each A half x 32 B rows: 2 x 2 MFMA 16x16 tiles.  A launch whose 64 x
//     64 tiles would leave CUs without one computes the first A half alone
//     (32 x 64 tiles, twice as many; the down projection, the up dgrad and
//     the merged down dgrad + dw2).
//   * LDS holds both operands K-contiguous, 128 bytes of K per row per stage
//     (32 fp32) plus 16 bytes of padding, which spreads the rows read by
//     consecutive lanes over distinct banks.  32 K per stage halves the
//     number of steps, each of which waits once for its global loads.  Two stages: the next K slice
//     is fetched into registers while the MFMAs consume the current one,
//     then stored into the other stage (one barrier per step).
//   * An operand whose source has K contiguous is copied 16 bytes per lane.
//     One whose source has the row dimension contiguous ([K][N] weights,
//     and both operands of the weight gradients) is read in 4x4 micro-blocks
//     and transposed in registers before the LDS store, so every MFMA
//     operand is one 16-byte LDS read per lane.
//   * Four v_mfma_f32_16x16x4_f32 per 16x16 tile and 64-byte K slice (full
//     fp32 products).  Lane l of a 16x16 accumulator holds 4 consecutive A
//     rows (4*(l/16) + 0..3) of B row l%16, so the output's contiguous
//     dimension sits on the A side and each lane stores 4 adjacent elements.
#include <atomic>

#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {

constexpr int kGemmThreads = 256;
constexpr int kTileA = 64;                 // A rows: two halves of kHalfA
constexpr int kHalfA = kTileA / 2;
constexpr int kTileB = 64;                 // B rows, from one source
constexpr int kKElems = 32;                // fp32 K per stage
constexpr int kKBytes = kKElems * 4;
constexpr int kLdsRow = kKBytes + 16;
constexpr int kLdsA = kTileA * kLdsRow;
constexpr int kLdsB = kTileB * kLdsRow;
constexpr int kLdsStage = kLdsA + kLdsB;
constexpr int kBPerBlock = kBlock / kTileB;   // B tiles per 128-row block

// One operand's source.  A: tile rows [0, half) start at p0 and rows
// [half, 2 half) at p1 (present when has1).  B: all rows from p0 (half =
// kTileB).  `ld` is the byte distance between consecutive source rows.  For
// a K-contiguous source a tile row is a source row; for a transposed source
// a tile row is a source column and K runs down the rows.
struct Operand {
  const char* p0;
  const char* p1;
  int64_t ld;
  int half;
  bool has1;
};

template <bool TRANS, int ROWS> struct Loader;

// K-contiguous source: 16 bytes per lane, 4 lanes per 64-byte row slice.
template <int ROWS> struct Loader<false, ROWS> {
  static constexpr int kSegs = kKBytes / 16;                 // 16-byte segments per row
  static constexpr int kChunks = ROWS * kSegs / kGemmThreads;
  static_assert(kChunks >= 1 && ROWS * kSegs % kGemmThreads == 0, "tile/block mismatch");
  u32x4 r[kChunks];
  __device__ __forceinline__ bool live(const Operand& op, int row) const {
    return row < op.half || op.has1;
  }
  __device__ __forceinline__ void load(const Operand& op, int ks, int tid) {
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
      const int c = tid + q * kGemmThreads;
      const int row = c / kSegs, seg = c % kSegs;
      if (!live(op, row)) continue;
      const char* base = row < op.half ? op.p0 + (int64_t)row * op.ld
                                       : op.p1 + (int64_t)(row - op.half) * op.ld;
      r[q] = ld16(base + (int64_t)ks * kKBytes + seg * 16);
    }
  }
  __device__ __forceinline__ void store(char* lds, const Operand& op, int tid) const {
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
      const int c = tid + q * kGemmThreads;
      const int row = c / kSegs, seg = c % kSegs;
      if (!live(op, row)) continue;
      *reinterpret_cast<u32x4*>(lds + row * kLdsRow + seg * 16) = r[q];
    }
  }
};

// Row-contiguous source: thread t reads 4 K-rows x 4 columns (16 bytes per
// K-row) and writes 4 LDS rows of 4 consecutive K values.
template <int ROWS> struct Loader<true, ROWS> {
  static constexpr int kNBlk = ROWS / 4;      // 4-column blocks per K-row
  static constexpr int kThreads = kNBlk * (kKElems / 4);
  static_assert(kThreads <= kGemmThreads, "one micro-block per thread");
  u32x4 v[4];
  __device__ __forceinline__ bool active(const Operand& op, int tid) const {
    return tid < kThreads && ((tid % kNBlk) * 4 < op.half || op.has1);
  }
  __device__ __forceinline__ void load(const Operand& op, int ks, int tid) {
    if (!active(op, tid)) return;
    const int kblk = tid / kNBlk, n0 = (tid % kNBlk) * 4;
    const char* col = n0 < op.half ? op.p0 + n0 * 4 : op.p1 + (n0 - op.half) * 4;
    const char* base = col + (int64_t)(ks * kKElems + kblk * 4) * op.ld;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) v[kk] = ld16(base + (int64_t)kk * op.ld);
  }
  __device__ __forceinline__ void store(char* lds, const Operand& op, int tid) const {
    if (!active(op, tid)) return;
    const int kblk = tid / kNBlk, n0 = (tid % kNBlk) * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 o = {v[0][c], v[1][c], v[2][c], v[3][c]};
      *reinterpret_cast<u32x4*>(lds + (n0 + c) * kLdsRow + kblk * 16) = o;
    }
  }
};

typedef f32x4 Acc[2][2];

// 16-row subtiles of wave (wm, wn): A subtile i in A half i, B subtile j.
__device__ __forceinline__ int a_row(int i, int wm) { return i * kHalfA + wm * 16; }
__device__ __forceinline__ int b_row(int j, int wn) { return wn * 32 + j * 16; }

__device__ __forceinline__ void mma_stage(Acc& acc, const char* lds, int wm, int wn, int lane,
                                          bool has1) {
  const char* la = lds;
  const char* lb = lds + kLdsA;
  const int lrow = lane & 15;
#pragma unroll
  for (int kk = 0; kk < kKElems / 16; ++kk) {
    // lanes of group l/16 hold K 16 kk + 4 (l/16) + 0..3; MFMA s takes the
    // s-th of them, so the four MFMAs cover the 16 K of this sub-step
    const int lk = kk * 64 + (lane >> 4) * 16;
    f32x4 b[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *reinterpret_cast<const f32x4*>(lb + (b_row(j, wn) + lrow) * kLdsRow + lk);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i == 1 && !has1) break;
      const f32x4 a = *reinterpret_cast<const f32x4*>(la + (a_row(i, wm) + lrow) * kLdsRow + lk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[j][s], acc[i][j], 0, 0, 0);
    }
  }
}

// acc += A_tile . B_tile^T over `ksteps` K slices of kKElems.
template <bool ATR, bool BTR>
__device__ __forceinline__ void mainloop(Acc& acc, const Operand& A, const Operand& B,
                                         int ksteps, char* lds) {
  if (ksteps <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  Loader<ATR, kTileA> la;
  Loader<BTR, kTileB> lb;
  la.load(A, 0, tid);
  lb.load(B, 0, tid);
  la.store(lds, A, tid);
  lb.store(lds + kLdsA, B, tid);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    char* cur = lds + (ks & 1) * kLdsStage;
    char* nxt = lds + ((ks + 1) & 1) * kLdsStage;
    const bool more = ks + 1 < ksteps;
    if (more) {
      la.load(A, ks + 1, tid);
      lb.load(B, ks + 1, tid);
    }
    mma_stage(acc, cur, wm, wn, lane, A.has1);
    if (more) {
      la.store(nxt, A, tid);
      lb.store(nxt + kLdsA, B, tid);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void zero(Acc& acc) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ void store4(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
__device__ __forceinline__ f32x4 load4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

#define GEMM_PROLOGUE                                                \
  __shared__ __attribute__((aligned(16))) char lds[2 * kLdsStage];   \
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;        \
  const int wm = w >> 1, wn = w & 1;                                 \
  const int lr = (lane >> 4) * 4, lc = lane & 15;                    \
  (void)lr; (void)lc;

// The B tile of the row-block products: 64 rows of a 128-row block.
__device__ __forceinline__ bool row_tile(const int32_t* tile_expert, int64_t& p0, int& e) {
  const int64_t bt = blockIdx.y;
  e = tile_expert[bt / kBPerBlock];
  p0 = bt * kTileB;
  return e >= 0;
}

// h1 = x_perm w1[e], h3 = x_perm w3[e], act = silu(h1) * h3 for 64 rows and
// 32 ffn columns (w1 columns in A half 0, the same w3 columns in A half 1).
// grid = (F/32, 2 max_tiles).
__global__ void __launch_bounds__(kGemmThreads)
gemm_up_kernel(const float* __restrict__ x_perm, const float* __restrict__ w1,
               const float* __restrict__ w3, int64_t H, int64_t F,
               const int32_t* __restrict__ tile_expert, float* __restrict__ h1,
               float* __restrict__ h3, float* __restrict__ act) {
  GEMM_PROLOGUE
  int64_t p0;
  int e;
  if (!row_tile(tile_expert, p0, e)) return;
  const int64_t f0 = (int64_t)blockIdx.x * kHalfA;
  const int64_t wofs = (int64_t)e * H * F + f0;
  const Operand A{reinterpret_cast<const char*>(w1 + wofs),
                  reinterpret_cast<const char*>(w3 + wofs), F * 4, kHalfA, true};
  const Operand B{reinterpret_cast<const char*>(x_perm + p0 * H), nullptr, H * 4, kTileB, false};
  Acc acc;
  zero(acc);
  mainloop<true, false>(acc, A, B, (int)(H / kKElems), lds);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t p = p0 + b_row(j, wn) + lc;
    const int64_t f = f0 + a_row(0, wm) + lr;
    const f32x4 v1 = acc[0][j], v3 = acc[1][j];
    f32x4 a;
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = gated_silu(v1[r], v3[r]);
    store4(h1 + p * F + f, v1);
    store4(h3 + p * F + f, v3);
    store4(act + p * F + f, a);
  }
}

// y_perm = act w2[e] for 64 rows and 64 hidden columns, or 32 when `narrow`
// (only the first A half: twice the tiles for a product too small to fill
// the CUs).  grid = (H/64 or H/32, 2 max_tiles).
__global__ void __launch_bounds__(kGemmThreads)
gemm_down_kernel(const float* __restrict__ act, const float* __restrict__ w2, int64_t H,
                 int64_t F, const int32_t* __restrict__ tile_expert, int narrow,
                 float* __restrict__ y_perm) {
  GEMM_PROLOGUE
  int64_t p0;
  int e;
  if (!row_tile(tile_expert, p0, e)) return;
  const int64_t h0 = (int64_t)blockIdx.x * (narrow ? kHalfA : kTileA);
  const float* wb = w2 + (int64_t)e * F * H + h0;
  const Operand A{reinterpret_cast<const char*>(wb), reinterpret_cast<const char*>(wb + kHalfA),
                  H * 4, kHalfA, !narrow && h0 + kHalfA < H};
  const Operand B{reinterpret_cast<const char*>(act + p0 * F), nullptr, F * 4, kTileB, false};
  Acc acc;
  zero(acc);
  mainloop<true, false>(acc, A, B, (int)(F / kKElems), lds);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i == 1 && !A.has1) break;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t p = p0 + b_row(j, wn) + lc;
      store4(y_perm + p * H + h0 + a_row(i, wm) + lr, acc[i][j]);
    }
  }
}

// dA = dy_perm w2[e]^T, then the gate's backward:
// dh3 = dA * silu(h1), dh1 = dA * h3 * s * (1 + h1 (1 - s)), s = sigmoid(h1).
// 64 rows and 64 ffn columns.
// (bx, by): the tile's grid coordinates.
__device__ __forceinline__ void down_dgrad_tile(const float* __restrict__ dy_perm,
                                                const float* __restrict__ w2, const float* h1,
                                                const float* h3, int64_t H, int64_t F,
                                                const int32_t* __restrict__ tile_expert,
                                                float* dh1, float* dh3, int bx, int by,
                                                bool narrow, char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wn = w & 1, wm = w >> 1;
  const int lr = (lane >> 4) * 4, lc = lane & 15;
  const int e = tile_expert[by / kBPerBlock];
  if (e < 0) return;
  const int64_t p0 = (int64_t)by * kTileB;
  const int64_t fb = (int64_t)bx * (narrow ? kHalfA : kTileA);
  const float* wb = w2 + (int64_t)e * F * H + fb * H;
  const Operand A{reinterpret_cast<const char*>(wb),
                  reinterpret_cast<const char*>(wb + kHalfA * H), H * 4, kHalfA,
                  !narrow && fb + kHalfA < F};
  const Operand B{reinterpret_cast<const char*>(dy_perm + p0 * H), nullptr, H * 4, kTileB, false};
  Acc acc;
  zero(acc);
  mainloop<false, false>(acc, A, B, (int)(H / kKElems), lds);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i == 1 && !A.has1) break;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t p = p0 + b_row(j, wn) + lc;
      const int64_t o = p * F + fb + a_row(i, wm) + lr;
      const f32x4 g1 = load4(h1 + o), g3 = load4(h3 + o);
      f32x4 d1, d3;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float da = acc[i][j][r];
        const float s = sigmoid(g1[r]);
        d3[r] = da * g1[r] * s;
        d1[r] = da * g3[r] * s * (1.0f + g1[r] * (1.0f - s));
      }
      store4(dh1 + o, d1);
      store4(dh3 + o, d3);
    }
  }
}

// dx_perm = dh1 w1[e]^T + dh3 w3[e]^T for 64 rows and 64 hidden columns.
// grid = (H/64, 2 max_tiles).
__global__ void __launch_bounds__(kGemmThreads)
gemm_up_dgrad_kernel(const float* __restrict__ dh1, const float* __restrict__ dh3,
                     const float* __restrict__ w1, const float* __restrict__ w3, int64_t H,
                     int64_t F, const int32_t* __restrict__ tile_expert, int narrow,
                     float* dx_perm) {
  GEMM_PROLOGUE
  int64_t p0;
  int e;
  if (!row_tile(tile_expert, p0, e)) return;
  const int64_t h0 = (int64_t)blockIdx.x * (narrow ? kHalfA : kTileA);
  const int64_t wofs = (int64_t)e * H * F + h0 * F;
  const bool has1 = !narrow && h0 + kHalfA < H;
  const int ks = (int)(F / kKElems);
  Acc acc;
  zero(acc);
  {
    const Operand A{reinterpret_cast<const char*>(w1 + wofs),
                    reinterpret_cast<const char*>(w1 + wofs + kHalfA * F), F * 4, kHalfA, has1};
    const Operand B{reinterpret_cast<const char*>(dh1 + p0 * F), nullptr, F * 4, kTileB, false};
    mainloop<false, false>(acc, A, B, ks, lds);
  }
  {
    const Operand A{reinterpret_cast<const char*>(w3 + wofs),
                    reinterpret_cast<const char*>(w3 + wofs + kHalfA * F), F * 4, kHalfA, has1};
    const Operand B{reinterpret_cast<const char*>(dh3 + p0 * F), nullptr, F * 4, kTileB, false};
    mainloop<false, false>(acc, A, B, ks, lds);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i == 1 && !has1) break;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t p = p0 + b_row(j, wn) + lc;
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
// 64 ffn x 64 hidden columns; (bx, by, e): the tile's grid coordinates.
__device__ __forceinline__ void wgrad_down_tile(const float* __restrict__ act,
                                                const float* __restrict__ dy_perm, int64_t H,
                                                int64_t F, const int32_t* __restrict__ tpe,
                                                const int32_t* __restrict__ padded_bins,
                                                float* __restrict__ dw2, int bx, int by, int e,
                                                bool narrow, char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wn = w & 1, wm = w >> 1;
  const int lr = (lane >> 4) * 4, lc = lane & 15;
  const int64_t h0 = (int64_t)bx * (narrow ? kHalfA : kTileA), f0 = (int64_t)by * kTileB;
  int64_t start;
  int n;
  expert_rows(e, tpe, padded_bins, start, n);
  const float* ab = dy_perm + start * H + h0;
  const Operand A{reinterpret_cast<const char*>(ab), reinterpret_cast<const char*>(ab + kHalfA),
                  H * 4, kHalfA, !narrow && h0 + kHalfA < H};
  const Operand B{reinterpret_cast<const char*>(act + start * F + f0), nullptr, F * 4, kTileB,
                  false};
  Acc acc;
  zero(acc);
  mainloop<true, true>(acc, A, B, n / kKElems, lds);
  float* out = dw2 + (int64_t)e * F * H;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i == 1 && !A.has1) break;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t f = f0 + b_row(j, wn) + lc;
      store4(out + f * H + h0 + a_row(i, wm) + lr, acc[i][j]);
    }
  }
}

// down dgrad + gate backward and dw2 in one launch (neither reads what the
// other writes): blocks [0, nd) are dgrad tiles ((F/cw) x (2 max_tiles),
// x fastest), the rest dw2 tiles ((H/cw) x (F/64) x E), with cw = 64
// columns, or 32 (the first A half) when `narrow`.
__global__ void __launch_bounds__(kGemmThreads)
gemm_down_dgrad_wgrad_down_kernel(const float* __restrict__ dy_perm,
                                  const float* __restrict__ w2, const float* h1,
                                  const float* h3, const float* __restrict__ act, int64_t H,
                                  int64_t F, const int32_t* __restrict__ tile_expert,
                                  const int32_t* __restrict__ tpe,
                                  const int32_t* __restrict__ padded_bins, float* dh1,
                                  float* dh3, float* __restrict__ dw2, int nd, int narrow) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kLdsStage];
  const int b = (int)blockIdx.x;
  const int cw = narrow ? kHalfA : kTileA;
  if (b < nd) {
    const int fx = (int)((F + cw - 1) / cw);
    down_dgrad_tile(dy_perm, w2, h1, h3, H, F, tile_expert, dh1, dh3, b % fx, b / fx,
                    narrow != 0, lds);
  } else {
    const int hx = (int)((H + cw - 1) / cw), fy = (int)((F + kTileB - 1) / kTileB);
    const int r = b - nd;
    wgrad_down_tile(act, dy_perm, H, F, tpe, padded_bins, dw2, r % hx, (r / hx) % fy,
                    r / (hx * fy), narrow != 0, lds);
  }
}

// dw1[e] = x_perm[rows_e]^T dh1[rows_e], dw3[e] = x_perm[rows_e]^T dh3[rows_e]
// ([H,F] each); zero for an empty expert.  32 ffn columns of each (A halves)
// x 64 hidden rows.  grid = (F/32, H/64, E).
__global__ void __launch_bounds__(kGemmThreads)
gemm_wgrad_up_kernel(const float* __restrict__ x_perm, const float* __restrict__ dh1,
                     const float* __restrict__ dh3, int64_t H, int64_t F,
                     const int32_t* __restrict__ tpe,
                     const int32_t* __restrict__ padded_bins, float* __restrict__ dw1,
                     float* __restrict__ dw3) {
  GEMM_PROLOGUE
  const int64_t f0 = (int64_t)blockIdx.x * kHalfA, h0 = (int64_t)blockIdx.y * kTileB;
  const int e = blockIdx.z;
  int64_t start;
  int n;
  expert_rows(e, tpe, padded_bins, start, n);
  const Operand A{reinterpret_cast<const char*>(dh1 + start * F + f0),
                  reinterpret_cast<const char*>(dh3 + start * F + f0), F * 4, kHalfA, true};
  const Operand B{reinterpret_cast<const char*>(x_perm + start * H + h0), nullptr, H * 4,
                  kTileB, false};
  Acc acc;
  zero(acc);
  mainloop<true, true>(acc, A, B, n / kKElems, lds);
  const int64_t eo = (int64_t)e * H * F;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t h = h0 + b_row(j, wn) + lc;
      const int64_t f = f0 + a_row(0, wm) + lr;
      store4((i == 0 ? dw1 : dw3) + eo + h * F + f, acc[i][j]);
    }
}

static unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// Whether a launch of cols x rows 64-column tiles should run 32-column tiles
// instead: when its 64-column tiles would not give every CU of the current
// device one.  Each output element is summed in the same order either way.
static bool narrow_tiles(unsigned cols, unsigned rows) {
  static std::atomic<int> cache[64];   // compute units per device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev].store(cus, std::memory_order_relaxed);
  }
  return (int64_t)cols * rows < (int64_t)cus;
}

template <typename T> static const T* cp(const void* p) { return static_cast<const T*>(p); }
template <typename T> static T* mp(void* p) { return static_cast<T*>(p); }

// B tiles of the row-block products: kBPerBlock per 128-row block.
static unsigned row_tiles(const Shape& s) { return (unsigned)(s.max_tiles * kBPerBlock); }

hipError_t launch_gemm_up(const Shape& s, const void* x_perm, const void* x, const void* w1,
                          const void* w3, const MetaPtrs& m, void* h1, void* h3,
                          void* act, hipStream_t stream) {
  if (s.bf16) return launch_bf16_up(s, x_perm, x, w1, w3, m, h1, h3, act, stream);
  if (x) return hipErrorNotSupported;   // rows from x: bf16 engine only
  const dim3 grid(cdiv(s.F, kHalfA), row_tiles(s));
  hipLaunchKernelGGL(gemm_up_kernel, grid, dim3(kGemmThreads), 0, stream,
                     cp<float>(x_perm), cp<float>(w1), cp<float>(w3), s.H, s.F,
                     m.tile_expert, mp<float>(h1), mp<float>(h3), mp<float>(act));
  return hipGetLastError();
}

hipError_t launch_gemm_down(const Shape& s, const void* act, const void* w2,
                            const MetaPtrs& m, void* y_perm, hipStream_t stream) {
  if (s.bf16) return launch_bf16_down(s, act, w2, m, y_perm, stream);
  const bool narrow = narrow_tiles(cdiv(s.H, kTileA), row_tiles(s));
  const dim3 grid(cdiv(s.H, narrow ? kHalfA : kTileA), row_tiles(s));
  hipLaunchKernelGGL(gemm_down_kernel, grid, dim3(kGemmThreads), 0, stream,
                     cp<float>(act), cp<float>(w2), s.H, s.F, m.tile_expert, narrow ? 1 : 0,
                     mp<float>(y_perm));
  return hipGetLastError();
}

hipError_t launch_gemm_down_dgrad_wgrad_down(const Shape& s, const void* dy_perm,
                                             const void* w2, const void* h1, const void* h3,
                                             const void* act, const MetaPtrs& m, void* dh1,
                                             void* dh3, void* dw2, hipStream_t stream) {
  if (s.bf16)
    return launch_bf16_down_dgrad_wgrad_down(s, dy_perm, w2, h1, h3, act, m, dh1, dh3, dw2,
                                             stream);
  const bool narrow = narrow_tiles(cdiv(s.F, kTileA) * row_tiles(s) +
                                       cdiv(s.H, kTileA) * cdiv(s.F, kTileB) * (unsigned)s.E,
                                   1);
  const int64_t cw = narrow ? kHalfA : kTileA;
  const unsigned nd = cdiv(s.F, cw) * row_tiles(s);
  const unsigned nw = cdiv(s.H, cw) * cdiv(s.F, kTileB) * (unsigned)s.E;
  hipLaunchKernelGGL(gemm_down_dgrad_wgrad_down_kernel, dim3(nd + nw), dim3(kGemmThreads), 0,
                     stream, cp<float>(dy_perm), cp<float>(w2), cp<float>(h1), cp<float>(h3),
                     cp<float>(act), s.H, s.F, m.tile_expert, m.tokens_per_expert,
                     m.padded_bins, mp<float>(dh1), mp<float>(dh3), mp<float>(dw2), (int)nd,
                     narrow ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_gemm_up_dgrad(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const void* x_perm,
                                const MetaPtrs& m, void* dx_perm, void* dw1, void* dw3,
                                hipStream_t stream) {
  if (s.bf16)
    return launch_bf16_up_dgrad(s, dh1, dh3, w1, w3, x_perm, m, dx_perm, dw1, dw3, stream);
  const bool narrow = narrow_tiles(cdiv(s.H, kTileA), row_tiles(s));
  const dim3 grid(cdiv(s.H, narrow ? kHalfA : kTileA), row_tiles(s));
  hipLaunchKernelGGL(gemm_up_dgrad_kernel, grid, dim3(kGemmThreads), 0, stream,
                     cp<float>(dh1), cp<float>(dh3), cp<float>(w1), cp<float>(w3), s.H,
                     s.F, m.tile_expert, narrow ? 1 : 0, mp<float>(dx_perm));
  return hipGetLastError();
}

hipError_t launch_gemm_wgrad_up(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const void* x_perm,
                                const MetaPtrs& m, void* dx_perm, void* dw1, void* dw3,
                                hipStream_t stream) {
  if (s.bf16)
    return launch_bf16_wgrad_up(s, dh1, dh3, w1, w3, x_perm, m, dx_perm, dw1, dw3, stream);
  const dim3 grid(cdiv(s.F, kHalfA), cdiv(s.H, kTileB), (unsigned)s.E);
  hipLaunchKernelGGL(gemm_wgrad_up_kernel, grid, dim3(kGemmThreads), 0, stream,
                     cp<float>(x_perm), cp<float>(dh1), cp<float>(dh3), s.H, s.F,
                     m.tokens_per_expert, m.padded_bins, mp<float>(dw1), mp<float>(dw3));
  return hipGetLastError();
}

}  // namespace dmoe
