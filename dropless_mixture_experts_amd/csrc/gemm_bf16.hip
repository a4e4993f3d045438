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
//     m dimension of a weight gradient); each wave owns 128 x 64 as 4 x 2
//     v_mfma_f32_32x32x16_bf16 tiles (128 fp32 accumulators).  The 32x32
//     form sustains several times the rate of 16x16x32 with one wave per
//     SIMD, which is all a 144 KB-LDS block allows.
//   * K step 64.  Three LDS stages of 48 KB (32 KB A + 16 KB B) are filled by
//     buffer_load ... lds (16 bytes per lane straight into LDS, no registers),
//     issued two K steps ahead of the MFMAs that consume them.  Each wave
//     fills whole 1 KB LDS blocks; the global address of every lane is
//     chosen so that the LDS image comes out swizzled.
//   * An operand whose source has K contiguous ("direct") is kept as
//     [row][64 k] (128-byte rows); its 16-byte chunk c of row r sits at chunk
//     c ^ ((r & 7) ^ ((r >> 3) & 1)) and is read with ds_read_b128.
//   * An operand whose source has its rows contiguous ([K][N] weights, and
//     both operands of the weight gradients: "trans") is kept as it lies in
//     memory, [64 k][128 n] per 128-column half, with the 64-byte unit u of
//     k-row k at u ^ (k & 3), and is read with two ds_read_b64_tr_b16: in
//     each 16-lane group, lane i fetches 4 values of k-row i/4 at columns
//     4(i%4).. and receives the 4 k-values of column i, which is exactly an
//     MFMA operand fragment.
//   * A tile that has only 128 A rows (a dimension that is an odd multiple
//     of 128) runs the same code with the second half compiled out.
#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {
namespace bfk {

constexpr int kThreads = 256;
constexpr int kRowB = 128;                    // bytes of K per direct LDS row
constexpr int kKStep = 64;                    // K per stage
constexpr int kRegA = 256 * kRowB;            // 32 KB
constexpr int kRegB = 128 * kRowB;            // 16 KB
constexpr int kHalf = 16384;                  // one 128-column trans half
constexpr int kStage = kRegA + kRegB;         // 48 KB
constexpr int kStages = 3;
constexpr int kLds = kStages * kStage;        // 144 KB

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p) {
  // raw buffer, no stride; every access is in bounds by construction, so
  // the range only has to cover them: take the largest positive size.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7fffffff, 0x00020000);
}

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N vector-memory operations of this
// wave in flight, and every LDS read of this wave completed (so a stage that
// is about to be refilled has no reads of it left in flight).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}
// Workgroup barrier without a memory fence: the fence of __syncthreads()
// would wait for every LDS DMA in flight, including the ones for later steps.
__device__ __forceinline__ void barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowB + ((chunk ^ swz(row)) << 4);
}

// One operand.  Tile rows [0,128) come from r0 and rows [128,256) from r1
// (A side only).  ld: bytes between consecutive source rows.
struct Op {
  rsrc_t r0, r1;
  uint32_t ld;
};

// Per-lane source offsets for the DMA of one operand.  A wave instruction
// fills one 1 KB LDS block: 8 direct rows (lane l -> row l/8, physical chunk
// l%8) or 4 trans k-rows (lane l -> k-row l/16, physical chunk l%16).  The
// swizzle of a block depends on the block only through one bit, so two
// offsets per lane cover every block.
template <bool TRANS>
struct Dma {
  uint32_t voff[2];
  __device__ __forceinline__ void init(uint32_t ld, int lane) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      if (!TRANS) {
        const int r = lane >> 3, c = (lane & 7) ^ r ^ v;
        voff[v] = (uint32_t)r * ld + (uint32_t)c * 16u;
      } else {
        const int r = lane >> 4, c = (lane & 15) ^ (r << 2);
        voff[v] = (uint32_t)r * ld + (uint32_t)c * 16u;
      }
    }
  }
};

__device__ __forceinline__ void dma16(rsrc_t r, char* lds_dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_dst, 16, voff, soff, 0, 0);
}

// A operand, one K step into `reg` (the A region of a stage).  Wave w fills
// blocks 8w..8w+7; waves 0-1 read rows [0,128) from r0, waves 2-3 rows
// [128,256) from r1.
template <bool TRANS, bool FULL>
__device__ __forceinline__ void issue_a(const Op& op, const Dma<TRANS>& d, int ks, int w,
                                        char* reg) {
  if (!FULL && w >= 2) return;
  const rsrc_t r = w < 2 ? op.r0 : op.r1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t soff;
    uint32_t vo;
    if (!TRANS) {
      soff = (uint32_t)ks * kRowB + (uint32_t)(64 * (w & 1) + 8 * i) * op.ld;
      vo = d.voff[i & 1];
    } else {
      soff = (uint32_t)(ks * kKStep + 4 * (8 * (w & 1) + i)) * op.ld;
      vo = d.voff[(i >> 1) & 1];
    }
    dma16(r, reg + (8 * w + i) * 1024, vo, soff);
  }
}

// B operand: wave w fills blocks 4w..4w+3.
template <bool TRANS>
__device__ __forceinline__ void issue_b(const Op& op, const Dma<TRANS>& d, int ks, int w,
                                        char* reg) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t soff;
    uint32_t vo;
    if (!TRANS) {
      soff = (uint32_t)ks * kRowB + (uint32_t)(32 * w + 8 * i) * op.ld;
      vo = d.voff[i & 1];
    } else {
      soff = (uint32_t)(ks * kKStep + 4 * (4 * w + i)) * op.ld;
      vo = d.voff[(i >> 1) & 1];
    }
    dma16(op.r0, reg + (4 * w + i) * 1024, vo, soff);
  }
}

// MFMA operand fragment for v_mfma_f32_32x32x16_bf16: 32 operand rows from
// `row0`, k-fragment kf (16 k values); lane l holds row row0 + l%32 and
// k = kf*16 + 8(l/32) + 0..7.
template <bool TRANS>
__device__ __forceinline__ bf16x8 frag(const char* reg, int row0, int kf, int lane) {
  if (!TRANS) {
    return *reinterpret_cast<const bf16x8*>(reg + lds_off(row0 + (lane & 31), kf * 2 + (lane >> 5)));
  } else {
    const int half = row0 >> 7, g = lane >> 4, i = lane & 15;
    const int k = kf * 16 + 8 * (g >> 1) + (i >> 2);
    const int n = (row0 & 127) + (g & 1) * 16 + 4 * (i & 3);
    const int c = n >> 3;
    const char* p = reg + half * kHalf + k * 256 + ((c ^ ((k & 3) << 2)) << 4) + (i & 1) * 8;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t)(const_cast<char*>(p)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t)(const_cast<char*>(p) + 4 * 256));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef f32x16 Acc[4][2];

// 32-row blocks of this wave: A blocks i = 0..3 (i < 2 in rows [0,128), i >= 2
// the same offsets in rows [128,256)), B blocks j = 0..1.
__device__ __forceinline__ int a_row(int i, int wm) { return (i >> 1) * 128 + wm * 64 + (i & 1) * 32; }
__device__ __forceinline__ int b_row(int j, int wn) { return wn * 64 + j * 32; }

// Fragments of one 16-wide k-fragment (24 VGPRs).
struct Frags {
  bf16x8 a[4];
  bf16x8 b[2];
};

template <bool ATR, bool BTR, bool FULL>
__device__ __forceinline__ void load_frags(Frags& f, const char* stage, int kf, int wm, int wn,
                                           int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) f.b[j] = frag<BTR>(stage + kRegA, b_row(j, wn), kf, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!FULL && i >= 2) break;
    f.a[i] = frag<ATR>(stage, a_row(i, wm), kf, lane);
  }
}

template <bool FULL>
__device__ __forceinline__ void mma(Acc& acc, const Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!FULL && i >= 2) break;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  }
}

// Wait until at most `later` DMA groups (one K step each) of this wave are in
// flight, and all of its LDS reads have landed.
template <bool FULL_LOADS>
__device__ __forceinline__ void wait_groups(int later) {
  if (FULL_LOADS) {
    if (later >= 2) wait_vm<24>(); else if (later == 1) wait_vm<12>(); else wait_vm<0>();
  } else {
    if (later >= 2) wait_vm<8>(); else if (later == 1) wait_vm<4>(); else wait_vm<0>();
  }
}

// Keeps the compiler from moving instructions across phase boundaries.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// acc += A . B^T over nk K steps.
//
// Each K step is four 16-wide k-fragments.  While the MFMAs of one fragment
// run, the LDS reads of the next are in flight.  Before the last fragment of
// step ks: wait for the DMA of step ks+1, barrier, start the DMA of step
// ks+3 into the stage of step ks (stages form a ring of three), and read the
// first fragment of step ks+1.  Ends with a barrier, so the LDS stages can
// be refilled right away (the up-projection dgrad runs two of these).
template <bool ATR, bool BTR, bool FULL>
__device__ __forceinline__ void mainloop(Acc& acc, const Op& A, const Op& B, int nk, char* lds) {
  if (nk <= 0) return;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  Dma<ATR> da;
  Dma<BTR> db;
  da.init(A.ld, lane);
  db.init(B.ld, lane);
  const bool full_loads = FULL || w < 2;   // waves that also load A
  auto issue = [&](int ks) {
    char* st = lds + (ks % kStages) * kStage;
    issue_a<ATR, FULL>(A, da, ks, w, st);
    issue_b<BTR>(B, db, ks, w, st + kRegA);
  };
  const int pre = nk < kStages ? nk : kStages;
  for (int s = 0; s < pre; ++s) issue(s);
  if (full_loads) wait_groups<true>(pre - 1); else wait_groups<false>(pre - 1);
  barrier();
  Frags f[2];
  load_frags<ATR, BTR, FULL>(f[0], lds, 0, wm, wn, lane);
  for (int ks = 0; ks < nk; ++ks) {
    const char* cur = lds + (ks % kStages) * kStage;
#pragma unroll
    for (int kf = 0; kf < 4; ++kf) {
      sched_fence();
      if (kf < 3) {
        load_frags<ATR, BTR, FULL>(f[(kf + 1) & 1], cur, kf + 1, wm, wn, lane);
      } else if (ks + 1 < nk) {
        const int later = (ks + 2 < nk) ? 1 : 0;   // step ks+2 still in flight
        if (full_loads) wait_groups<true>(later); else wait_groups<false>(later);
        barrier();
        if (ks + 3 < nk) issue(ks + 3);
        load_frags<ATR, BTR, FULL>(f[0], lds + ((ks + 1) % kStages) * kStage, 0, wm, wn, lane);
      }
      mma<FULL>(acc, f[kf & 1]);
    }
  }
  sched_fence();
  wait_vm<0>();
  barrier();
}

__device__ __forceinline__ void zero(Acc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[i][j][t] = 0.f;
}

// Accumulator (i, j) of lane l holds, for g = 0..3, the 4 consecutive A rows
// a_row(i) + 8g + 4(l/32) + 0..3 of B row b_row(j) + l%32.
__device__ __forceinline__ f32x4 quad(const f32x16& v, int g) {
  return f32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
}
template <bool FULL, class Fn>
__device__ __forceinline__ void for_quads(const Acc& acc, int wm, int wn, int lane, Fn&& fn) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!FULL && i >= 2) break;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int brow = b_row(j, wn) + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        fn(a_row(i, wm) + 8 * g + 4 * (lane >> 5), brow, quad(acc[i][j], g));
    }
  }
}

// ---- Block -> tile order --------------------------------------------------
// Workgroups are dealt to the 8 XCDs round-robin (block b runs on XCD b % 8),
// and each XCD has its own L2.  Each XCD is given one contiguous range of the
// logical tile order, so the blocks that share operands share an L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

// Logical index of block b among `total` tiles, or -1 if the block is spare.
__device__ __forceinline__ int xcd_tile(int b, int total) {
  const int per = (total + kXcds - 1) / kXcds;
  const int l = b / kXcds;
  if (l >= per) return -1;
  const int L = (b % kXcds) * per + l;
  return L < total ? L : -1;
}

// Row-tiled products: (m, n) for logical index L over MT x NT tiles, in
// groups of kGroupM row tiles walked column by column, so that concurrent
// blocks reuse both the token rows and the weight columns.
__device__ __forceinline__ void group_mn(int L, int MT, int NT, int& m, int& n) {
  const int per_group = kGroupM * NT;
  const int g = L / per_group;
  const int m0 = g * kGroupM;
  const int gm = min(kGroupM, MT - m0);
  const int r = L - g * per_group;
  m = m0 + r % gm;
  n = r / gm;
}

// Row-tiled tile of this block from the live row count; false if spare.
__device__ __forceinline__ bool row_tile(const int32_t* num_padded_rows, int NT,
                                         int64_t& mt, int64_t& nt) {
  const int MT = *num_padded_rows / kBlock;
  const int L = xcd_tile(blockIdx.x, MT * NT);
  if (L < 0) return false;
  int m, n;
  group_mn(L, MT, NT, m, n);
  mt = m;
  nt = n;
  return true;
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
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;            \
  const int wm = w >> 1, wn = w & 1;

// h1 = x_perm w1[e], h3 = x_perm w3[e], act = silu(h1) * h3 for one 128-row
// block and 128 ffn columns (w1 columns in A rows 0..127, the same w3
// columns in A rows 128..255, so A blocks i and i+2 pair up).
__global__ void __launch_bounds__(kThreads)
up_kernel(const bf16* __restrict__ x_perm, const bf16* __restrict__ w1,
          const bf16* __restrict__ w3, int64_t H, int64_t F,
          const int32_t* __restrict__ tile_expert,
          const int32_t* __restrict__ num_padded_rows, bf16* __restrict__ h1,
          bf16* __restrict__ h3, bf16* __restrict__ act) {
  BF_PROLOGUE
  int64_t mt, nt;
  if (!row_tile(num_padded_rows, (int)(F / 128), mt, nt)) return;
  const int64_t f0 = nt * 128;
  const int e = tile_expert[mt];
  if (e < 0) return;
  const int64_t wofs = (int64_t)e * H * F + f0;
  const Op A{make_rsrc(w1 + wofs), make_rsrc(w3 + wofs), (uint32_t)(F * 2)};
  const Op B{make_rsrc(x_perm + mt * kBlock * H), make_rsrc(x_perm), (uint32_t)(H * 2)};
  Acc acc;
  zero(acc);
  mainloop<true, false, true>(acc, A, B, (int)(H / kKStep), lds);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t p = mt * kBlock + b_row(j, wn) + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t f = f0 + a_row(i, wm) + 8 * g + 4 * (lane >> 5);
        const f32x4 v1 = quad(acc[i][j], g), v3 = quad(acc[i + 2][j], g);
        f32x4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = silu(v1[r]) * v3[r];
        store4(h1 + p * F + f, v1);
        store4(h3 + p * F + f, v3);
        store4(act + p * F + f, a);
      }
    }
}

// y_perm = act w2[e] for one 128-row block and 256 (or 128) hidden columns.
template <bool FULL>
__device__ __forceinline__ void down_body(const bf16* act, const bf16* w2, int64_t H,
                                          int64_t F, int64_t mt, int64_t h0, int e,
                                          bf16* y_perm, char* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const bf16* wb = w2 + (int64_t)e * F * H + h0;
  const Op A{make_rsrc(wb), make_rsrc(wb + 128), (uint32_t)(H * 2)};
  const Op B{make_rsrc(act + mt * kBlock * F), make_rsrc(act), (uint32_t)(F * 2)};
  Acc acc;
  zero(acc);
  mainloop<true, false, FULL>(acc, A, B, (int)(F / kKStep), lds);
  bf16* out = y_perm + mt * kBlock * H + h0;
  for_quads<FULL>(acc, wm, wn, lane, [&](int arow, int brow, const f32x4& v) {
    store4(out + (int64_t)brow * H + arow, v);
  });
}

__global__ void __launch_bounds__(kThreads)
down_kernel(const bf16* __restrict__ act, const bf16* __restrict__ w2, int64_t H,
            int64_t F, const int32_t* __restrict__ tile_expert,
            const int32_t* __restrict__ num_padded_rows, bf16* __restrict__ y_perm) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  int64_t mt, nt;
  if (!row_tile(num_padded_rows, (int)((H + 255) / 256), mt, nt)) return;
  const int64_t h0 = nt * 256;
  const int e = tile_expert[mt];
  if (e < 0) return;
  if (h0 + 256 <= H)
    down_body<true>(act, w2, H, F, mt, h0, e, y_perm, lds);
  else
    down_body<false>(act, w2, H, F, mt, h0, e, y_perm, lds);
}

// dA = dy_perm w2[e]^T, then the gate's backward:
// dh3 = dA * silu(h1), dh1 = dA * h3 * s * (1 + h1 (1 - s)), s = sigmoid(h1).
template <bool FULL>
__device__ __forceinline__ void down_dgrad_body(const bf16* dy_perm, const bf16* w2,
                                                const bf16* h1, const bf16* h3, int64_t H,
                                                int64_t F, int64_t mt, int64_t fb, int e,
                                                bf16* dh1, bf16* dh3, char* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const bf16* wb = w2 + (int64_t)e * F * H + fb * H;
  const Op A{make_rsrc(wb), make_rsrc(wb + 128 * H), (uint32_t)(H * 2)};
  const Op B{make_rsrc(dy_perm + mt * kBlock * H), make_rsrc(dy_perm), (uint32_t)(H * 2)};
  Acc acc;
  zero(acc);
  mainloop<false, false, FULL>(acc, A, B, (int)(H / kKStep), lds);
  const int64_t base = mt * kBlock * F + fb;
  for_quads<FULL>(acc, wm, wn, lane, [&](int arow, int brow, const f32x4& da) {
    const int64_t o = base + (int64_t)brow * F + arow;
    const f32x4 g1 = load4(h1 + o), g3 = load4(h3 + o);
    f32x4 d1, d3;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s = 1.0f / (1.0f + __expf(-g1[r]));
      d3[r] = da[r] * g1[r] * s;
      d1[r] = da[r] * g3[r] * s * (1.0f + g1[r] * (1.0f - s));
    }
    store4(dh1 + o, d1);
    store4(dh3 + o, d3);
  });
}

__global__ void __launch_bounds__(kThreads)
down_dgrad_kernel(const bf16* __restrict__ dy_perm, const bf16* __restrict__ w2,
                  const bf16* h1, const bf16* h3, int64_t H, int64_t F,
                  const int32_t* __restrict__ tile_expert,
                  const int32_t* __restrict__ num_padded_rows, bf16* dh1, bf16* dh3) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  int64_t mt, nt;
  if (!row_tile(num_padded_rows, (int)((F + 255) / 256), mt, nt)) return;
  const int64_t fb = nt * 256;
  const int e = tile_expert[mt];
  if (e < 0) return;
  if (fb + 256 <= F)
    down_dgrad_body<true>(dy_perm, w2, h1, h3, H, F, mt, fb, e, dh1, dh3, lds);
  else
    down_dgrad_body<false>(dy_perm, w2, h1, h3, H, F, mt, fb, e, dh1, dh3, lds);
}

// dx_perm = dh1 w1[e]^T + dh3 w3[e]^T.
template <bool FULL>
__device__ __forceinline__ void up_dgrad_body(const bf16* dh1, const bf16* dh3,
                                              const bf16* w1, const bf16* w3, int64_t H,
                                              int64_t F, int64_t mt, int64_t h0, int e,
                                              bf16* dx_perm, char* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int64_t wofs = (int64_t)e * H * F + h0 * F;
  const int nk = (int)(F / kKStep);
  Acc acc;
  zero(acc);
  {
    const Op A{make_rsrc(w1 + wofs), make_rsrc(w1 + wofs + 128 * F), (uint32_t)(F * 2)};
    const Op B{make_rsrc(dh1 + mt * kBlock * F), make_rsrc(dh1), (uint32_t)(F * 2)};
    mainloop<false, false, FULL>(acc, A, B, nk, lds);
  }
  {
    const Op A{make_rsrc(w3 + wofs), make_rsrc(w3 + wofs + 128 * F), (uint32_t)(F * 2)};
    const Op B{make_rsrc(dh3 + mt * kBlock * F), make_rsrc(dh3), (uint32_t)(F * 2)};
    mainloop<false, false, FULL>(acc, A, B, nk, lds);
  }
  bf16* out = dx_perm + mt * kBlock * H + h0;
  for_quads<FULL>(acc, wm, wn, lane, [&](int arow, int brow, const f32x4& v) {
    store4(out + (int64_t)brow * H + arow, v);
  });
}

__global__ void __launch_bounds__(kThreads)
up_dgrad_kernel(const bf16* __restrict__ dh1, const bf16* __restrict__ dh3,
                const bf16* __restrict__ w1, const bf16* __restrict__ w3, int64_t H,
                int64_t F, const int32_t* __restrict__ tile_expert,
                const int32_t* __restrict__ num_padded_rows, bf16* dx_perm) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  int64_t mt, nt;
  if (!row_tile(num_padded_rows, (int)((H + 255) / 256), mt, nt)) return;
  const int64_t h0 = nt * 256;
  const int e = tile_expert[mt];
  if (e < 0) return;
  if (h0 + 256 <= H)
    up_dgrad_body<true>(dh1, dh3, w1, w3, H, F, mt, h0, e, dx_perm, lds);
  else
    up_dgrad_body<false>(dh1, dh3, w1, w3, H, F, mt, h0, e, dx_perm, lds);
}

// dw2[e] = act[rows_e]^T dy_perm[rows_e] ([F,H]); zero for an empty expert.
template <bool FULL>
__device__ __forceinline__ void wgrad_down_body(const bf16* act, const bf16* dy_perm,
                                                int64_t H, int64_t F, int64_t start, int n,
                                                int64_t h0, int64_t f0, int e, bf16* dw2,
                                                char* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const bf16* ab = dy_perm + start * H + h0;
  const Op A{make_rsrc(ab), make_rsrc(ab + 128), (uint32_t)(H * 2)};
  const Op B{make_rsrc(act + start * F + f0), make_rsrc(act), (uint32_t)(F * 2)};
  Acc acc;
  zero(acc);
  mainloop<true, true, FULL>(acc, A, B, n / kKStep, lds);
  bf16* out = dw2 + (int64_t)e * F * H + f0 * H + h0;
  for_quads<FULL>(acc, wm, wn, lane, [&](int arow, int brow, const f32x4& v) {
    store4(out + (int64_t)brow * H + arow, v);
  });
}

__global__ void __launch_bounds__(kThreads)
wgrad_down_kernel(const bf16* __restrict__ act, const bf16* __restrict__ dy_perm,
                  int64_t H, int64_t F, int E, const int32_t* __restrict__ tpe,
                  const int32_t* __restrict__ padded_bins, bf16* __restrict__ dw2) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  // tiles of one expert are consecutive: each XCD works on whole experts
  const int NH = (int)((H + 255) / 256), NF = (int)(F / 128);
  const int L = xcd_tile(blockIdx.x, E * NH * NF);
  if (L < 0) return;
  const int e = L / (NH * NF);
  const int t = L - e * (NH * NF);
  const int64_t h0 = (int64_t)(t % NH) * 256, f0 = (int64_t)(t / NH) * 128;
  const int n = round_up_block(tpe[e]);
  const int64_t start = padded_bins[e] - n;
  if (h0 + 256 <= H)
    wgrad_down_body<true>(act, dy_perm, H, F, start, n, h0, f0, e, dw2, lds);
  else
    wgrad_down_body<false>(act, dy_perm, H, F, start, n, h0, f0, e, dw2, lds);
}

// dw1[e] = x_perm[rows_e]^T dh1[rows_e], dw3[e] = x_perm[rows_e]^T dh3[rows_e]
// ([H,F] each; dh1 columns in A rows 0..127, dh3 in A rows 128..255).
__global__ void __launch_bounds__(kThreads)
wgrad_up_kernel(const bf16* __restrict__ x_perm, const bf16* __restrict__ dh1,
                const bf16* __restrict__ dh3, int64_t H, int64_t F, int E,
                const int32_t* __restrict__ tpe, const int32_t* __restrict__ padded_bins,
                bf16* __restrict__ dw1, bf16* __restrict__ dw3) {
  BF_PROLOGUE
  const int NF = (int)(F / 128), NH = (int)(H / 128);
  const int L = xcd_tile(blockIdx.x, E * NF * NH);
  if (L < 0) return;
  const int e = L / (NF * NH);
  const int t = L - e * (NF * NH);
  const int64_t f0 = (int64_t)(t % NF) * 128, h0 = (int64_t)(t / NF) * 128;
  const int n = round_up_block(tpe[e]);
  const int64_t start = padded_bins[e] - n;
  const Op A{make_rsrc(dh1 + start * F + f0), make_rsrc(dh3 + start * F + f0), (uint32_t)(F * 2)};
  const Op B{make_rsrc(x_perm + start * H + h0), make_rsrc(x_perm), (uint32_t)(H * 2)};
  Acc acc;
  zero(acc);
  mainloop<true, true, true>(acc, A, B, n / kKStep, lds);
  const int64_t eo = (int64_t)e * H * F + h0 * F + f0;
  for_quads<true>(acc, wm, wn, lane, [&](int arow, int brow, const f32x4& v) {
    // A rows 0..127 are dw1 columns, 128..255 the same dw3 columns
    store4((arow < 128 ? dw1 : dw3) + eo + (int64_t)brow * F + (arow & 127), v);
  });
}

}  // namespace bfk

static unsigned cdiv_u(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// Enough blocks for every XCD to take ceil(total / 8) tiles.
static dim3 xcd_grid(int64_t total) { return dim3(8u * cdiv_u(total, 8)); }

hipError_t launch_bf16_up(const Shape& s, const void* x_perm, const void* w1, const void* w3,
                          const MetaPtrs& m, void* h1, void* h3, void* act,
                          hipStream_t stream) {
  hipLaunchKernelGGL(bfk::up_kernel, xcd_grid(cdiv_u(s.F, 128) * s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(x_perm),
                     static_cast<const bf16*>(w1), static_cast<const bf16*>(w3), s.H, s.F,
                     m.tile_expert, m.num_padded_rows, static_cast<bf16*>(h1),
                     static_cast<bf16*>(h3),
                     static_cast<bf16*>(act));
  return hipGetLastError();
}

hipError_t launch_bf16_down(const Shape& s, const void* act, const void* w2,
                            const MetaPtrs& m, void* y_perm, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::down_kernel, xcd_grid(cdiv_u(s.H, 256) * s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(act),
                     static_cast<const bf16*>(w2), s.H, s.F, m.tile_expert,
                     m.num_padded_rows, static_cast<bf16*>(y_perm));
  return hipGetLastError();
}

hipError_t launch_bf16_down_dgrad(const Shape& s, const void* dy_perm, const void* w2,
                                  const void* h1, const void* h3, const MetaPtrs& m,
                                  void* dh1, void* dh3, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::down_dgrad_kernel, xcd_grid(cdiv_u(s.F, 256) * s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(dy_perm),
                     static_cast<const bf16*>(w2), static_cast<const bf16*>(h1),
                     static_cast<const bf16*>(h3), s.H, s.F, m.tile_expert,
                     m.num_padded_rows, static_cast<bf16*>(dh1), static_cast<bf16*>(dh3));
  return hipGetLastError();
}

hipError_t launch_bf16_up_dgrad(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const MetaPtrs& m,
                                void* dx_perm, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::up_dgrad_kernel, xcd_grid(cdiv_u(s.H, 256) * s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(dh1),
                     static_cast<const bf16*>(dh3), static_cast<const bf16*>(w1),
                     static_cast<const bf16*>(w3), s.H, s.F, m.tile_expert,
                     m.num_padded_rows, static_cast<bf16*>(dx_perm));
  return hipGetLastError();
}

hipError_t launch_bf16_wgrad_down(const Shape& s, const void* act, const void* dy_perm,
                                  const MetaPtrs& m, void* dw2, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::wgrad_down_kernel,
                     xcd_grid((int64_t)cdiv_u(s.H, 256) * cdiv_u(s.F, 128) * s.E),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(act),
                     static_cast<const bf16*>(dy_perm), s.H, s.F, s.E, m.tokens_per_expert,
                     m.padded_bins, static_cast<bf16*>(dw2));
  return hipGetLastError();
}

hipError_t launch_bf16_wgrad_up(const Shape& s, const void* x_perm, const void* dh1,
                                const void* dh3, const MetaPtrs& m, void* dw1, void* dw3,
                                hipStream_t stream) {
  hipLaunchKernelGGL(bfk::wgrad_up_kernel,
                     xcd_grid((int64_t)cdiv_u(s.F, 128) * cdiv_u(s.H, 128) * s.E),
                     dim3(bfk::kThreads), 0, stream, static_cast<const bf16*>(x_perm),
                     static_cast<const bf16*>(dh1), static_cast<const bf16*>(dh3), s.H,
                     s.F, s.E, m.tokens_per_expert, m.padded_bins, static_cast<bf16*>(dw1),
                     static_cast<bf16*>(dw3));
  return hipGetLastError();
}

}  // namespace dmoe
