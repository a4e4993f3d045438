// bf16 grouped GEMM over expert-tagged row blocks (gfx950 MFMA).
//
// The products are those of the MegaBlocks chapter "02 · dropless MoE 与
// block-sparse 重构" §3 (sdd: x_perm w1 / x_perm w3, dsd: act w2, on the row
// blocks of each expert only) and their backward, exactly as in the generic
// engine of gemm.hip; this file is the bf16 fast path.
//
// Engine
//   * 512 threads = 8 waves (2 x 4).  A block computes a 256 x 256 tile:
//     256 "A rows" along the output's contiguous dimension (weights side)
//     x 256 "B rows" (two 128-row blocks of the same expert, or the m
//     dimension of a weight gradient).  Each wave owns 128 x 64 as 4 x 2
//     v_mfma_f32_32x32x16_bf16 tiles (128 fp32 accumulators); two waves
//     share each SIMD.  The 256 x 256 tile halves the bytes each CU pulls
//     per FLOP compared with 256 x 128, which is what bounds these
//     products: the number of memory requests a CU can keep in flight.
//   * K step 64.  Two LDS stages of 64 KB (32 KB A + 32 KB B) are filled by
//     buffer_load ... lds (16 bytes per lane straight into LDS, no
//     registers).  Each wave fills whole 1 KB LDS blocks; the global address
//     of every lane is chosen so that the LDS image comes out swizzled.
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
//   * Either half of A or B may be absent (a dimension that is an odd
//     multiple of 128, or an expert with an odd number of row blocks); the
//     same code runs with that half compiled out.
#include "dmoe_device.h"
#include "dmoe_internal.h"

namespace dmoe {
namespace bfk {

constexpr int kThreads = 512;
constexpr int kRowB = 128;                    // bytes of K per direct LDS row
constexpr int kKStep = 64;                    // K per stage
constexpr int kReg = 256 * kRowB;             // 32 KB per operand per stage
constexpr int kHalf = 16384;                  // one 128-row (or -column) half
constexpr int kStage = 2 * kReg;              // 64 KB
constexpr int kStages = 2;
constexpr int kLds = kStages * kStage;        // 128 KB

// Buffer resource: base, no stride, the largest record count, 32-bit data
// format (every access is in bounds by construction, so the range only has
// to cover them).
typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_t;
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ rsrc_t make_rsrc(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return rsrc_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, 0x7fffffffu, 0x00020000u};
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
// Keeps the compiler from moving instructions across phase boundaries.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowB + ((chunk ^ swz(row)) << 4);
}

// One operand.  Tile rows (direct) or columns (trans) [0,128) come from r0
// and [128,256) from r1.  ld: bytes between consecutive source rows.
struct Op {
  rsrc_t r0, r1;
  uint32_t ld;
};

// Per-lane source offset for the DMA of one operand.  A wave instruction
// fills one 1 KB LDS block: 8 direct rows (lane l -> row l/8, physical chunk
// l%8) or 4 trans k-rows (lane l -> k-row l/16, physical chunk l%16).  The
// direct swizzle of a block depends on the block only through its parity.
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

// 16 bytes per lane from r + voff + soff into LDS at lds_addr + 16 * lane.
// Written as asm so that the compiler does not see an LDS write it cannot
// place: it would then make every transposed LDS read wait for all DMA in
// flight, the prefetch of later steps included.  Completion is awaited
// explicitly (wait_vm + barrier) before a stage is read.  The asm has no
// register outputs.  The nops cover the SGPR-written-by-VALU and M0-write
// hazards of an LDS DMA.
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ void dma16(const rsrc_t& rv, uint32_t lds_addr, uint32_t voff,
                                      uint32_t soff) {
  const rsrc_t r{uniform(rv[0]), uniform(rv[1]), uniform(rv[2]), uniform(rv[3])};
  asm volatile(
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(r), "s"(uniform(soff)), "{m0}"(uniform(lds_addr))
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)const_cast<char*>(p);
}

// One operand, one K step into the LDS region at address `reg` (32 KB = 32
// blocks of 1 KB).  Wave w fills blocks 4w..4w+3, all in half w / 4.
template <bool TRANS>
__device__ __forceinline__ void issue(const Op& op, const Dma<TRANS>& d, int ks, int w,
                                      uint32_t reg) {
  const rsrc_t r = w < 4 ? op.r0 : op.r1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bb = 4 * (w & 3) + i;            // block within the half
    uint32_t soff, vo;
    if (!TRANS) {
      soff = (uint32_t)ks * kRowB + (uint32_t)(8 * bb) * op.ld;
      vo = d.voff[i & 1];
    } else {
      soff = (uint32_t)(ks * kKStep + 4 * bb) * op.ld;
      vo = d.voff[0];
    }
    dma16(r, reg + (4 * w + i) * 1024, vo, soff);
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
    char* p = const_cast<char*>(reg) + half * kHalf + k * 256 + ((c ^ ((k & 3) << 2)) << 4) +
              (i & 1) * 8;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t)p);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t)(p + 4 * 256));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

typedef f32x16 Acc[4][2];

// 32-row blocks of wave (wm, wn): A blocks i = 0..3 (i < 2 in A rows
// [0,128), i >= 2 at the same offsets in [128,256)), B blocks j = 0..1.
__device__ __forceinline__ int a_row(int i, int wm) { return (i >> 1) * 128 + wm * 64 + (i & 1) * 32; }
__device__ __forceinline__ int b_row(int j, int wn) { return wn * 64 + j * 32; }

// Fragments of one 16-wide k-fragment (24 VGPRs).
struct Frags {
  bf16x8 a[4];
  bf16x8 b[2];
};

template <bool ATR, bool BTR, bool FA>
__device__ __forceinline__ void load_frags(Frags& f, const char* stage, int kf, int wm, int wn,
                                           int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) f.b[j] = frag<BTR>(stage + kReg, b_row(j, wn), kf, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!FA && i >= 2) break;
    f.a[i] = frag<ATR>(stage, a_row(i, wm), kf, lane);
  }
}

template <bool FA>
__device__ __forceinline__ void mma(Acc& acc, const Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!FA && i >= 2) break;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  }
}

// DMA of K step ks into its stage (lds: LDS address of the stages).
template <bool ATR, bool BTR>
__device__ __forceinline__ void start_step(const Op& A, const Op& B, const Dma<ATR>& da,
                                           const Dma<BTR>& db, int ks, int w, bool load_a,
                                           bool load_b, uint32_t lds) {
  const uint32_t st = lds + (ks % kStages) * kStage;
  if (load_a) issue<ATR>(A, da, ks, w, st);
  if (load_b) issue<BTR>(B, db, ks, w, st + kReg);
}

// acc += A . B^T over nk K steps (FA / FB: second half of A / B present).
//
// Each K step is four 16-wide k-fragments.  While the MFMAs of one fragment
// run, the LDS reads of the next are in flight.  Before the last fragment of
// step ks: wait for the DMA of step ks+1, barrier, start the DMA of step
// ks+2 into the stage of step ks (nobody reads it any more) and read the
// first fragment of step ks+1.  Ends with a barrier, so the LDS stages can
// be refilled right away (the up-projection dgrad runs two of these).
template <bool ATR, bool BTR, bool FA, bool FB>
__device__ __forceinline__ void mainloop(Acc& acc, const Op& A, const Op& B, int nk, char* lds) {
  if (nk <= 0) return;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 2, wn = w & 3;
  const bool load_a = FA || w < 4, load_b = FB || w < 4;
  const bool work = FB || wn < 2;           // this wave has B rows
  Dma<ATR> da;
  Dma<BTR> db;
  da.init(A.ld, lane);
  db.init(B.ld, lane);
  const uint32_t lbase = uniform(lds_addr(lds));
  start_step<ATR, BTR>(A, B, da, db, 0, w, load_a, load_b, lbase);
  if (nk > 1) {
    start_step<ATR, BTR>(A, B, da, db, 1, w, load_a, load_b, lbase);
    // wait for step 0: step 1 (0, 4 or 8 instructions) may stay in flight
    if (load_a && load_b) wait_vm<8>(); else if (load_a || load_b) wait_vm<4>(); else wait_vm<0>();
  } else {
    wait_vm<0>();
  }
  barrier();
  Frags f[2];
  if (work) load_frags<ATR, BTR, FA>(f[0], lds, 0, wm, wn, lane);
  for (int ks = 0; ks < nk; ++ks) {
    const char* cur = lds + (ks % kStages) * kStage;
#pragma unroll
    for (int kf = 0; kf < 4; ++kf) {
      sched_fence();
      if (kf < 3) {
        if (work) load_frags<ATR, BTR, FA>(f[(kf + 1) & 1], cur, kf + 1, wm, wn, lane);
      } else if (ks + 1 < nk) {
        wait_vm<0>();                       // step ks+1 landed (nothing later in flight)
        barrier();
        if (ks + 2 < nk) start_step<ATR, BTR>(A, B, da, db, ks + 2, w, load_a, load_b, lbase);
        if (work)
          load_frags<ATR, BTR, FA>(f[0], lds + ((ks + 1) % kStages) * kStage, 0, wm, wn, lane);
      }
      if (work) mma<FA>(acc, f[kf & 1]);
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
template <bool FA, bool FB, class Fn>
__device__ __forceinline__ void for_quads(const Acc& acc, int lane, Fn&& fn) {
  const int w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;
  if (!FB && wn >= 2) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!FA && i >= 2) break;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int brow = b_row(j, wn) + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        fn(i, a_row(i, wm) + 8 * g + 4 * (lane >> 5), brow, quad(acc[i][j], g));
    }
  }
}

__device__ __forceinline__ void store4(bf16* p, const f32x4& v) {
  const uint32_t a = __builtin_bit_cast(uint16_t, from_f32<bf16>(v[0])) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(v[1])) << 16);
  const uint32_t b = __builtin_bit_cast(uint16_t, from_f32<bf16>(v[2])) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(v[3])) << 16);
  *reinterpret_cast<u32x2*>(p) = u32x2{a, b};
}
__device__ __forceinline__ f32x4 unpack4(const u32x2& u) {
  return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// ---- Block -> tile order --------------------------------------------------
// Workgroups are dealt to the 8 XCDs round-robin (block b runs on XCD b % 8),
// and each XCD has its own L2.  Each XCD is given one contiguous range of the
// logical tile order, so the blocks that share operands share an L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

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

// The (pair of) row blocks and the column tile of this block, from the live
// metadata; false if the block is spare.  two: the pair has two blocks.
struct RowTile {
  int64_t mt;    // first 128-row block
  int64_t nt;    // column tile
  int e;         // expert
  bool two;
};
__device__ __forceinline__ bool row_tile(const int32_t* num_pairs, const int32_t* pair_first,
                                         const int32_t* tile_expert,
                                         const int32_t* num_padded_rows, int NT, RowTile& t) {
  const int S = *num_pairs;
  const int L = xcd_tile(blockIdx.x, S * NT);
  if (L < 0) return false;
  int s, n;
  group_mn(L, S, NT, s, n);
  const int m = pair_first[s];
  const int MT = *num_padded_rows / kBlock;
  t.mt = m;
  t.nt = n;
  t.e = tile_expert[m];
  t.two = m + 1 < MT && tile_expert[m + 1] == t.e;
  return true;
}

#define ROW_TILE_ARGS                                                                   \
  const int32_t *__restrict__ tile_expert, const int32_t *__restrict__ num_padded_rows, \
      const int32_t *__restrict__ pair_first, const int32_t *__restrict__ num_pairs

// Runs CALL with FA and FB as compile-time constants.
#define DISPATCH2(FA_, FB_, CALL)                                   \
  do {                                                              \
    if (FA_) {                                                      \
      if (FB_) { constexpr bool FA = true, FB = true; CALL; }       \
      else { constexpr bool FA = true, FB = false; CALL; }          \
    } else {                                                        \
      if (FB_) { constexpr bool FA = false, FB = true; CALL; }      \
      else { constexpr bool FA = false, FB = false; CALL; }         \
    }                                                               \
  } while (0)

// h1 = x_perm w1[e], h3 = x_perm w3[e], act = silu(h1) * h3 for one pair of
// row blocks and 128 ffn columns (w1 columns in A rows 0..127, the same w3
// columns in A rows 128..255, so A blocks i and i+2 pair up).
template <bool FB>
__device__ __forceinline__ void up_body(const bf16* x_perm, const bf16* w1, const bf16* w3,
                                        int64_t H, int64_t F, const RowTile& t, bf16* h1,
                                        bf16* h3, bf16* act, char* lds) {
  const int lane = threadIdx.x & 63;
  const int64_t f0 = t.nt * 128;
  const int64_t wofs = (int64_t)t.e * H * F + f0;
  const bf16* xb = x_perm + t.mt * kBlock * H;
  const Op A{make_rsrc(w1 + wofs), make_rsrc(w3 + wofs), (uint32_t)(F * 2)};
  const Op B{make_rsrc(xb), make_rsrc(xb + kBlock * H), (uint32_t)(H * 2)};
  Acc acc;
  zero(acc);
  mainloop<true, false, true, FB>(acc, A, B, (int)(H / kKStep), lds);
  const int64_t base = t.mt * kBlock * F + f0;
  const int w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;
  if (!FB && wn >= 2) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t prow = b_row(j, wn) + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t o = base + prow * F + a_row(i, wm) + 8 * g + 4 * (lane >> 5);
        const f32x4 v1 = quad(acc[i][j], g), v3 = quad(acc[i + 2][j], g);
        f32x4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = silu(v1[r]) * v3[r];
        store4(h1 + o, v1);
        store4(h3 + o, v3);
        store4(act + o, a);
      }
    }
}

__global__ void __launch_bounds__(kThreads)
up_kernel(const bf16* __restrict__ x_perm, const bf16* __restrict__ w1,
          const bf16* __restrict__ w3, int64_t H, int64_t F, ROW_TILE_ARGS,
          bf16* __restrict__ h1, bf16* __restrict__ h3, bf16* __restrict__ act) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  RowTile t;
  if (!row_tile(num_pairs, pair_first, tile_expert, num_padded_rows, (int)(F / 128), t)) return;
  if (t.two)
    up_body<true>(x_perm, w1, w3, H, F, t, h1, h3, act, lds);
  else
    up_body<false>(x_perm, w1, w3, H, F, t, h1, h3, act, lds);
}

// y_perm = act w2[e] for one pair of row blocks and 256 (or 128) hidden columns.
template <bool FA, bool FB>
__device__ __forceinline__ void down_body(const bf16* act, const bf16* w2, int64_t H,
                                          int64_t F, const RowTile& t, bf16* y_perm,
                                          char* lds) {
  const int lane = threadIdx.x & 63;
  const int64_t h0 = t.nt * 256;
  const bf16* wb = w2 + (int64_t)t.e * F * H + h0;
  const bf16* ab = act + t.mt * kBlock * F;
  const Op A{make_rsrc(wb), make_rsrc(wb + 128), (uint32_t)(H * 2)};
  const Op B{make_rsrc(ab), make_rsrc(ab + kBlock * F), (uint32_t)(F * 2)};
  Acc acc;
  zero(acc);
  mainloop<true, false, FA, FB>(acc, A, B, (int)(F / kKStep), lds);
  bf16* out = y_perm + t.mt * kBlock * H + h0;
  for_quads<FA, FB>(acc, lane, [&](int, int arow, int brow, const f32x4& v) {
    store4(out + (int64_t)brow * H + arow, v);
  });
}

__global__ void __launch_bounds__(kThreads)
down_kernel(const bf16* __restrict__ act, const bf16* __restrict__ w2, int64_t H,
            int64_t F, ROW_TILE_ARGS, bf16* __restrict__ y_perm) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  RowTile t;
  if (!row_tile(num_pairs, pair_first, tile_expert, num_padded_rows, (int)((H + 255) / 256), t))
    return;
  DISPATCH2(t.nt * 256 + 256 <= H, t.two, (down_body<FA, FB>(act, w2, H, F, t, y_perm, lds)));
}

// dA = dy_perm w2[e]^T, then the gate's backward:
// dh3 = dA * silu(h1), dh1 = dA * h3 * s * (1 + h1 (1 - s)), s = sigmoid(h1).
template <bool FA, bool FB>
__device__ __forceinline__ void down_dgrad_body(const bf16* dy_perm, const bf16* w2,
                                                const bf16* h1, const bf16* h3, int64_t H,
                                                int64_t F, const RowTile& t, bf16* dh1,
                                                bf16* dh3, char* lds) {
  const int lane = threadIdx.x & 63;
  const int64_t fb = t.nt * 256;
  const bf16* wb = w2 + (int64_t)t.e * F * H + fb * H;
  const bf16* db = dy_perm + t.mt * kBlock * H;
  const Op A{make_rsrc(wb), make_rsrc(wb + 128 * H), (uint32_t)(H * 2)};
  const Op B{make_rsrc(db), make_rsrc(db + kBlock * H), (uint32_t)(H * 2)};
  Acc acc;
  zero(acc);
  mainloop<false, false, FA, FB>(acc, A, B, (int)(H / kKStep), lds);
  const int64_t base = t.mt * kBlock * F + fb;
  const int w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;
  if (!FB && wn >= 2) return;
  // h1/h3 of half of this lane's outputs are loaded before any of them is
  // stored, so the loads overlap (dh1/dh3 may alias h1/h3, which keeps the
  // compiler from hoisting a load above an earlier store; each element is
  // read by the lane that overwrites it).
#pragma unroll
  for (int i0 = 0; i0 < 4; i0 += 2) {
    if (!FA && i0 >= 2) break;
    u32x2 g1[2][2][4], g3[2][2][4];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t o = base + (int64_t)(b_row(j, wn) + (lane & 31)) * F +
                            a_row(i0 + ii, wm) + 8 * g + 4 * (lane >> 5);
          g1[ii][j][g] = *reinterpret_cast<const u32x2*>(h1 + o);
          g3[ii][j][g] = *reinterpret_cast<const u32x2*>(h3 + o);
        }
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t o = base + (int64_t)(b_row(j, wn) + (lane & 31)) * F +
                            a_row(i0 + ii, wm) + 8 * g + 4 * (lane >> 5);
          const f32x4 da = quad(acc[i0 + ii][j], g);
          const f32x4 x1 = unpack4(g1[ii][j][g]), x3 = unpack4(g3[ii][j][g]);
          f32x4 d1, d3;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float s = 1.0f / (1.0f + __expf(-x1[r]));
            d3[r] = da[r] * x1[r] * s;
            d1[r] = da[r] * x3[r] * s * (1.0f + x1[r] * (1.0f - s));
          }
          store4(dh1 + o, d1);
          store4(dh3 + o, d3);
        }
  }
}

__global__ void __launch_bounds__(kThreads)
down_dgrad_kernel(const bf16* __restrict__ dy_perm, const bf16* __restrict__ w2,
                  const bf16* h1, const bf16* h3, int64_t H, int64_t F, ROW_TILE_ARGS,
                  bf16* dh1, bf16* dh3) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  RowTile t;
  if (!row_tile(num_pairs, pair_first, tile_expert, num_padded_rows, (int)((F + 255) / 256), t))
    return;
  DISPATCH2(t.nt * 256 + 256 <= F, t.two,
            (down_dgrad_body<FA, FB>(dy_perm, w2, h1, h3, H, F, t, dh1, dh3, lds)));
}

// dx_perm = dh1 w1[e]^T + dh3 w3[e]^T.
template <bool FA, bool FB>
__device__ __forceinline__ void up_dgrad_body(const bf16* dh1, const bf16* dh3,
                                              const bf16* w1, const bf16* w3, int64_t H,
                                              int64_t F, const RowTile& t, bf16* dx_perm,
                                              char* lds) {
  const int lane = threadIdx.x & 63;
  const int64_t h0 = t.nt * 256;
  const int64_t wofs = (int64_t)t.e * H * F + h0 * F;
  const int nk = (int)(F / kKStep);
  Acc acc;
  zero(acc);
  {
    const bf16* db = dh1 + t.mt * kBlock * F;
    const Op A{make_rsrc(w1 + wofs), make_rsrc(w1 + wofs + 128 * F), (uint32_t)(F * 2)};
    const Op B{make_rsrc(db), make_rsrc(db + kBlock * F), (uint32_t)(F * 2)};
    mainloop<false, false, FA, FB>(acc, A, B, nk, lds);
  }
  {
    const bf16* db = dh3 + t.mt * kBlock * F;
    const Op A{make_rsrc(w3 + wofs), make_rsrc(w3 + wofs + 128 * F), (uint32_t)(F * 2)};
    const Op B{make_rsrc(db), make_rsrc(db + kBlock * F), (uint32_t)(F * 2)};
    mainloop<false, false, FA, FB>(acc, A, B, nk, lds);
  }
  bf16* out = dx_perm + t.mt * kBlock * H + h0;
  for_quads<FA, FB>(acc, lane, [&](int, int arow, int brow, const f32x4& v) {
    store4(out + (int64_t)brow * H + arow, v);
  });
}

__global__ void __launch_bounds__(kThreads)
up_dgrad_kernel(const bf16* __restrict__ dh1, const bf16* __restrict__ dh3,
                const bf16* __restrict__ w1, const bf16* __restrict__ w3, int64_t H,
                int64_t F, ROW_TILE_ARGS, bf16* dx_perm) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  RowTile t;
  if (!row_tile(num_pairs, pair_first, tile_expert, num_padded_rows, (int)((H + 255) / 256), t))
    return;
  DISPATCH2(t.nt * 256 + 256 <= H, t.two,
            (up_dgrad_body<FA, FB>(dh1, dh3, w1, w3, H, F, t, dx_perm, lds)));
}

// dw2[e] = act[rows_e]^T dy_perm[rows_e] ([F,H]); zero for an empty expert.
// A = 256 (or 128) hidden columns of dy_perm, B = 256 (or 128) ffn columns
// of act, K = the expert's padded rows.
template <bool FA, bool FB>
__device__ __forceinline__ void wgrad_down_body(const bf16* act, const bf16* dy_perm,
                                                int64_t H, int64_t F, int64_t start, int n,
                                                int64_t h0, int64_t f0, int e, bf16* dw2,
                                                char* lds) {
  const int lane = threadIdx.x & 63;
  const bf16* ab = dy_perm + start * H + h0;
  const bf16* bb = act + start * F + f0;
  const Op A{make_rsrc(ab), make_rsrc(ab + 128), (uint32_t)(H * 2)};
  const Op B{make_rsrc(bb), make_rsrc(bb + 128), (uint32_t)(F * 2)};
  Acc acc;
  zero(acc);
  mainloop<true, true, FA, FB>(acc, A, B, n / kKStep, lds);
  bf16* out = dw2 + (int64_t)e * F * H + f0 * H + h0;
  for_quads<FA, FB>(acc, lane, [&](int, int arow, int brow, const f32x4& v) {
    store4(out + (int64_t)brow * H + arow, v);
  });
}

__global__ void __launch_bounds__(kThreads)
wgrad_down_kernel(const bf16* __restrict__ act, const bf16* __restrict__ dy_perm,
                  int64_t H, int64_t F, int E, const int32_t* __restrict__ tpe,
                  const int32_t* __restrict__ padded_bins, bf16* __restrict__ dw2) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  // tiles of one expert are consecutive: each XCD works on whole experts
  const int NH = (int)((H + 255) / 256), NF = (int)((F + 255) / 256);
  const int L = xcd_tile(blockIdx.x, E * NH * NF);
  if (L < 0) return;
  const int e = L / (NH * NF);
  const int t = L - e * (NH * NF);
  const int64_t h0 = (int64_t)(t % NH) * 256, f0 = (int64_t)(t / NH) * 256;
  const int n = round_up_block(tpe[e]);
  const int64_t start = padded_bins[e] - n;
  DISPATCH2(h0 + 256 <= H, f0 + 256 <= F,
            (wgrad_down_body<FA, FB>(act, dy_perm, H, F, start, n, h0, f0, e, dw2, lds)));
}

// dw1[e] = x_perm[rows_e]^T dh1[rows_e], dw3[e] = x_perm[rows_e]^T dh3[rows_e]
// ([H,F] each).  A = 128 ffn columns of dh1 (rows 0..127) and the same
// columns of dh3 (rows 128..255), B = 256 (or 128) hidden columns of x_perm.
template <bool FB>
__device__ __forceinline__ void wgrad_up_body(const bf16* x_perm, const bf16* dh1,
                                              const bf16* dh3, int64_t H, int64_t F,
                                              int64_t start, int n, int64_t h0, int64_t f0,
                                              int e, bf16* dw1, bf16* dw3, char* lds) {
  const int lane = threadIdx.x & 63;
  const bf16* xb = x_perm + start * H + h0;
  const Op A{make_rsrc(dh1 + start * F + f0), make_rsrc(dh3 + start * F + f0), (uint32_t)(F * 2)};
  const Op B{make_rsrc(xb), make_rsrc(xb + 128), (uint32_t)(H * 2)};
  Acc acc;
  zero(acc);
  mainloop<true, true, true, FB>(acc, A, B, n / kKStep, lds);
  const int64_t eo = (int64_t)e * H * F + h0 * F + f0;
  for_quads<true, FB>(acc, lane, [&](int, int arow, int brow, const f32x4& v) {
    // A rows 0..127 are dw1 columns, 128..255 the same dw3 columns
    store4((arow < 128 ? dw1 : dw3) + eo + (int64_t)brow * F + (arow & 127), v);
  });
}

__global__ void __launch_bounds__(kThreads)
wgrad_up_kernel(const bf16* __restrict__ x_perm, const bf16* __restrict__ dh1,
                const bf16* __restrict__ dh3, int64_t H, int64_t F, int E,
                const int32_t* __restrict__ tpe, const int32_t* __restrict__ padded_bins,
                bf16* __restrict__ dw1, bf16* __restrict__ dw3) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  const int NF = (int)(F / 128), NH = (int)((H + 255) / 256);
  const int L = xcd_tile(blockIdx.x, E * NF * NH);
  if (L < 0) return;
  const int e = L / (NF * NH);
  const int t = L - e * (NF * NH);
  const int64_t f0 = (int64_t)(t % NF) * 128, h0 = (int64_t)(t / NF) * 256;
  const int n = round_up_block(tpe[e]);
  const int64_t start = padded_bins[e] - n;
  if (h0 + 256 <= H)
    wgrad_up_body<true>(x_perm, dh1, dh3, H, F, start, n, h0, f0, e, dw1, dw3, lds);
  else
    wgrad_up_body<false>(x_perm, dh1, dh3, H, F, start, n, h0, f0, e, dw1, dw3, lds);
}

}  // namespace bfk

static unsigned cdiv_u(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// Enough blocks for every XCD to take ceil(total / 8) tiles.
static dim3 xcd_grid(int64_t total) { return dim3(8u * cdiv_u(total, 8)); }

template <typename T> static const T* cb(const void* p) { return static_cast<const T*>(p); }
template <typename T> static T* mb(void* p) { return static_cast<T*>(p); }

hipError_t launch_bf16_up(const Shape& s, const void* x_perm, const void* w1, const void* w3,
                          const MetaPtrs& m, void* h1, void* h3, void* act,
                          hipStream_t stream) {
  hipLaunchKernelGGL(bfk::up_kernel, xcd_grid(cdiv_u(s.F, 128) * s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, cb<bf16>(x_perm), cb<bf16>(w1),
                     cb<bf16>(w3), s.H, s.F, m.tile_expert, m.num_padded_rows, m.pair_first,
                     m.num_pairs, mb<bf16>(h1), mb<bf16>(h3), mb<bf16>(act));
  return hipGetLastError();
}

hipError_t launch_bf16_down(const Shape& s, const void* act, const void* w2,
                            const MetaPtrs& m, void* y_perm, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::down_kernel, xcd_grid(cdiv_u(s.H, 256) * s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, cb<bf16>(act), cb<bf16>(w2), s.H, s.F,
                     m.tile_expert, m.num_padded_rows, m.pair_first, m.num_pairs,
                     mb<bf16>(y_perm));
  return hipGetLastError();
}

hipError_t launch_bf16_down_dgrad(const Shape& s, const void* dy_perm, const void* w2,
                                  const void* h1, const void* h3, const MetaPtrs& m,
                                  void* dh1, void* dh3, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::down_dgrad_kernel, xcd_grid(cdiv_u(s.F, 256) * s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, cb<bf16>(dy_perm), cb<bf16>(w2),
                     cb<bf16>(h1), cb<bf16>(h3), s.H, s.F, m.tile_expert, m.num_padded_rows,
                     m.pair_first, m.num_pairs, mb<bf16>(dh1), mb<bf16>(dh3));
  return hipGetLastError();
}

hipError_t launch_bf16_up_dgrad(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const MetaPtrs& m,
                                void* dx_perm, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::up_dgrad_kernel, xcd_grid(cdiv_u(s.H, 256) * s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, cb<bf16>(dh1), cb<bf16>(dh3),
                     cb<bf16>(w1), cb<bf16>(w3), s.H, s.F, m.tile_expert, m.num_padded_rows,
                     m.pair_first, m.num_pairs, mb<bf16>(dx_perm));
  return hipGetLastError();
}

hipError_t launch_bf16_wgrad_down(const Shape& s, const void* act, const void* dy_perm,
                                  const MetaPtrs& m, void* dw2, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::wgrad_down_kernel,
                     xcd_grid((int64_t)cdiv_u(s.H, 256) * cdiv_u(s.F, 256) * s.E),
                     dim3(bfk::kThreads), 0, stream, cb<bf16>(act), cb<bf16>(dy_perm), s.H,
                     s.F, s.E, m.tokens_per_expert, m.padded_bins, mb<bf16>(dw2));
  return hipGetLastError();
}

hipError_t launch_bf16_wgrad_up(const Shape& s, const void* x_perm, const void* dh1,
                                const void* dh3, const MetaPtrs& m, void* dw1, void* dw3,
                                hipStream_t stream) {
  hipLaunchKernelGGL(bfk::wgrad_up_kernel,
                     xcd_grid((int64_t)cdiv_u(s.F, 128) * cdiv_u(s.H, 256) * s.E),
                     dim3(bfk::kThreads), 0, stream, cb<bf16>(x_perm), cb<bf16>(dh1),
                     cb<bf16>(dh3), s.H, s.F, s.E, m.tokens_per_expert, m.padded_bins,
                     mb<bf16>(dw1), mb<bf16>(dw3));
  return hipGetLastError();
}

}  // namespace dmoe
