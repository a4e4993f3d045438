// bf16 grouped GEMM over expert-tagged row blocks (gfx950 MFMA).
//
// The products are those of the MegaBlocks chapter "02 · dropless MoE 与
// block-sparse 重构" §3 (sdd: x_perm w1 / x_perm w3, dsd: act w2, on the row
// blocks of each expert only) and their backward, exactly as in the generic
// engine of gemm.hip; this file is the bf16 fast path.
//
// Engine
//   * 512 threads = 8 waves (2 x 4).  A block computes 256 x 256 output
//     tiles: 256 "A rows" along the output's contiguous dimension (weights
//     side) x 256 "B rows" (two 128-row blocks of the same expert, or the m
//     dimension of a weight gradient).  Each wave owns 128 x 64 as 4 x 2
//     v_mfma_f32_32x32x16_bf16 tiles (128 fp32 accumulators); two waves
//     share each SIMD.  The 256 x 256 tile halves the bytes each CU pulls
//     per FLOP compared with 256 x 128, which is what bounds these products.
//     Two products (kFlip: the down projection and the up-projection dgrad)
//     use the other layout, 4 x 2 waves of 64 x 128 each: their A operand
//     then has each fragment read by two waves instead of four, and a tile
//     without its second B half keeps all four SIMDs busy instead of two.
//   * Persistent: one block per CU walks its share of the tiles.  The first
//     two K steps of the next tile are fetched while the current tile
//     finishes and stores its outputs, so neither the start of a block nor
//     the latency of its first loads nor the epilogue idles the matrix cores
//     between tiles.  Tiles are dealt per XCD (block b runs on XCD b % 8, and
//     each XCD has its own L2): each XCD takes one contiguous range of the
//     tile order and its blocks walk it side by side, so concurrent tiles
//     share operands in one L2.
//   * K step 64.  Two LDS stages of 64 KB (32 KB A + 32 KB B) are filled by
//     buffer_load ... lds (16 bytes per lane straight into LDS, no
//     registers).  Each wave fills whole 1 KB LDS blocks; the global address
//     of every lane is chosen so that the LDS image comes out swizzled.
//   * Ping-pong: the two waves of a SIMD run half a phase apart, one issuing
//     the MFMAs of two k-fragments while the other reads its next two from
//     LDS, swapping at a barrier (Pipe::run).
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
//   * A tile whose second half of A or B does not exist (a dimension that is
//     an odd multiple of 128, or an expert with an odd number of row blocks)
//     loads its first half twice, so every wave issues the same loads; the
//     waves of a missing B half skip their MFMAs and no missing half is
//     stored.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <type_traits>

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
constexpr int kStgWave = 4096;                // epilogue staging per wave
constexpr int kLds = 2 * kStage + 8 * kStgWave;   // two stages + staging, 160 KB
constexpr int kDmaPerStep = 8;                // DMA instructions per wave per K step

// Buffer resource: base, no stride, the largest record count, 32-bit data
// format (every access is in bounds by construction, so the range only has
// to cover them).
typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_t;
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ rsrc_t make_rsrc(const char* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return rsrc_t{uniform((uint32_t)a), uniform((uint32_t)(a >> 32) & 0xffffu), 0x7fffffffu,
                0x00020000u};
}
// The same with `bytes` records: a lane whose offset is at or past `bytes`
// reads zeros (the buffer range check), which is how a pad row's token
// row reads as zeros when rows come straight from x.
__device__ __forceinline__ rsrc_t make_rsrc_n(const char* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return rsrc_t{uniform((uint32_t)a), uniform((uint32_t)(a >> 32) & 0xffffu), uniform(bytes),
                0x00020000u};
}
// Offset given to a pad row: past the records of any x of under 2 GB.
constexpr uint32_t kNoRow = 0x80000000u;
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)const_cast<char*>(p);
}

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N vector-memory operations of this
// wave in flight, and every LDS read of this wave completed (so a stage that
// is about to be refilled has no reads of it left in flight).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}
// wait_vm for a count known at run time (wave-uniform), by a binary search
// over the immediates LO..HI; a count outside it waits for everything, which
// is never wrong.
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_range(int n) {
  if constexpr (LO == HI) {
    wait_vm<LO>();
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID) wait_vm_range<LO, MID>(n);
    else wait_vm_range<MID + 1, HI>(n);
  }
}
__device__ __forceinline__ void wait_vm_n(int n) {
  if (n <= 0 || n > 63) wait_vm<0>();
  else wait_vm_range<1, 63>(n);
}
// s_waitcnt lgkmcnt(0) only.
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
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

// 16 bytes per lane from r + voff + soff into LDS at lds + 16 * lane.
// Written as asm so that the compiler does not see an LDS write it cannot
// place: it would then make every transposed LDS read wait for all DMA in
// flight, the prefetch of later steps included.  Completion is awaited
// explicitly (wait_vm + barrier) before a stage is read.  The asm has no
// register outputs.  The nops cover the SGPR-written-by-VALU and M0-write
// hazards of an LDS DMA.
__device__ __forceinline__ void dma16(const rsrc_t& r, uint32_t lds, uint32_t voff,
                                      uint32_t soff) {
  asm volatile(
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(r), "s"(uniform(soff)), "{m0}"(uniform(lds))
      : "memory");
}
// The same with the non-temporal hint, for rows that one block reads once.
__device__ __forceinline__ void dma16_nt(const rsrc_t& r, uint32_t lds, uint32_t voff) {
  asm volatile(
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen nt lds"
      :
      : "v"(voff), "s"(r), "s"(0u), "{m0}"(uniform(lds))
      : "memory");
}

// One operand, one K step into the LDS region at address `reg` (32 KB = 32
// blocks of 1 KB).  Wave w fills blocks 4w..4w+3, all in half w / 4 (p0 or
// p1: the byte address of that half's first row or column).  The base
// address is advanced in 64 bits, so only offsets within one step are 32-bit.
template <bool TRANS>
__device__ __forceinline__ void issue(const char* p0, const char* p1, uint32_t ld,
                                      const Dma<TRANS>& d, int ks, int w, uint32_t reg) {
  const char* p = w < 4 ? p0 : p1;
  if (!TRANS)
    p += (uint64_t)(32 * (w & 3)) * ld + (uint64_t)ks * kRowB;   // 32 rows, this k range
  else
    p += (uint64_t)(ks * kKStep + 16 * (w & 3)) * ld;            // 16 k-rows
  const rsrc_t r = make_rsrc(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t soff = (uint32_t)(TRANS ? 4 * i : 8 * i) * ld;
    dma16(r, reg + (4 * w + i) * 1024, TRANS ? d.voff[0] : d.voff[i & 1], soff);
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

template <bool ATR, bool BTR>
__device__ __forceinline__ void load_frags(Frags& f, const char* stage, int kf, int wm, int wn,
                                           int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) f.b[j] = frag<BTR>(stage + kReg, b_row(j, wn), kf, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = frag<ATR>(stage, a_row(i, wm), kf, lane);
}

__device__ __forceinline__ void mma(Acc& acc, const Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// The flipped layout (K::kFlip): wave (wm, wn) owns A rows wn*64 + 32i (i <
// 2) and B rows wm*128 + 32j (j < 4), so the two waves of a SIMD (same wn)
// split the B rows and a missing B half (wm = 1) idles one wave per SIMD.
// Per K step a wave reads 8 A and 16 B fragments against 16 and 8: with a
// transposed A (two ds_read_b64_tr_b16 per fragment) that is 32 LDS read
// instructions instead of 40.  Measured: the down projection 2-3% faster on
// the fine-grained and the 256-expert layers, the up-projection dgrad about
// 1%, the coarse layer level; the sums are the same MFMAs in the same order,
// so the results are bit-identical.  The up projection keeps the first
// layout: its gate pairs each H1 column with the same H3 column in one wave.
struct FragsF {
  bf16x8 a[2];
  bf16x8 b[4];
};
template <bool ATR, bool BTR>
__device__ __forceinline__ void load_frags_f(FragsF& f, const char* stage, int kf, int wm, int wn,
                                             int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = frag<BTR>(stage + kReg, wm * 128 + j * 32, kf, lane);
#pragma unroll
  for (int i = 0; i < 2; ++i) f.a[i] = frag<ATR>(stage, wn * 64 + i * 32, kf, lane);
}
// accumulator (i, j) of the flipped layout lives in acc[2i + j/2][j%2]
__device__ __forceinline__ void mma_f(Acc& acc, const FragsF& f) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[2 * i + (j >> 1)][j & 1] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[2 * i + (j >> 1)][j & 1], 0, 0, 0);
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
__device__ __forceinline__ f32x4 unpack4(const u32x2& u) {
  return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint16_t, from_f32<bf16>(a)) |
         ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(b)) << 16);
}

// ---- Epilogue stores through LDS ------------------------------------------------
// A wave's outputs of one A half form a 64 (B rows) x 64 (A rows) block, A
// rows contiguous in memory.  In accumulator layout a store instruction would
// touch 32 rows with 16 bytes each; instead the wave writes 32 B rows at a
// time to its own 4 KB of LDS and reads them back as whole rows, so each
// store instruction writes 8 full 128-byte rows.  Row r sits at 128 r with
// its 16-byte chunk c at c ^ ((r >> 1) & 7) (the 32 rows written by one
// instruction spread over all banks but for a factor of two).  The global
// stores carry the non-temporal hint: no kernel reads an output while it is
// being written, and the hint measured about 1% off the layer's step.
__device__ __forceinline__ u32x2 pack4(const f32x4& v) {
  return u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
}

// Stores per wave of one stage_pass call and of one stage_out call.
constexpr int kStoresPerPass = 4;
constexpr int kStoresPerBlock = 2 * kStoresPerPass;

// The lane index through an opaque move: the addresses of the staging code
// depend on the lane only, and would otherwise be hoisted out of the tile
// loop and kept in registers across the whole K loop.
__device__ __forceinline__ int opaque_lane(int lane_in) {
  int lane;
  asm volatile("v_mov_b32 %0, %1" : "=v"(lane) : "v"(lane_in));
  return lane;
}

// Byte offset in a 32-row staging region of the 4 values (8 bytes) that lane
// `lane` holds in accumulator layout for A block ii, quad g.
__device__ __forceinline__ int acc_slot(int lane, int ii, int g) {
  const int r = lane & 31;
  const int col = ii * 32 + 8 * g + 4 * (lane >> 5);
  return r * 128 + (((col >> 3) ^ ((r >> 1) & 7)) << 4) + ((col >> 2) & 1) * 8;
}

// B rows [32 j, 32 j + 32) of the wave's block.  out: element (B row 0, A row
// 0) of the block; ldo: elements between B rows.  val(ii, g): the 4 values
// (bf16, packed) of A block ii (0/1 in the half), B block j, quad g, in
// accumulator layout.  st: the wave's staging space.
template <class Val>
__device__ __forceinline__ int stage_pass(char* st, bf16* out, int64_t ldo, int lane_in, int j,
                                          Val&& val) {
  const int lane = opaque_lane(lane_in);
  wait_lds();   // the reads of the previous rows are done
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<u32x2*>(st + acc_slot(lane, ii, g)) = val(ii, g);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = it * 8 + (lane >> 3), c = lane & 7;
    const u32x4 v = *reinterpret_cast<const u32x4*>(st + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + (int64_t)(j * 32 + r) * ldo + c * 8));
  }
  return kStoresPerPass;
}
// The whole block: val(ii, j, g).
template <class Val>
__device__ __forceinline__ int stage_out(char* st, bf16* out, int64_t ldo, int lane, Val&& val) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
    stage_pass(st, out, ldo, lane, j, [&](int ii, int g) { return val(ii, j, g); });
  return kStoresPerBlock;
}

// 32 rows x 64 elements (128 bytes each, `ld` bytes apart, from `src`) into a
// 4 KB LDS region at `lds` by DMA, in the swizzled layout of the staging
// space: LDS row r holds source row r with its chunk c at c ^ ((r >> 1) & 7).
// Each such row is read by one block only, so the loads are non-temporal.
__device__ __forceinline__ void dma_rows(const char* src, uint32_t ld, uint32_t lds, int lane) {
  const rsrc_t rs = make_rsrc(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = i * 8 + (lane >> 3), pc = lane & 7;
    const int c = pc ^ ((r >> 1) & 7);
    dma16_nt(rs, lds + i * 1024, (uint32_t)r * ld + (uint32_t)c * 16u);
  }
}

// LDS space of one wave for its epilogue: `stg` is its own 4 KB; `a` and `b`
// (LDS addresses `a_addr`, `b_addr`) are the 4 KB blocks its DMA fills in the
// stage the last K step used -- free until step 1 of the next tile is
// started, which happens after the epilogue only for products with
// kLateStep1.
struct Epi {
  char* stg;
  const char* a;
  const char* b;
  uint32_t a_addr, b_addr;
};

// The common case: A half h of the accumulators, stored as they are.
__device__ __forceinline__ int stage_half(char* st, const Acc& acc, int h, bf16* out,
                                          int64_t ldo, int lane) {
  return stage_out(st, out, ldo, lane,
                   [&](int ii, int j, int g) { return pack4(quad(acc[2 * h + ii][j], g)); });
}

// ---- Tiles ------------------------------------------------------------------
// One output tile: `steps` K steps in one or two segments of `nk` steps (the
// up-projection dgrad sums two products).  u, v and e are read by the
// kernel's own operand and epilogue code.
struct Job {
  int steps, nk;
  int kind;         // which product of a merged launch (0 or 1)
  int e;            // expert
  int start;        // weight gradients: the expert's first padded row
  bool fa, fb;      // second half of A / B present
  int64_t u, v;     // tile coordinates
};

constexpr int kGroupM = 8;

// k-fragments per phase of the main loop: two (16 MFMAs per wave) measured
// faster than one; four would need four fragment sets, more VGPRs than two
// waves per SIMD leave.
constexpr int kPhaseFrags = 2;

static_assert(kPhaseFrags == 1 || kPhaseFrags == 2, "one or two fragments per phase");

// The pair of row blocks (u = first 128-row block) and the column tile (v)
// of logical row tile L, from the live metadata.  The pairs of each expert
// (consecutive, from its first block) are split into ceil(p / kGroupM)
// groups of near-equal size; a group of gm pairs from pair g0 owns logical
// tiles [g0 NT, (g0 + gm) NT), walked column by column (pair g0 + r % gm,
// column r / gm), so that concurrent blocks share one expert's weight
// columns and its token rows.
struct RowTiles {
  const int32_t *tile_expert, *pair_first, *padded_bins;
  int pairs, NT;
  __device__ __forceinline__ void init(const int32_t* te, const int32_t* pf,
                                       const int32_t* num_pairs, const int32_t* pb, int nt) {
    tile_expert = te;
    pair_first = pf;
    padded_bins = pb;
    pairs = *num_pairs;
    NT = nt;
  }
  __device__ __forceinline__ int total() const { return pairs * NT; }
  // every tile has the same K: equal shares
  __device__ __forceinline__ void xcd_range(int x, int& lo, int& hi) const {
    const int per = (total() + 7) / 8;
    lo = min(total(), x * per);
    hi = min(total(), lo + per);
  }
  __device__ __forceinline__ void get(int L, Job& j) const {
    const int q = L / NT;                 // a pair of L's group
    const int mq = pair_first[q];
    const int e = tile_expert[mq];
    const int b0 = e > 0 ? padded_bins[e - 1] / kBlock : 0;   // the expert's blocks [b0, b1)
    const int b1 = padded_bins[e] / kBlock;
    const int pe = (b1 - b0 + 1) / 2;     // its pairs, the first one se
    const int se = q - (mq - b0) / 2;
    const int ng = (pe + kGroupM - 1) / kGroupM;
    // group gi = [se + ceil(gi pe / ng), se + ceil((gi + 1) pe / ng)) holds q
    const int gi = (q - se) * ng / pe;
    const int g0 = se + (gi * pe + ng - 1) / ng;
    const int gm = se + ((gi + 1) * pe + ng - 1) / ng - g0;
    const int r = L - g0 * NT;
    const int m = b0 + 2 * (g0 - se + r % gm);
    j.e = e;
    j.fb = m + 1 < b1;
    j.u = m;
    j.v = r / gm;
  }
};

#define ROW_TILE_ARGS                                                              \
  const int32_t *__restrict__ tile_expert, const int32_t *__restrict__ pair_first, \
      const int32_t *__restrict__ num_pairs, const int32_t *__restrict__ padded_bins

// ---- The products, as operand + epilogue policies ----------------------------

// Where a product's B operand comes from: its own array (kXNone), or token
// rows of x fetched straight into the tile, the gather fused into the operand
// loads (kXDirect, B rows are padded rows with K along the row): padded row p
// is row row_token[p] of x, zeros for a pad row (row_token < 0).
enum XMode { kXNone, kXDirect };

struct XRows {
  const bf16* x;              // [T, H]
  const int32_t* row_token;   // [P]
  uint32_t bytes;             // T * H * 2, below 2 GB
};

// h1 = x_perm w1[e], h3 = x_perm w3[e], act = silu(h1) * h3 for one pair of
// row blocks and 128 ffn columns (w1 columns in A rows 0..127, the same w3
// columns in A rows 128..255, so A blocks i and i+2 pair up).  X: the rows of
// x_perm come straight from x (xr).
template <bool X>
struct UpT {
  static constexpr bool kLateStep1 = false;
  static constexpr bool kUsesFreeStage = false;
  static constexpr bool kFlip = false;
  static constexpr bool ATR = true, BTR = false;
  static constexpr XMode kXB = X ? kXDirect : kXNone;
  const bf16 *x_perm, *w1, *w3;
  int64_t H, F;
  bf16 *h1, *h3, *act;
  RowTiles rt;
  XRows xr;
  // first padded row of the 32 B rows that wave w loads
  __device__ int64_t x_rows(const Job& j, int w) const {
    return j.u * kBlock + (w < 4 ? 0 : (j.fb ? kBlock : 0)) + 32 * (w & 3);
  }
  __device__ uint32_t lda() const { return (uint32_t)(F * 2); }
  __device__ uint32_t ldb() const { return (uint32_t)(H * 2); }
  __device__ void xcd_range(int x, int& lo, int& hi) const { rt.xcd_range(x, lo, hi); }
  __device__ void tile(int L, Job& j) const {
    rt.get(L, j);
    j.fa = true;
    j.nk = j.steps = (int)(H / kKStep);
  }
  __device__ void operands(const Job& j, int, const char*& a0, const char*& a1, const char*& b0,
                           const char*& b1) const {
    const int64_t wofs = (int64_t)j.e * H * F + j.v * 128;
    a0 = (const char*)(w1 + wofs);
    a1 = (const char*)(w3 + wofs);
    b0 = (const char*)(x_perm + j.u * kBlock * H);
    b1 = j.fb ? b0 + kBlock * H * 2 : b0;
  }
  __device__ int epilogue(const Job& j, const Acc& acc, const Epi& ep) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;
    if (!j.fb && wn >= 2) return 0;
    const int64_t o = j.u * kBlock * F + j.v * 128 + (int64_t)(wn * 64) * F + wm * 64;
    stage_half(ep.stg, acc, 0, h1 + o, F, lane);
    stage_half(ep.stg, acc, 1, h3 + o, F, lane);
    // act from the stored (bf16-rounded) h1 and h3
    return 2 * kStoresPerBlock + stage_out(ep.stg, act + o, F, lane, [&](int ii, int jj, int g) {
      const f32x4 v1 = unpack4(pack4(quad(acc[ii][jj], g)));
      const f32x4 v3 = unpack4(pack4(quad(acc[2 + ii][jj], g)));
      f32x4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = gated_silu(v1[r], v3[r]);
      return pack4(a);
    });
  }
};

using Up = UpT<false>;

// y_perm = act w2[e] for one pair of row blocks and 256 (or 128) hidden columns.
struct Down {
  static constexpr bool kLateStep1 = false;
  static constexpr bool kUsesFreeStage = false;
  static constexpr bool kFlip = true;
  static constexpr bool ATR = true, BTR = false;
  static constexpr XMode kXB = kXNone;
  const bf16 *act, *w2;
  int64_t H, F;
  bf16* y_perm;
  RowTiles rt;
  __device__ uint32_t lda() const { return (uint32_t)(H * 2); }
  __device__ uint32_t ldb() const { return (uint32_t)(F * 2); }
  __device__ void xcd_range(int x, int& lo, int& hi) const { rt.xcd_range(x, lo, hi); }
  __device__ void tile(int L, Job& j) const {
    rt.get(L, j);
    j.fa = j.v * 256 + 256 <= H;
    j.nk = j.steps = (int)(F / kKStep);
  }
  __device__ void operands(const Job& j, int, const char*& a0, const char*& a1, const char*& b0,
                           const char*& b1) const {
    a0 = (const char*)(w2 + (int64_t)j.e * F * H + j.v * 256);
    a1 = j.fa ? a0 + 128 * 2 : a0;
    b0 = (const char*)(act + j.u * kBlock * F);
    b1 = j.fb ? b0 + kBlock * F * 2 : b0;
  }
  __device__ int epilogue(const Job& j, const Acc& acc, const Epi& ep) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;
    // flipped layout: hidden columns wn*64 .. +64 of the tile, token rows wm*128 .. +128
    if (!j.fb && wm == 1) return 0;
    if (!j.fa && wn >= 2) return 0;
    bf16* out = y_perm + j.u * kBlock * H + j.v * 256 + (int64_t)(wm * 128) * H + wn * 64;
    int n = 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      n += stage_pass(ep.stg, out, H, lane, jj, [&](int ii, int g) {
        return pack4(quad(acc[2 * ii + (jj >> 1)][jj & 1], g));
      });
    return n;
  }
};

// dA = dy_perm w2[e]^T, then the gate's backward:
// dh3 = dA * silu(h1), dh1 = dA * h3 * s * (1 + h1 (1 - s)), s = sigmoid(h1).
struct DownDgrad {
  // step 1 of the next tile is issued after the epilogue, which uses the
  // free stage to bring in h1 and h3
  static constexpr bool kLateStep1 = true;
  static constexpr bool kUsesFreeStage = true;
  static constexpr bool kFlip = false;
  static constexpr bool ATR = false, BTR = false;
  static constexpr XMode kXB = kXNone;
  const bf16 *dy_perm, *w2, *h1, *h3;
  int64_t H, F;
  bf16 *dh1, *dh3;
  RowTiles rt;
  __device__ uint32_t lda() const { return (uint32_t)(H * 2); }
  __device__ uint32_t ldb() const { return (uint32_t)(H * 2); }
  static constexpr int kEpiSteps = 4;   // h1, h3 in and dh1, dh3 out: ~4 K steps of traffic
  __device__ int tile_steps() const { return (int)(H / kKStep); }
  __device__ void xcd_range(int x, int& lo, int& hi) const { rt.xcd_range(x, lo, hi); }
  __device__ void tile(int L, Job& j) const {
    rt.get(L, j);
    j.fa = j.v * 256 + 256 <= F;
    j.nk = j.steps = (int)(H / kKStep);
  }
  __device__ void operands(const Job& j, int, const char*& a0, const char*& a1, const char*& b0,
                           const char*& b1) const {
    a0 = (const char*)(w2 + (int64_t)j.e * F * H + j.v * 256 * H);
    a1 = j.fa ? a0 + 128 * H * 2 : a0;
    b0 = (const char*)(dy_perm + j.u * kBlock * H);
    b1 = j.fb ? b0 + kBlock * H * 2 : b0;
  }
  __device__ int epilogue(const Job& j, const Acc& acc, const Epi& ep) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;
    if (!j.fb && wn >= 2) return 0;
    const int64_t base = j.u * kBlock * F + j.v * 256;
    const int64_t wo = base + (int64_t)(wn * 64) * F + wm * 64;
    // h1 and h3 come in 32-row passes (two per A half) by DMA into the two
    // free 4 KB blocks of this wave, in the staging layout, and are read back
    // in accumulator layout; the DMA of the next pass is in flight while one
    // is computed and stored.  dh1/dh3 may alias h1/h3: every element is read
    // before the pass that overwrites it is stored, and passes are disjoint.
    const int npass = j.fa ? 4 : 2;
    const uint32_t ld = (uint32_t)(F * 2);
    const auto src = [&](const bf16* t, int q) {
      return reinterpret_cast<const char*>(t + wo + (q >> 1) * 128 + (int64_t)((q & 1) * 32) * F);
    };
    dma_rows(src(h1, 0), ld, ep.a_addr, lane);
    dma_rows(src(h3, 0), ld, ep.b_addr, lane);
    int n = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q >= npass) break;
      const int h = q >> 1, jr = q & 1;
      // pass q landed (younger: the stores of pass q - 1)
      if (q == 0) wait_vm<0>(); else wait_vm<2 * kStoresPerPass>();
      u32x2 g1[2][4], g3[2][4];
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          g1[ii][g] = *reinterpret_cast<const u32x2*>(ep.a + acc_slot(lane, ii, g));
          g3[ii][g] = *reinterpret_cast<const u32x2*>(ep.b + acc_slot(lane, ii, g));
        }
      wait_lds();
      if (q + 1 < npass) {
        dma_rows(src(h1, q + 1), ld, ep.a_addr, lane);
        dma_rows(src(h3, q + 1), ld, ep.b_addr, lane);
      }
      // dh3 = dA * silu(h1), dh1 = dA * h3 * s * (1 + h1 (1 - s)), s = sigmoid(h1)
      u32x2 d1[2][4], d3[2][4];
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 da = quad(acc[2 * h + ii][jr], g), x1 = unpack4(g1[ii][g]),
                      x3 = unpack4(g3[ii][g]);
          f32x4 v1, v3;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sg = sigmoid(x1[r]);
            v3[r] = da[r] * x1[r] * sg;
            v1[r] = da[r] * x3[r] * sg * (1.0f + x1[r] * (1.0f - sg));
          }
          d1[ii][g] = pack4(v1);
          d3[ii][g] = pack4(v3);
        }
      n += stage_pass(ep.stg, dh1 + wo + h * 128, F, lane, jr,
                      [&](int ii, int g) { return d1[ii][g]; });
      n += stage_pass(ep.stg, dh3 + wo + h * 128, F, lane, jr,
                      [&](int ii, int g) { return d3[ii][g]; });
    }
    return n;
  }
};

// dx_perm = dh1 w1[e]^T + dh3 w3[e]^T: two K segments into one accumulator
// (one, dh1 w1[e]^T, when `two` is false: the dgrad of a single grouped
// linear map).
struct UpDgrad {
  static constexpr bool kLateStep1 = false;
  static constexpr bool kUsesFreeStage = false;
  static constexpr bool kFlip = true;
  static constexpr bool ATR = false, BTR = false;
  static constexpr XMode kXB = kXNone;
  const bf16 *dh1, *dh3, *w1, *w3;
  int64_t H, F;
  bf16* dx_perm;
  RowTiles rt;
  bool two = true;
  __device__ uint32_t lda() const { return (uint32_t)(F * 2); }
  __device__ uint32_t ldb() const { return (uint32_t)(F * 2); }
  static constexpr int kEpiSteps = 2;
  __device__ int tile_steps() const { return (int)((two ? 2 : 1) * F / kKStep); }
  __device__ void xcd_range(int x, int& lo, int& hi) const { rt.xcd_range(x, lo, hi); }
  __device__ void tile(int L, Job& j) const {
    rt.get(L, j);
    j.fa = j.v * 256 + 256 <= H;
    j.nk = (int)(F / kKStep);
    j.steps = two ? 2 * j.nk : j.nk;
  }
  __device__ void operands(const Job& j, int seg, const char*& a0, const char*& a1,
                           const char*& b0, const char*& b1) const {
    const int64_t wofs = (int64_t)j.e * H * F + j.v * 256 * F;
    a0 = (const char*)((seg ? w3 : w1) + wofs);
    a1 = j.fa ? a0 + 128 * F * 2 : a0;
    b0 = (const char*)((seg ? dh3 : dh1) + j.u * kBlock * F);
    b1 = j.fb ? b0 + kBlock * F * 2 : b0;
  }
  __device__ int epilogue(const Job& j, const Acc& acc, const Epi& ep) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;
    // flipped layout: hidden columns wn*64 .. +64 of the tile, token rows wm*128 .. +128
    if (!j.fb && wm == 1) return 0;
    if (!j.fa && wn >= 2) return 0;
    bf16* out = dx_perm + j.u * kBlock * H + j.v * 256 + (int64_t)(wm * 128) * H + wn * 64;
    int n = 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      n += stage_pass(ep.stg, out, H, lane, jj, [&](int ii, int g) {
        return pack4(quad(acc[2 * ii + (jj >> 1)][jj & 1], g));
      });
    return n;
  }
};

// Weight-gradient tiles have K = the expert's padded rows, so equal tile
// counts are not equal work under skewed routing.  Expert e costs its 128-row
// blocks + 1 (its K steps plus an epilogue of about two K steps, in units of
// two K steps), so that the experts before e cost pre(e) = padded_bins[e - 1]
// / 128 + e and all of them W = pre(E).  The tiles of expert e are
// consecutive in the tile order and share its cost equally; XCD x computes
// the tiles whose cost lies in [x W / 8, (x + 1) W / 8), so every XCD gets
// an eighth of the work up to one tile, and an expert may straddle two XCDs
// (both then fetch its rows: one expert per boundary).  Every block of every
// launch derives the same ranges from padded_bins.
struct CostSplit {
  const int32_t* padded_bins;
  int E;
  __device__ int pre(int e) const { return e == 0 ? 0 : padded_bins[e - 1] / kBlock + e; }
  // the tile that holds cost position c, or E * tpe for c >= W
  __device__ int tile_at(int64_t c, int tpe) const {
    if (c >= pre(E)) return E * tpe;
    int a = 0, z = E - 1;                 // the last expert with pre(e) <= c
    while (a < z) {
      const int mid = (a + z + 1) >> 1;
      if (pre(mid) <= c) a = mid; else z = mid - 1;
    }
    const int p0 = pre(a);
    return a * tpe + (int)((c - p0) * tpe / (pre(a + 1) - p0));
  }
  __device__ void range(int x, int tpe, int& lo, int& hi) const {
    const int64_t W = pre(E);
    lo = tile_at(x * W / 8, tpe);
    hi = tile_at((x + 1) * W / 8, tpe);
  }
};

// dw2[e] = act[rows_e]^T dy_perm[rows_e] ([F,H]); zero for an empty expert.
// A = 256 (or 128) hidden columns of dy_perm (u = h0), B = 256 (or 128) ffn
// columns of act (v = f0), K = the expert's padded rows.
struct WgradDown {
  static constexpr bool kLateStep1 = false;
  static constexpr bool kUsesFreeStage = false;
  static constexpr bool kFlip = false;
  static constexpr bool ATR = true, BTR = true;
  static constexpr XMode kXB = kXNone;
  const bf16 *act, *dy_perm;
  int64_t H, F;
  int E;
  const int32_t *tpe, *padded_bins;
  bf16* dw2;
  __device__ uint32_t lda() const { return (uint32_t)(H * 2); }
  __device__ uint32_t ldb() const { return (uint32_t)(F * 2); }
  __device__ int nh() const { return (int)((H + 255) / 256); }
  __device__ int nf() const { return (int)((F + 255) / 256); }
  static constexpr int kEpiSteps = 2;
  __device__ int tiles_per_expert() const { return nh() * nf(); }
  __device__ int expert_steps(int e) const { return round_up_block(tpe[e]) / kKStep; }
  __device__ void xcd_range(int x, int& lo, int& hi) const {
    CostSplit{padded_bins, E}.range(x, tiles_per_expert(), lo, hi);
  }
  __device__ void tile(int L, Job& j) const {
    // the tiles of one expert are consecutive: each XCD works on whole experts
    const int NH = nh(), NF = nf();
    const int e = L / (NH * NF);
    const int t = L - e * (NH * NF);
    j.u = (int64_t)(t % NH) * 256;
    j.v = (int64_t)(t / NH) * 256;
    j.fa = j.u + 256 <= H;
    j.fb = j.v + 256 <= F;
    const int n = round_up_block(tpe[e]);
    j.nk = j.steps = n / kKStep;
    j.e = e;
    j.start = padded_bins[e] - n;
  }
  __device__ void operands(const Job& j, int, const char*& a0, const char*& a1, const char*& b0,
                           const char*& b1) const {
    const int64_t start = j.start;
    a0 = (const char*)(dy_perm + start * H + j.u);
    a1 = j.fa ? a0 + 128 * 2 : a0;
    b0 = (const char*)(act + start * F + j.v);
    b1 = j.fb ? b0 + 128 * 2 : b0;
  }
  __device__ int epilogue(const Job& j, const Acc& acc, const Epi& ep) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;
    if (!j.fb && wn >= 2) return 0;
    bf16* out = dw2 + (int64_t)j.e * F * H + j.v * H + j.u + (int64_t)(wn * 64) * H +
                wm * 64;
    int n = stage_half(ep.stg, acc, 0, out, H, lane);
    if (j.fa) n += stage_half(ep.stg, acc, 1, out + 128, H, lane);
    return n;
  }
};

// dw1[e] = x_perm[rows_e]^T dh1[rows_e], dw3[e] = x_perm[rows_e]^T dh3[rows_e]
// ([H,F] each).  A = 128 ffn columns of dh1 (rows 0..127) and the same
// columns of dh3 (rows 128..255) (u = f0), B = 256 (or 128) hidden columns
// of x_perm (v = h0).
struct WgradUp {
  static constexpr bool kLateStep1 = false;
  static constexpr bool kUsesFreeStage = false;
  static constexpr bool kFlip = false;
  static constexpr bool ATR = true, BTR = true;
  static constexpr XMode kXB = kXNone;
  const bf16 *x_perm, *dh1, *dh3;
  int64_t H, F;
  int E;
  const int32_t *tpe, *padded_bins;
  bf16 *dw1, *dw3;
  __device__ uint32_t lda() const { return (uint32_t)(F * 2); }
  __device__ uint32_t ldb() const { return (uint32_t)(H * 2); }
  __device__ int nf() const { return (int)(F / 128); }
  __device__ int nh() const { return (int)((H + 255) / 256); }
  static constexpr int kEpiSteps = 2;
  __device__ int tiles_per_expert() const { return nf() * nh(); }
  __device__ int expert_steps(int e) const { return round_up_block(tpe[e]) / kKStep; }
  __device__ void xcd_range(int x, int& lo, int& hi) const {
    CostSplit{padded_bins, E}.range(x, tiles_per_expert(), lo, hi);
  }
  __device__ void tile(int L, Job& j) const {
    const int NF = nf(), NH = nh();
    const int e = L / (NF * NH);
    const int t = L - e * (NF * NH);
    j.u = (int64_t)(t % NF) * 128;
    j.v = (int64_t)(t / NF) * 256;
    j.fa = true;
    j.fb = j.v + 256 <= H;
    const int n = round_up_block(tpe[e]);
    j.nk = j.steps = n / kKStep;
    j.e = e;
    j.start = padded_bins[e] - n;
  }
  __device__ void operands(const Job& j, int, const char*& a0, const char*& a1, const char*& b0,
                           const char*& b1) const {
    const int64_t start = j.start;
    a0 = (const char*)(dh1 + start * F + j.u);
    a1 = (const char*)(dh3 + start * F + j.u);
    b0 = (const char*)(x_perm + start * H + j.v);
    b1 = j.fb ? b0 + 128 * 2 : b0;
  }
  __device__ int epilogue(const Job& j, const Acc& acc, const Epi& ep) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;
    if (!j.fb && wn >= 2) return 0;
    // A rows 0..127 are dw1 columns, 128..255 the same dw3 columns
    const int64_t o = (int64_t)j.e * H * F + j.v * F + j.u + (int64_t)(wn * 64) * F +
                      wm * 64;
    return stage_half(ep.stg, acc, 0, dw1 + o, F, lane) + stage_half(ep.stg, acc, 1, dw3 + o, F, lane);
  }
};

// ---- The persistent pipeline ---------------------------------------------------

template <class K>
struct Pipe {
  const K& k;
  char* lds;            // the two stages
  uint32_t lbase;       // their LDS address
  int g;                // K steps run so far by this block (selects the stage)
  int w, wm, wn, lane;
  Dma<K::ATR> da;
  Dma<K::BTR> db;
  // B rows straight from x (K::kXB == kXDirect): na holds the padded-row ->
  // token lookup of the next tile's 32 rows of this wave (one vector load,
  // issued a tile ahead by lookup()); boff, this tile's row offsets, worked
  // out from it at step 0.  The lookup is read only after an explicit wait
  // that covers it: the compiler cannot see the DMA, so a wait of its own
  // there would be for all vector memory in flight, the DMA included.
  uint32_t na = 0;
  uint32_t boff[4] = {0u, 0u, 0u, 0u};

  __device__ __forceinline__ uint32_t stage_addr(int s) const { return lbase + (s & 1) * kStage; }

  // Issues tile j's first lookups; returns the vector-memory operations
  // issued (they are younger than everything in flight).
  __device__ __forceinline__ int lookup(const Job& j) {
    if constexpr (K::kXB == kXDirect) {
      na = (uint32_t)k.xr.row_token[k.x_rows(j, w) + (lane & 31)];
      return 1;
    } else {
      return 0;
    }
  }
  __device__ __forceinline__ const char* stage_ptr(int s) const { return lds + (s & 1) * kStage; }

  // DMA of step s of tile j into the stage of this block's step gs.
  __device__ __forceinline__ void issue_step(const Job& j, int s, int gs) {
    const int seg = s >= j.nk ? 1 : 0;
    const int ks = s - seg * j.nk;
    const char *a0, *a1, *b0, *b1;
    k.operands(j, seg, a0, a1, b0, b1);
    const uint32_t st = stage_addr(gs);
    // B rows straight from x: the lanes fill the same LDS image as issue<>,
    // each from its row's token row of x (a pad row's offset is past the
    // records of x).  The offsets are worked out before any DMA of this
    // step goes out (see na).
    uint32_t off[4];
    if constexpr (K::kXB == kXDirect) {
      // instruction i, lane l: B row 8i + l/8 of the wave's 32, physical
      // chunk l%8 (the direct swizzle of a block of parity i%2)
      const uint32_t ld = k.ldb();
      if (s == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = __builtin_amdgcn_ds_bpermute((8 * i + (lane >> 3)) << 2, (int)na);
          const uint32_t c = (uint32_t)((lane & 7) ^ (lane >> 3) ^ (i & 1)) << 4;
          boff[i] = (tok >= 0 ? (uint32_t)tok * ld : kNoRow) + c;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) off[i] = boff[i] + (uint32_t)ks * kRowB;
    }
    issue<K::ATR>(a0, a1, k.lda(), da, ks, w, st);
    if constexpr (K::kXB == kXNone) {
      issue<K::BTR>(b0, b1, k.ldb(), db, ks, w, st + kReg);
    } else {
      const rsrc_t r = make_rsrc_n(reinterpret_cast<const char*>(k.xr.x), k.xr.bytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16(r, st + kReg + (4 * w + i) * 1024, off[i], 0u);
    }
  }

  // The K loop of one tile for one group of waves (G0: wm == 0), after the
  // barrier that follows the landing of step 0.  The two waves of each SIMD
  // (wm = 0 and wm = 1 share one) run half a phase apart: while one issues
  // the MFMAs of two k-fragments, the other reads its next two fragments
  // from LDS, and they swap at a barrier, so the matrix core and the LDS are
  // each kept busy by one wave at a time.  With chunk c = 2s + h (k-
  // fragments 2h, 2h + 1 of step s), group 0 computes c in phase 2c and
  // reads c + 1 in phase 2c + 1; group 1 reads c in phase 2c and computes it
  // in phase 2c + 1.  Stage s is last read in phase 4s + 2; at its end every
  // wave waits for its DMA of step s + 1 (for s = 0 letting w1 younger
  // operations stay in flight), and after that barrier each wave starts its
  // DMA of step s + 2 -- past the end of the tile, step 0 of `nxt`, by
  // next(gs), which may belong to another product -- in its next read
  // phase.  Both groups run the same barriers: one after every phase but
  // the last, so group 0 goes on to its stores while group 1 runs the last
  // phase's MFMAs.  Group 0 reads chunk 0 first (its phase 0 computes it).
  template <bool G0, class Next>
  __device__ __forceinline__ void group_loop(Acc& acc, const Job& cur, const Job& nxt, int w1,
                                             Next&& next) {
    constexpr int PF = kPhaseFrags;          // fragments per phase
    constexpr int NP = 4 / PF;               // phases of each kind per step
    const int n = cur.steps;
    const bool work = K::kFlip ? (cur.fb || wm == 0) : (cur.fb || wn < 2);
    // the DMA of step t >= 2 (or of the next tile's step 0 when t == n)
    const auto dma = [&](int t) {
      if (t < n) issue_step(cur, t, g + t);
      else if (t == n && nxt.steps > 0) next(g + t);
    };
    std::conditional_t<K::kFlip, FragsF, Frags> f[2];
    const auto load = [&](const char* st, int q) {   // fragments of chunk q of a step
      if (work)
#pragma unroll
        for (int i = 0; i < PF; ++i) {
          if constexpr (K::kFlip)
            load_frags_f<K::ATR, K::BTR>(f[(q * PF + i) & 1], st, q * PF + i, wm, wn, lane);
          else
            load_frags<K::ATR, K::BTR>(f[(q * PF + i) & 1], st, q * PF + i, wm, wn, lane);
        }
    };
    const auto compute = [&](int q) {
      if (work) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < PF; ++i) {
          if constexpr (K::kFlip) mma_f(acc, f[(q * PF + i) & 1]);
          else mma(acc, f[(q * PF + i) & 1]);
        }
        __builtin_amdgcn_s_setprio(0);
      }
    };
    if (G0) load(stage_ptr(g), 0);
    for (int s = 0; s < n; ++s) {
      const char* cst = stage_ptr(g + s);
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        // group 0 computes chunk q, group 1 reads it
        sched_fence();
        if (G0) {
          compute(q);
        } else {
          if (q == 0 && s > 0) dma(s + 1);
          load(cst, q);
          wait_lds();
        }
        sched_fence();
        if (q == NP - 1 && s + 1 < n) {     // the last read of step s: step s + 1 landed
          if (s == 0) wait_vm_n(w1); else wait_vm<0>();
        }
        barrier();
        // group 0 reads the next chunk, group 1 computes chunk q
        sched_fence();
        if (G0) {
          if (q < NP - 1) {
            load(cst, q + 1);
          } else if (s + 1 < n) {
            dma(s + 2);
            load(stage_ptr(g + s + 1), 0);
          }
          wait_lds();
        } else {
          compute(q);
        }
        sched_fence();
        if (s + 1 < n || q + 1 < NP) barrier();
      }
    }
  }
};

// The products of one launch as the engine sees them: K1 alone (kTwo =
// false), or K1 and K2 chosen per tile by Job::kind.
template <class K1, class K2, bool kTwo>
struct Ops {
  const K1& k1;
  const K2& k2;
  Pipe<K1>& p1;
  Pipe<K2>& p2;
  __device__ __forceinline__ bool first(const Job& j) const { return !kTwo || j.kind == 0; }
  __device__ __forceinline__ void issue(const Job& j, int s, int gs) const {
    if (first(j)) p1.issue_step(j, s, gs);
    else p2.issue_step(j, s, gs);
  }
  __device__ __forceinline__ int lookup(const Job& j) const {
    return first(j) ? p1.lookup(j) : p2.lookup(j);
  }
  // whether the tile's epilogue reads through its free-stage blocks, so that
  // step 1 of the next tile (which lands there) must wait for it
  __device__ __forceinline__ bool late(const Job& j) const {
    return first(j) ? K1::kLateStep1 : K2::kLateStep1;
  }
  __device__ __forceinline__ int epilogue(const Job& j, const Acc& acc, const Epi& ep) const {
    return first(j) ? k1.epilogue(j, acc, ep) : k2.epilogue(j, acc, ep);
  }
  template <bool G0, class Next>
  __device__ __forceinline__ void loop(Acc& acc, const Job& j, const Job& nxt, int g, int w1,
                                       Next&& next) {
    if (first(j)) {
      p1.g = g;
      p1.template group_loop<G0>(acc, j, nxt, w1, next);
    } else {
      p2.g = g;
      p2.template group_loop<G0>(acc, j, nxt, w1, next);
    }
  }
};

// This block's `total` tiles (tile_of(i)).  Steps 0 and 1 of the next tile
// are fetched while the current one finishes and stores, so neither a
// block's start nor the epilogue leaves the next tile's loads unissued.
// Group 0 (wm == 0) stores a tile while group 1 runs the MFMAs of its last
// phase.  Tiles without K steps (empty experts) run no barrier and store
// zeros.  Every barrier is reached by all waves: one after the landing of
// step 0 and 4 n - 1 in the K loop of each tile with n > 0 steps.  (Keeping
// group 1's accumulators until the next tile's first phase, to store them
// under group 0's MFMAs, measured 11% slower: the stores take several
// phases, so group 0 waits for them at the next barrier.)
template <class O, class TileOf>
__device__ __forceinline__ void engine(O& o, int total, TileOf&& tile_of, char* lds,
                                       uint32_t lbase, char* stg, int w) {
  const auto epi_at = [&](int g) {   // this wave's blocks of the free stage after step g - 1
    const int fs = ((g + 1) & 1) * kStage + 4 * w * 1024;
    return Epi{stg, lds + fs, lds + fs + kReg, lbase + fs, lbase + fs + kReg};
  };
  int g = 0;                 // K steps run so far (selects the stage)
  Job cur = tile_of(0);
  bool primed = false;       // steps 0 and (if it has one) 1 of cur are in flight
  int w0 = 0, w1 = 0;        // younger vm operations allowed at the waits for steps 0, 1
  for (int i = 0;; ++i) {
    Job nxt;
    nxt.steps = 0;
    nxt.kind = 0;
    if (i + 1 < total) nxt = tile_of(i + 1);
    const int n = cur.steps;
    Acc acc;
    zero(acc);
    bool started = false;
    if (n > 0) {
      if (!primed) {
        o.lookup(cur);
        o.issue(cur, 0, g);
        if (n > 1) o.issue(cur, 1, g + 1);
        w0 = n > 1 ? kDmaPerStep : 0;
        w1 = 0;
      }
      wait_vm_n(w0);                       // step 0 landed
      barrier();
      // the next tile's B-row lookups (x rows), younger than all in flight
      const int lk = nxt.steps > 0 ? o.lookup(nxt) : 0;
      const auto next = [&](int gs) { o.issue(nxt, 0, gs); };
      if (w < 4) o.template loop<true>(acc, cur, nxt, g, w1 + lk, next);
      else o.template loop<false>(acc, cur, nxt, g, w1 + lk, next);
      g += n;
      started = n >= 2 && nxt.steps > 0;
    }
    primed = started;
    // step 1 of the next tile goes into the stage the last K step used (all
    // its reads are done); before the stores unless the epilogue reads
    // through that stage, so that the stores drain while the next tile runs
    const bool step1 = primed && nxt.steps > 1;
    const bool lt = o.late(cur);
    if (!lt && step1) o.issue(nxt, 1, g + 1);
    const int nst = o.epilogue(cur, acc, epi_at(g));
    if (i + 1 >= total) break;
    if (lt && step1) {
      wait_lds();                          // this wave's free-stage reads are done
      o.issue(nxt, 1, g + 1);
    }
    // in flight, oldest first: step 0, [step 1,] the stores [, step 1]
    w0 = (step1 ? kDmaPerStep : 0) + nst;
    w1 = lt ? 0 : nst;
    cur = nxt;
  }
}

// One block per CU.  XCD x = blockIdx % 8 owns the logical tiles [lo, hi)
// that the product assigns it; its S blocks take them round-robin, so at any
// time they work on S consecutive tiles.  In the 4x2 layout (kFlip) a last
// round that would leave more than half of the blocks idle is dealt in
// 128-row halves instead: blocks r < t take the first row block of the t
// leftover tiles, blocks t..2t-1 the second one (none when the tile has a
// single block).  A one-block tile keeps every SIMD busy with one wave and
// fetches half the row operand, so it ends well before a whole tile would.
// Every branch that reaches a barrier is uniform over the block.
template <class K>
__device__ __forceinline__ void persistent(const K& k) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  static_assert(K::kLateStep1 || !K::kUsesFreeStage, "the free stage is refilled before the epilogue");
  const int S = (int)(gridDim.x / 8);
  const int x = (int)(blockIdx.x % 8), r = (int)(blockIdx.x / 8);
  int lo, hi;
  k.xcd_range(x, lo, hi);
  lo = (int)uniform((uint32_t)lo);
  hi = (int)uniform((uint32_t)hi);
  int full = hi - lo, tail = 0;      // tiles dealt whole; leftover tiles dealt in halves
  if constexpr (K::kFlip) {
    const int t = full % S;
    if (t > 0 && 2 * t <= S) {
      full -= t;
      tail = t;
    }
  }
  const int nfull = full > r ? (full - r + S - 1) / S : 0;
  int half_tile = -1, half = 0;      // this block's half of a leftover tile
  if (r < 2 * tail) {
    half = r < tail ? 0 : 1;
    half_tile = lo + full + r - half * tail;
    if (half == 1) {
      Job t;
      k.tile(half_tile, t);
      if (!t.fb) half_tile = -1;
    }
  }
  const int total = nfull + (half_tile >= 0 ? 1 : 0);
  if (total <= 0) return;
  const uint32_t lbase = uniform(lds_addr(lds));
  Pipe<K> p{k, lds, lbase, 0};
  p.lane = threadIdx.x & 63;
  p.w = (int)uniform(threadIdx.x >> 6);
  p.wm = p.w >> 2;
  p.wn = p.w & 3;
  p.da.init(k.lda(), p.lane);
  p.db.init(k.ldb(), p.lane);
  char* const stg = lds + 2 * kStage + p.w * kStgWave;
  Ops<K, K, false> o{k, k, p, p};
  const auto tile_of = [&](int i) {
    Job j;
    if (i < nfull) {
      k.tile(lo + r + i * S, j);
    } else {
      k.tile(half_tile, j);
      j.u += half;
      j.fb = false;
    }
    j.kind = 0;
    return j;
  };
  engine(o, total, tile_of, lds, lbase, stg, p.w);
}


// Two independent products in one persistent launch, so that the short
// weight-gradient tiles of K2 fill the last round of K1's row tiles instead
// of leaving CUs idle between two launches.  K1 has row tiles of equal cost
// (tile_steps() K steps plus an epilogue); K2 has whole experts per XCD
// (tiles_per_expert() tiles of expert_steps(e) K steps).  Within XCD x the
// S blocks first take K1's tiles round-robin; with n1 = a S + m, blocks
// 0..m-1 get one tile more, so the other S - m are free one K1 tile earlier
// and take the first K2 tiles round-robin among themselves (phase A), as
// many as keep each of them within one K1 tile of extra work.  Then all S blocks take the remaining K2
// tiles round-robin (phase B), so concurrent blocks still work on
// consecutive tiles; phase B deals in order of the blocks' load so far
// (light blocks with one phase-A tile fewer, then the m heavy blocks, then
// the other light blocks), so that its last partial round goes to the
// least loaded.  Every wave computes the same schedule from the live
// metadata; blocks do not communicate.
//
// kTailFill runs K1 and phase A only, and a later launch with kRest (same
// grid) runs phase B: other work can then sit between the two, here the
// gather's backward, which reads K1's output while it is still in the
// last-level cache.
enum DualMode { kAll, kTailFill, kRest };

template <class K1, class K2, DualMode M = kAll>
struct DualSched {
  int lo1, lo2, r, S, m, nA;
  int rho;          // this block's place in the phase-B order
  int c1, cA, cB;   // this block's tiles of K1, of phase A, of phase B

  // The longest prefix of K2's tiles [lo, hi) that, dealt round-robin over
  // `nb` blocks, gives no block more than `gap` K steps: ceil(n / nb) tiles
  // of at most the largest cost among them.  lo and hi may fall inside an
  // expert's tiles.
  __device__ static int prefix_tiles(const K2& k2, int lo, int hi, int nb, int gap) {
    const int tpe = k2.tiles_per_expert();
    int n = 0, cmax = 1;
    for (int e = lo / tpe; e * tpe < hi; ++e) {
      const int avail = min(hi, (e + 1) * tpe) - max(lo, e * tpe);   // e's tiles in [lo, hi)
      cmax = max(cmax, k2.expert_steps(e) + K2::kEpiSteps);
      const int cap = (gap / cmax) * nb;   // tiles allowed at this cost
      if (cap <= n) break;
      if (cap < n + avail) return cap;
      n += avail;
    }
    return n;
  }

  // filled: whether a kTailFill launch ran phase A (kRest only)
  __device__ void init(const K1& k1, const K2& k2, int x, int r_, int S_, bool filled = true) {
    r = r_;
    S = S_;
    int hi1, hi2;
    k1.xcd_range(x, lo1, hi1);
    k2.xcd_range(x, lo2, hi2);
    lo1 = (int)uniform((uint32_t)lo1);
    lo2 = (int)uniform((uint32_t)lo2);
    const int n1 = (int)uniform((uint32_t)(hi1 - lo1));
    const int n2 = (int)uniform((uint32_t)(hi2 - lo2));
    m = n1 % S;
    c1 = n1 / S + (r < m ? 1 : 0);
    nA = 0;
    if (m > 0 && filled)
      nA = (int)uniform((uint32_t)prefix_tiles(k2, lo2, lo2 + n2, S - m,
                                               k1.tile_steps() + K1::kEpiSteps));
    cA = (r >= m && nA > r - m) ? (nA - (r - m) + (S - m) - 1) / (S - m) : 0;
    const int rem = nA % (S - m);   // light blocks r - m < rem have one more phase-A tile
    if (r >= m) rho = r - m >= rem ? r - m - rem : S - rem + (r - m);
    else rho = S - m - rem + r;
    const int nB = n2 - nA;
    cB = nB > rho ? (nB - rho + S - 1) / S : 0;
    if (M == kTailFill) cB = 0;
    if (M == kRest) {               // a fresh launch: plain round-robin
      c1 = cA = 0;
      rho = r;
      cB = nB > r ? (nB - r + S - 1) / S : 0;
    }
  }
  __device__ int count() const { return c1 + cA + cB; }
  // this block's i-th tile (each branch fills its own Job, so that all of
  // them stay in registers)
  __device__ Job job(const K1& k1, const K2& k2, int i) const {
    if (M != kRest && i < c1) {
      Job a;
      k1.tile(lo1 + r + i * S, a);
      a.kind = 0;
      return a;
    }
    i -= c1;
    Job b;
    k2.tile(i < cA ? lo2 + (r - m) + i * (S - m) : lo2 + nA + rho + (i - cA) * S, b);
    b.kind = 1;
    return b;
  }
};

template <DualMode M = kAll, class K1, class K2>
__device__ __forceinline__ void persistent_dual(const K1& k1, const K2& k2, bool filled = true) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  static_assert(K1::kLateStep1 || !K1::kUsesFreeStage, "the free stage is refilled before the epilogue");
  static_assert(K2::kLateStep1 || !K2::kUsesFreeStage, "the free stage is refilled before the epilogue");
  const int S = (int)(gridDim.x / 8);
  const int x = (int)(blockIdx.x % 8), r = (int)(blockIdx.x / 8);
  DualSched<K1, K2, M> sc;
  sc.init(k1, k2, x, r, S, filled);
  const int total = sc.count();
  if (total <= 0) return;
  const uint32_t lbase = uniform(lds_addr(lds));
  const int lane = threadIdx.x & 63, w = (int)uniform(threadIdx.x >> 6);
  Pipe<K1> p1{k1, lds, lbase, 0};
  Pipe<K2> p2{k2, lds, lbase, 0};
  p1.lane = p2.lane = lane;
  p1.w = p2.w = w;
  p1.wm = p2.wm = w >> 2;
  p1.wn = p2.wn = w & 3;
  p1.da.init(k1.lda(), lane);
  p1.db.init(k1.ldb(), lane);
  p2.da.init(k2.lda(), lane);
  p2.db.init(k2.ldb(), lane);
  char* const stg = lds + 2 * kStage + w * kStgWave;
  const auto tile_of = [&](int i) { return sc.job(k1, k2, i); };
  if constexpr (M == kRest) {   // K2 tiles only
    Ops<K2, K2, false> o{k2, k2, p2, p2};
    engine(o, total, tile_of, lds, lbase, stg, w);
  } else {
    Ops<K1, K2, true> o{k1, k2, p1, p2};
    engine(o, total, tile_of, lds, lbase, stg, w);
  }
}

// X: x_perm is x itself ([T, H]) and B rows come through row_token.
template <bool X>
__global__ void __launch_bounds__(kThreads)
up_kernel(const bf16* __restrict__ x_perm, const bf16* __restrict__ w1,
          const bf16* __restrict__ w3, int64_t H, int64_t F, ROW_TILE_ARGS,
          const int32_t* __restrict__ row_token, uint32_t x_bytes,
          bf16* __restrict__ h1, bf16* __restrict__ h3, bf16* __restrict__ act) {
  UpT<X> k{x_perm, w1, w3, H, F, h1, h3, act};
  k.rt.init(tile_expert, pair_first, num_pairs, padded_bins, (int)(F / 128));
  k.xr = XRows{x_perm, row_token, x_bytes};
  persistent(k);
}

__global__ void __launch_bounds__(kThreads)
down_kernel(const bf16* __restrict__ act, const bf16* __restrict__ w2, int64_t H,
            int64_t F, ROW_TILE_ARGS, bf16* __restrict__ y_perm) {
  Down k{act, w2, H, F, y_perm};
  k.rt.init(tile_expert, pair_first, num_pairs, padded_bins, (int)((H + 255) / 256));
  persistent(k);
}

__global__ void __launch_bounds__(kThreads)
up_dgrad_kernel(const bf16* __restrict__ dh1, const bf16* __restrict__ dh3,
                const bf16* __restrict__ w1, const bf16* __restrict__ w3, int64_t H,
                int64_t F, ROW_TILE_ARGS, bf16* dx_perm) {
  UpDgrad k{dh1, dh3, w1, w3, H, F, dx_perm};
  k.rt.init(tile_expert, pair_first, num_pairs, padded_bins, (int)((H + 255) / 256));
  persistent(k);
}

// dx_perm = dh1 w1^T + dh3 w3^T, with the first dw1/dw3 tiles filling its
// last round (kTailFill); wgrad_up_kernel (kRest, same grid, filled = 1)
// does the rest.
__global__ void __launch_bounds__(kThreads)
up_dgrad_fill_kernel(const bf16* __restrict__ dh1, const bf16* __restrict__ dh3,
                     const bf16* __restrict__ w1, const bf16* __restrict__ w3,
                     const bf16* __restrict__ x_perm, int64_t H, int64_t F, int E,
                     ROW_TILE_ARGS, const int32_t* __restrict__ tpe, bf16* dx_perm,
                     bf16* __restrict__ dw1, bf16* __restrict__ dw3) {
  UpDgrad k1{dh1, dh3, w1, w3, H, F, dx_perm};
  k1.rt.init(tile_expert, pair_first, num_pairs, padded_bins, (int)((H + 255) / 256));
  persistent_dual<kTailFill>(
      k1, WgradUp{x_perm, dh1, dh3, H, F, E, tpe, padded_bins, dw1, dw3});
}

// down dgrad + gate backward (dh1, dh3) and dw2 in one launch: both read
// dy_perm, neither reads what the other writes.
__global__ void __launch_bounds__(kThreads)
down_dgrad_wgrad_down_kernel(const bf16* __restrict__ dy_perm, const bf16* __restrict__ w2,
                             const bf16* h1, const bf16* h3, const bf16* __restrict__ act,
                             int64_t H, int64_t F, int E, ROW_TILE_ARGS,
                             const int32_t* __restrict__ tpe, bf16* dh1, bf16* dh3,
                             bf16* __restrict__ dw2) {
  DownDgrad k1{dy_perm, w2, h1, h3, H, F, dh1, dh3};
  k1.rt.init(tile_expert, pair_first, num_pairs, padded_bins, (int)((F + 255) / 256));
  persistent_dual(k1, WgradDown{act, dy_perm, H, F, E, tpe, padded_bins, dw2});
}

__global__ void __launch_bounds__(kThreads)
wgrad_up_kernel(const bf16* __restrict__ dh1, const bf16* __restrict__ dh3,
                const bf16* __restrict__ w1, const bf16* __restrict__ w3,
                const bf16* __restrict__ x_perm, int64_t H, int64_t F, int E, ROW_TILE_ARGS,
                const int32_t* __restrict__ tpe, int filled, bf16* dx_perm, bf16* __restrict__ dw1, bf16* __restrict__ dw3) {
  UpDgrad k1{dh1, dh3, w1, w3, H, F, dx_perm};
  k1.rt.init(tile_expert, pair_first, num_pairs, padded_bins, (int)((H + 255) / 256));
  persistent_dual<kRest>(k1, WgradUp{x_perm, dh1, dh3, H, F, E, tpe, padded_bins, dw1, dw3},
                         filled != 0);
}

// The dgrad and the weight gradient of a single grouped linear map y = x w[e]
// (w [E, H, F]) in one launch, as the down dgrad and dw2 share one:
// dx_perm [P, H] = dy_perm [P, F] w[e]^T and dw [E, H, F] = x_perm [P, H]^T
// dy_perm [P, F] per expert (zero for an empty expert).  Both read dy_perm and
// neither reads what the other writes, so the weight-gradient tiles fill the
// dgrad's last round of row tiles.
__global__ void __launch_bounds__(kThreads)
dgrad_wgrad_kernel(const bf16* __restrict__ dy_perm, const bf16* __restrict__ w,
                   const bf16* __restrict__ x_perm, int64_t H, int64_t F, int E, ROW_TILE_ARGS,
                   const int32_t* __restrict__ tpe, bf16* __restrict__ dx_perm,
                   bf16* __restrict__ dw) {
  UpDgrad k1{dy_perm, dy_perm, w, w, H, F, dx_perm};
  k1.two = false;
  k1.rt.init(tile_expert, pair_first, num_pairs, padded_bins, (int)((H + 255) / 256));
  // WgradDown's (H, F) name its output dw [E, F, H]: here (F, H)
  persistent_dual(k1, WgradDown{x_perm, dy_perm, F, H, E, tpe, padded_bins, dw});
}

}  // namespace bfk

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (cached per device).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// One block per CU (a multiple of 8: one share per XCD), fewer when there are
// fewer tiles.
static dim3 persistent_grid(int64_t max_total) {
  const int64_t slots = std::max<int64_t>(1, device_cus() / 8);
  const int64_t per = std::max<int64_t>(1, cdiv(max_total, 8));
  return dim3((unsigned)(8 * std::min(per, slots)));
}

template <typename T> static const T* cb(const void* p) { return static_cast<const T*>(p); }
template <typename T> static T* mb(void* p) { return static_cast<T*>(p); }

// Bytes of x [T, H] bf16, the records of its buffer resource (the callers
// check that it stays below 2 GB).
static uint32_t x_bytes(const Shape& s) { return (uint32_t)(s.T * s.H * 2); }

hipError_t launch_bf16_up(const Shape& s, const void* x_perm, const void* x, const void* w1,
                          const void* w3, const MetaPtrs& m, void* h1, void* h3, void* act,
                          hipStream_t stream) {
  const dim3 grid = persistent_grid(cdiv(s.F, 128) * s.max_tiles);
  if (x)
    hipLaunchKernelGGL(bfk::up_kernel<true>, grid, dim3(bfk::kThreads), 0, stream, cb<bf16>(x),
                       cb<bf16>(w1), cb<bf16>(w3), s.H, s.F, m.tile_expert, m.pair_first,
                       m.num_pairs, m.padded_bins, m.row_token, x_bytes(s), mb<bf16>(h1),
                       mb<bf16>(h3), mb<bf16>(act));
  else
    hipLaunchKernelGGL(bfk::up_kernel<false>, grid, dim3(bfk::kThreads), 0, stream,
                       cb<bf16>(x_perm), cb<bf16>(w1), cb<bf16>(w3), s.H, s.F, m.tile_expert,
                       m.pair_first, m.num_pairs, m.padded_bins, m.row_token, 0u,
                       mb<bf16>(h1), mb<bf16>(h3), mb<bf16>(act));
  return hipGetLastError();
}

hipError_t launch_bf16_down(const Shape& s, const void* act, const void* w2,
                            const MetaPtrs& m, void* y_perm, hipStream_t stream) {
  hipLaunchKernelGGL(bfk::down_kernel, persistent_grid(cdiv(s.H, 256) * s.max_tiles),
                     dim3(bfk::kThreads), 0, stream, cb<bf16>(act), cb<bf16>(w2), s.H, s.F,
                     m.tile_expert, m.pair_first, m.num_pairs, m.padded_bins,
                     mb<bf16>(y_perm));
  return hipGetLastError();
}

// The up-projection dgrad and dw1/dw3 are two launches on one grid, with the
// gather's backward between them.  When the dgrad's last round of row tiles
// is expected to be less than 90% full, the first launch also takes the
// dw1/dw3 tiles that fill it (see DualSched).  The estimate assumes balanced
// routing: each expert has T k / E rows, so about T k / (256 E) + 1/2 pairs
// of row blocks.  It depends on the shape only, so both launches agree.
static dim3 up_dgrad_grid(const Shape& s) {
  return persistent_grid(cdiv(s.H, 256) * s.max_tiles + cdiv(s.F, 128) * cdiv(s.H, 256) * s.E);
}

static bool up_dgrad_fills_tail(const Shape& s) {
  const double rows = (double)s.T * s.k / s.E;
  const double tiles = s.E * (rows / 256.0 + 0.5) * (double)cdiv(s.H, 256);
  const double rounds = tiles / (double)up_dgrad_grid(s).x;
  return rounds / std::ceil(rounds) < 0.9;
}

hipError_t launch_bf16_up_dgrad(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const void* x_perm,
                                const MetaPtrs& m, void* dx_perm, void* dw1, void* dw3,
                                hipStream_t stream) {
  if (up_dgrad_fills_tail(s)) {
    hipLaunchKernelGGL(bfk::up_dgrad_fill_kernel, up_dgrad_grid(s), dim3(bfk::kThreads), 0,
                       stream, cb<bf16>(dh1), cb<bf16>(dh3), cb<bf16>(w1), cb<bf16>(w3),
                       cb<bf16>(x_perm), s.H, s.F, s.E, m.tile_expert, m.pair_first,
                       m.num_pairs, m.padded_bins, m.tokens_per_expert, mb<bf16>(dx_perm),
                       mb<bf16>(dw1), mb<bf16>(dw3));
  } else {
    hipLaunchKernelGGL(bfk::up_dgrad_kernel, persistent_grid(cdiv(s.H, 256) * s.max_tiles),
                       dim3(bfk::kThreads), 0, stream, cb<bf16>(dh1), cb<bf16>(dh3),
                       cb<bf16>(w1), cb<bf16>(w3), s.H, s.F, m.tile_expert,
                       m.pair_first, m.num_pairs, m.padded_bins, mb<bf16>(dx_perm));
  }
  return hipGetLastError();
}

hipError_t launch_bf16_down_dgrad_wgrad_down(const Shape& s, const void* dy_perm,
                                             const void* w2, const void* h1, const void* h3,
                                             const void* act, const MetaPtrs& m, void* dh1,
                                             void* dh3, void* dw2, hipStream_t stream) {
  const int64_t t1 = cdiv(s.F, 256) * s.max_tiles;
  const int64_t t2 = cdiv(s.H, 256) * cdiv(s.F, 256) * s.E;
  hipLaunchKernelGGL(bfk::down_dgrad_wgrad_down_kernel, persistent_grid(t1 + t2),
                     dim3(bfk::kThreads), 0, stream, cb<bf16>(dy_perm), cb<bf16>(w2),
                     cb<bf16>(h1), cb<bf16>(h3), cb<bf16>(act), s.H, s.F, s.E,
                     m.tile_expert, m.pair_first, m.num_pairs, m.padded_bins,
                     m.tokens_per_expert, mb<bf16>(dh1), mb<bf16>(dh3), mb<bf16>(dw2));
  return hipGetLastError();
}

hipError_t launch_bf16_wgrad_up(const Shape& s, const void* dh1, const void* dh3,
                                const void* w1, const void* w3, const void* x_perm,
                                const MetaPtrs& m, void* dx_perm, void* dw1, void* dw3,
                                hipStream_t stream) {
  hipLaunchKernelGGL(bfk::wgrad_up_kernel, up_dgrad_grid(s), dim3(bfk::kThreads), 0, stream,
                     cb<bf16>(dh1), cb<bf16>(dh3), cb<bf16>(w1), cb<bf16>(w3),
                     cb<bf16>(x_perm), s.H, s.F, s.E, m.tile_expert, m.pair_first,
                     m.num_pairs, m.padded_bins, m.tokens_per_expert,
                     up_dgrad_fills_tail(s) ? 1 : 0, mb<bf16>(dx_perm), mb<bf16>(dw1),
                     mb<bf16>(dw3));
  return hipGetLastError();
}

// dx_perm [P, H] = dy_perm [P, F] w[e]^T and dw [E, H, F] = x_perm [P, H]^T
// dy_perm [P, F] per expert, with w [E, H, F], in one launch.
hipError_t launch_bf16_dgrad_wgrad(const Shape& s, const void* dy_perm, const void* w,
                                   const void* x_perm, const MetaPtrs& m, void* dx_perm,
                                   void* dw, hipStream_t stream) {
  const int64_t t1 = cdiv(s.H, 256) * s.max_tiles;
  const int64_t t2 = cdiv(s.H, 256) * cdiv(s.F, 256) * s.E;
  hipLaunchKernelGGL(bfk::dgrad_wgrad_kernel, persistent_grid(t1 + t2), dim3(bfk::kThreads), 0,
                     stream, cb<bf16>(dy_perm), cb<bf16>(w), cb<bf16>(x_perm), s.H, s.F, s.E,
                     m.tile_expert, m.pair_first, m.num_pairs, m.padded_bins,
                     m.tokens_per_expert, mb<bf16>(dx_perm), mb<bf16>(dw));
  return hipGetLastError();
}

}  // namespace dmoe
