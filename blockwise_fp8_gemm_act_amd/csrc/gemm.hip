// Blockwise-scaled FP8 GEMM for gfx950 (CDNA4 matrix cores).
//
//   out[m][n] = sum over 128-deep K slices kb of  sA(m,kb) * sB(n,kb) * P_kb[m][n],
//   P_kb[m][n] = sum_{k in slice kb} dec(a[m][k]) * dec(b[n][k])   (fp32, matrix cores)
//
// The pages put the matrix multiplications of the main linear layers on this
// FP8 path with fine-grained block scaling after DeepSeek-V3 (en.roboind.com
// article on Puro-2B, section "FP8 takes advantage of the RTX 5090's low
// precision efficiency").  Both operands are stored K-contiguous ("TN"), so
// fprop (X W^T), dgrad (dY W, with W's codes pre-transposed) and wgrad
// (dY^T X, with 128x1-quantized transposes) are all this one contraction; they
// differ only in B's scale layout:
//   block-scaled B (fprop, dgrad): sB(n,kb) = sb[n/128][kb]
//   row-scaled B   (wgrad):        sB(n,kb) = sb[kb][n]
//
// Design (MFMA-bound; ~1300-2750 flop per byte of operands at the layer
// shapes):
//  - one workgroup of 8 waves computes a 256x256 output tile; each wave owns
//    64 (M) x 128 (N): 4 x 8 blocks of 16x16, 128 fp32 accumulators per lane;
//  - each 128-deep K slice of A and B (2 x 32 KB of e4m3) is copied global ->
//    LDS by the DMA path (global_load_lds_dwordx4, no VGPR round trip) into
//    one of two buffers while the other is consumed: 128 KB of the 160 KB LDS.
//    When every tile of a launch is interior (kSpread), a slice's copies go
//    out one A/B row-group pair per n-block step over the first four steps
//    instead of in one burst, which stalls the issuing waves less;
//  - one v_mfma_f32_16x16x128_f8f6f4 covers exactly one 16x16 block of one
//    slice, so its result is the slice partial P_kb; it is promoted at once:
//    acc = fma(P, sA*sB, acc);
//  - the barrier that publishes slice kb+1 sits before the last of slice kb's
//    eight n-block steps, so the next slice's fragment and scale reads overlap
//    MFMAs instead of stalling all waves at once at the slice boundary;
//  - LDS rows are 128 B; the 16-byte chunk c of row r sits at chunk
//    c ^ swz(r), swz(r) = r1 | (r2 ^ r4) << 2 (ri: bit i of r), which keeps
//    both fragment read patterns (16 lanes reading one chunk column of 16
//    consecutive A rows, or of the 16 B rows 8a + b, a, b < 4) free of bank
//    conflicts.  gfx950 serves a 16-byte LDS read 16 consecutive lanes at a
//    time over 64 four-byte banks, and the bank of dword d is
//    (d mod 64) XOR (bit 8 of d) << 3 (measured: bank-conflict counters of
//    read patterns, fitted exactly).  That hardware term already moves row
//    bit 3 into chunk bit 1, so the swizzle leaves that bit alone;
//  - the output leaves straight from the accumulators as 16-byte stores; lane
//    pairs trade halves through a DPP swap so that every store instruction
//    writes whole 128-byte row segments (8 cache lines, not 16 half lines);
//  - the row-scaled kernel also comes with 192- and 128-column tiles, which
//    the planner picks per shape when they fill the chip in fewer rounds;
//  - rows past M or N are read from clamped (valid) rows and never stored;
//    K chunks past K read a 16-byte zero page, so a ragged last slice adds 0;
//  - an item's slices are promoted in a fixed order that depends on its row
//    tile alone (a rotation by (tm % 8) / 8 of its K range, which keeps the
//    items that share an XCD's L2 in lockstep and staggers the 8 XCDs), so
//    every output element sees the same order whatever the column tiling;
//    optional split-K writes fp32 partials to a workspace that a second
//    kernel sums in a fixed order.  Results are deterministic;
//  - accumulate mode (fp32 out): out = fp32(out + GEMM), one addition of the
//    finished GEMM value per element, in the store epilogue or, with split-K,
//    in the reduction.  It lets micro-batches add their weight gradients into
//    one fp32 buffer (the pages tune micro-batch sizes per pipeline stage:
//    en.roboind.com article, section "Unit cost, higher computing power");
//  - SwiGLU mode (fprop of a fused gate/up weight, bf16 out): a tile covers
//    128 h columns, i.e. 128 gate and 128 up rows of B interleaved in groups
//    of 4, and the epilogue writes the 1x128 codes and scales of
//    h = bf16(silu(g) * u) -- the down projection's FP8 input -- with the
//    bf16 gate/up output optional.  The epilogue runs after the item's last
//    slice and does not overlap MFMA work, which makes it cost more than the
//    separate SwiGLU quantizer pass unless the gate/up output is dropped;
//  - token-major wgrad (kKT): A and B arrive as [K][M] / [K][N] codes (the
//    128x1 codes left untransposed by their quantizer); slices are copied as
//    token rows and the MFMA fragments are assembled by transposing LDS
//    reads (ds_read_b64_tr_b8), four per fragment.  Products and their order
//    are those of the wgrad on the transposed operands.
#include "device_common.h"
#include "launch.h"

#include <atomic>
#include <type_traits>

namespace puro {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kThreads = 512;
constexpr int kSliceBytes = kBM * kBK;            // 32 KB per operand per slice

__device__ __align__(16) uint8_t g_zero16[16];     // zero-initialized at load

struct GemmArgs {
  const uint8_t *a;
  const float *sa;
  const uint8_t *b;
  const float *sb;
  void *out;
  float *ws;
  int64_t M, N, K;
  int nk;          // ceil(K / 128)
  int tiles_m, tiles_n;
  int splits;      // K-loop splits (1: no workspace)
  int spl;         // slices per split
  int tile0;       // this launch covers output tiles tile0 .. tile0 + ntiles - 1
  int ntiles;      //   (tile t: row tile t % tiles_m, column tile t / tiles_m)
  int bn;          // output tile width: 256, or 192 / 128 for the row-scaled kernel
  int blocked;     // items in XCD blocks of 4 x 8 tiles (tile_of); set by the host
  int banded;      // tiles numbered in row bands (band_tile); set by the host
  // fused SwiGLU epilogue only: B holds gate rows [0, I) and up rows [I, 2I);
  // out is the optional bf16 gate/up output [M][2I]
  int64_t I;
  uint8_t *hq;     // codes of h [M][I]
  float *hs;       // their 1x128 scales [I/128][M]
};


// Global -> LDS DMA (gfx950 global_load_lds).  The LDS destination of lane i
// is M0 + 16*i (dwordx4) or M0 + 4*i (dword); M0 is set and restored inside
// the statement.  These write only LDS (no VGPR results); completion is
// awaited explicitly with s_waitcnt vmcnt(0) before the barrier that
// publishes a slice.  They are written as asm so that the compiler does not
// make every later LDS read wait for them.
__device__ __forceinline__ void dma16_s(const void *sbase, uint32_t voff, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}
__device__ __forceinline__ void dma16_v(const void *vaddr, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(vaddr), "s"(lds)
      : "memory");
}
__device__ __forceinline__ void dma4_s(const void *sbase, uint32_t voff, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// The 8 copies of one interior slice for this wave: row groups 4w+j (j = 0..3)
// of A and of B.  Lane offsets vj already include row group j; the 64-bit
// bases point at the wave's first row group in the slice; A lands at `lds`
// + 1024 j and B at `lds` + 32 KB + 1024 j.  M0 is saved once and stepped
// with scalar adds.
__device__ __forceinline__ void dma_slice8(const void *abase, const void *bbase, uint32_t v0, uint32_t v1,
                                           uint32_t v2, uint32_t v3, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %6\n\t"
      "s_sub_u32 m0, m0, 0x7c00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %5\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %6\n\t"
      "s_sub_u32 m0, m0, 0x7c00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %5\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %6\n\t"
      "s_sub_u32 m0, m0, 0x7c00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %5\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %6\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(abase), "s"(bbase), "s"(lds)
      : "memory", "scc");
}

// One row group of A and the same row group of B: two of dma_slice8's eight
// copies (M0 = lds for A, lds + 32 KB for B).
__device__ __forceinline__ void dma_pair(const void *abase, const void *bbase, uint32_t v, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(v), "s"(abase), "s"(bbase), "s"(lds)
      : "memory", "scc");
}

// One copy into A's half and one into B's (lds + 32 KB), with their own lane
// offsets: a row-group pair of a token-major slice.
__device__ __forceinline__ void dma_pair_ab(const void *abase, const void *bbase, uint32_t va, uint32_t vb,
                                            uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %3\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %4\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(va), "v"(vb), "s"(abase), "s"(bbase), "s"(lds)
      : "memory", "scc");
}

// The same 8 copies with separate lane offsets for B (its rows do not follow
// A's row pattern in the fused SwiGLU kernel).
__device__ __forceinline__ void dma_slice8ab(const void *abase, const void *bbase, uint32_t a0, uint32_t a1,
                                             uint32_t a2, uint32_t a3, uint32_t b0, uint32_t b1, uint32_t b2,
                                             uint32_t b3, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %11\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %9\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %5, %10\n\t"
      "s_sub_u32 m0, m0, 0x7c00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %9\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %6, %10\n\t"
      "s_sub_u32 m0, m0, 0x7c00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %9\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %7, %10\n\t"
      "s_sub_u32 m0, m0, 0x7c00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %9\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %8, %10\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b0), "v"(b1), "v"(b2), "v"(b3), "s"(abase), "s"(bbase), "s"(lds)
      : "memory", "scc");
}

// Copies of one interior slice for a tile narrower than 256 columns: the
// wave's 4 row groups of A (lane offsets v0..v3, LDS at lda + 1024 j) and its
// NGB row groups of B (lane offsets vb[j], LDS at ldb + 1024 j).
template <int NGB>
__device__ __forceinline__ void dma_slice_narrow(const void *abase, const void *bbase, uint32_t v0, uint32_t v1,
                                                 uint32_t v2, uint32_t v3, const uint32_t (&vb)[NGB], uint32_t lda,
                                                 uint32_t ldb) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %5\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %5\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %5\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(abase), "s"(lda)
      : "memory", "scc");
  if constexpr (NGB == 3) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %4\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %4\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %4\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(vb[0]), "v"(vb[1]), "v"(vb[2]), "s"(bbase), "s"(ldb)
        : "memory", "scc");
  } else {
    static_assert(NGB == 2, "3 or 2 row groups of B per wave");
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(vb[0]), "v"(vb[1]), "s"(bbase), "s"(ldb)
        : "memory", "scc");
  }
}

// The 8 copies of one token-major slice for this wave: copy j brings tile rows
// 16w + 4j .. 16w + 4j + 3 of A (at `lds` + 1024 j) and of B (32 KB further),
// 256 bytes each.  The row step is folded into the eight 64-bit bases; the
// lane offsets repeat with the parity of j.
__device__ __forceinline__ void dma_slice8kt(const void *a0, const void *a1, const void *a2, const void *a3,
                                             const void *b0, const void *b1, const void *b2, const void *b3,
                                             uint32_t va0, uint32_t va1, uint32_t vb0, uint32_t vb1, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %13\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %9, %1\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %11, %5\n\t"
      "s_sub_u32 m0, m0, 0x7c00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %10, %2\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %12, %6\n\t"
      "s_sub_u32 m0, m0, 0x7c00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %9, %3\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %11, %7\n\t"
      "s_sub_u32 m0, m0, 0x7c00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %10, %4\n\t"
      "s_add_u32 m0, m0, 0x8000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %12, %8\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(a0), "s"(a1), "s"(a2), "s"(a3), "s"(b0), "s"(b1), "s"(b2), "s"(b3), "v"(va0), "v"(va1), "v"(vb0),
        "v"(vb1), "s"(lds)
      : "memory", "scc");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Row-band numbering of the tiles of a GEMM with 8 column tiles whose A
// operand is larger than the MALL holds: tiles 256b .. 256b+255 are band b,
// row tiles 32b .. 32b+31 (fewer in a last, partial band) across all 8 column
// tiles, walked down M.  A whole round of 256 items is then one band: each
// XCD's 32 items are 4 row tiles x 8 column tiles (12 panels, as in the row-tile
// walk) and each A panel is read in one round only, where the walk reads it
// once per 4 column tiles.  A plan that computes its first 256 tiles whole and
// splits the rest splits a band of whole row tiles.
__host__ __device__ __forceinline__ void band_tile(int tile, int tiles_m, int &tm, int &tn) {
  const int b = tile >> 8, j = tile & 255;
  const int h = min(32, tiles_m - 32 * b);
  tm = 32 * b + j % h;
  tn = j / h;
}

// One work item: a 256x256 output tile and one split of its K slices.  All
// fields are uniform across the workgroup.
struct Tile {
  int m0, n0;                // first row of A / of B (M, N < 2^31)
  int kb_begin, kb_end;
  int rot;                   // the item's slices run kb_begin + rot, ..., kb_end - 1, kb_begin, ...
  int rows_a, rows_b;        // valid rows of A / B in the tile
  int split;
  int local;                 // tile index within this launch (tile - tile0): its block of the workspace
};

// glu: the tile covers h columns n0 .. n0+127 (B rows: 128 gate + 128 up rows).
__device__ __forceinline__ Tile tile_of(const GemmArgs &g, int item, bool glu = false) {
  Tile t;
  int tm, tn, xk;
  if (g.blocked) {
    // Blocked order (weight gradients whose whole tile grid, times the splits,
    // fills rounds of 256 items; tiles_m % 4 == 0, tiles_n % 8 == 0).  Item
    // 256r + 8w + x belongs to block 8r + x and is tile (w % 4, w / 4) of it:
    // the 32 items that workgroups b = x (mod 8) run together on one XCD are
    // one split of a 4 x 8 group of tiles, sharing 4 A and 8 B panels (12
    // panels for 32 items, against 33 or more in the row-tile walk below when
    // the row tiles are few).  Blocks run split-major, then along M, then N.
    const int x = item & 7, w = (item >> 3) & 31, blk = ((item >> 8) << 3) | x;
    const int bpm = g.tiles_m >> 2, bps = bpm * (g.tiles_n >> 3);
    t.split = blk / bps;
    const int bb = blk - t.split * bps;
    tm = (bb % bpm) * 4 + (w & 3);
    tn = (bb / bpm) * 8 + (w >> 2);
    t.local = tn * g.tiles_m + tm;       // the launch covers every tile (tile0 = 0)
    xk = x;
  } else {
    t.split = item / g.ntiles;
    t.local = item - t.split * g.ntiles;
    const int tile = g.tile0 + t.local;
    if (g.banded) {
      band_tile(tile, g.tiles_m, tm, tn);
    } else {
      tm = tile % g.tiles_m;             // consecutive items walk down M: they share B
      tn = tile / g.tiles_m;
    }
    xk = tm & 7;
  }
  t.m0 = tm * kBM;
  t.n0 = tn * (glu ? kBK : g.bn);
  t.kb_begin = t.split * g.spl;
  t.kb_end = min(g.nk, t.kb_begin + g.spl);
  // Items that run on one XCD at the same time (item = b + rG, workgroup b on
  // XCD b % 8, G a multiple of 8) share item % 8, which is tm % 8 when the
  // row-tile count is a multiple of 8 (and the block's x in the blocked
  // order): they walk K in lockstep, sharing their A and B panels through
  // that XCD's L2, and the 8 XCDs start 1/8 of the K range apart.  In the
  // row-tile walk the order depends on the row tile alone, so an output
  // element is summed in the same order by the plain fprop and by the fused
  // SwiGLU kernel (whose column tiles differ).
  t.rot = (int)(((unsigned)xk * (unsigned)(t.kb_end - t.kb_begin)) / 8u);
  t.rows_a = min((int)g.M - t.m0, kBM);
  t.rows_b = glu ? kBN : min((int)g.N - t.n0, g.bn);
  return t;
}

// K slice of step i (0 .. kb_end - kb_begin - 1) of an item.
__device__ __forceinline__ int kb_at(const Tile &t, int i) {
  int k = t.rot + i;
  const int n = t.kb_end - t.kb_begin;
  if (k >= n) k -= n;
  return t.kb_begin + k;
}

// Persistent kernel: workgroup b computes work items b, b + G, b + 2G, ...
// (G = gridDim.x, at most one workgroup per compute unit), treating their K
// slices as one stream: the first slice of the next item is copied while the
// last slice of the current one is computed, and the current item's output
// leaves with direct global stores that drain while the next item computes.
// kNB: n-blocks of 16 columns per wave, so the tile is 256 x BN with BN = 32 kNB
// (8: 256; the row-scaled kernel also comes with 6 and 4, BN = 192 and 128, so
// that more shapes fill the compute units in whole rounds without a split of K).
template <bool kRowScaledB, bool kBf16Out, bool kToWs, bool kAcc = false, bool kGlu = false, bool kKT = false,
          int kNB = 8, bool kSpread = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_bw_kernel(GemmArgs g) {
  static_assert(kNB == 8 || (kRowScaledB && (kNB == 6 || kNB == 4)), "narrow tiles: row-scaled kernel only");
  static_assert(!kSpread || (kNB == 8 && !kGlu), "spread copies: interior 256-wide tiles");
  constexpr int BN = 32 * kNB;            // tile width
  constexpr int WN = 16 * kNB;            // columns per wave
  constexpr int NGB = kNB / 2;            // 8-row groups of B copied by each wave
  static_assert(!kAcc || (!kBf16Out && !kToWs), "accumulate mode stores fp32 directly");
  static_assert(!kGlu || (!kRowScaledB && kBf16Out && !kToWs && !kAcc), "the SwiGLU epilogue follows an fprop");
  static_assert(!kKT || (kRowScaledB && !kGlu), "token-major operands are the wgrad's");
  // [buf][A/B][256 rows x 128 B] operand slices (token-major: 128 token rows
  // x 256 B); [buf][sA/sB][256] scales
  __shared__ __align__(1024) uint8_t smem[2][2][kSliceBytes];
  __shared__ __align__(16) float sscale[2][2][kBM];
  __shared__ __align__(16) uint32_t xamax[kGlu ? 2 * kBM : 1];   // SwiGLU: row maxima of |h| per half tile

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int total_items = g.ntiles * g.splits;
  int item = blockIdx.x;
  if (item >= total_items) return;
  const int K = (int)g.K;
  const bool ktail = (K & (kBK - 1)) != 0;

  // ---- global -> LDS copy plan.  Wave w fills LDS row groups grp = 4w + j
  // (j = 0..3) of 8 rows; lane -> row grp*8 + (lane/8), physical chunk lane%8,
  // whose logical chunk is (lane%8) ^ swz(row).  Rows past M / N are
  // redirected to the tile's first row (finite codes whose products are
  // never stored).
  const int rig = lane >> 3;
  auto dma_chunk = [](int ln, int j) {          // logical chunk (bytes) of lane ln in group j
    const int rg = ln >> 3;
    return ((ln & 7) ^ (((rg >> 1) & 1) | ((((rg >> 2) ^ (j >> 1)) & 1) << 2))) * 16;
  };
  const uint32_t lds0 = lds_addr(&smem[0][0][0]);
  const uint32_t lds_s0 = lds_addr(&sscale[0][0][0]);
  // Interior tiles: lane offsets (row group j, row rig, logical chunk) are
  // shared by A and B; the wave's first row group and the K slice go into the
  // scalar bases.
  // Token-major operands (kKT): tile row k holds 256 bytes (16 chunks of 16
  // M or N values) of token k of the slice; chunk c of row k sits at chunk
  // c ^ kt_swz(k), kt_swz(k) = (k & 7) | ((k >> 5) & 1) << 3, so that the
  // transposing fragment reads below (rows 32q + 8s + r, r < 8) are free of
  // bank conflicts.  Lane l of copy j fills row 16w + 4j + l/16 at physical
  // chunk l % 16; the offsets depend on j only through its parity.  A B tile
  // narrower than 256 columns (nch chunks) keeps the 256-byte row: a lane
  // whose logical chunk lies past the tile copies the tile's last chunk into
  // a slot no fragment reads.
  auto kt_voff = [&](int j, int64_t ld, int nch) -> uint32_t {
    const int kr = 4 * j + (lane >> 4);                       // row within the wave's 16 (< 16)
    const int sw = (kr & 7) | (((w >> 1) & 1) << 3);          // kt_swz(16w + kr)
    return (uint32_t)((lane >> 4) * ld + (min((lane & 15) ^ sw, nch - 1) << 4));
  };
  const uint32_t voff0 = kKT ? kt_voff(0, g.M, 16) : (uint32_t)(rig * K + dma_chunk(lane, 0));
  const uint32_t voff1 = kKT ? kt_voff(1, g.M, 16) : (uint32_t)((8 + rig) * K + dma_chunk(lane, 1));
  const uint32_t voff2 = kKT ? kt_voff(0, g.N, BN / 16) : (uint32_t)((16 + rig) * K + dma_chunk(lane, 2));
  const uint32_t voff3 = kKT ? kt_voff(1, g.N, BN / 16) : (uint32_t)((24 + rig) * K + dma_chunk(lane, 3));
  // Narrow tiles: wave w copies B row groups NGB w + j (j < NGB); the chunk
  // swizzle takes bit 1 of the row group (row bit 4), which is not j's own here.
  auto dma_chunk_b = [&](int j) {
    const int grp = NGB * w + j;
    return ((lane & 7) ^ (((rig >> 1) & 1) | ((((rig >> 2) ^ (grp >> 1)) & 1) << 2))) * 16;
  };
  uint32_t vb[NGB];
#pragma unroll
  for (int j = 0; j < NGB; ++j) vb[j] = (uint32_t)((8 * j + rig) * K + dma_chunk_b(j));

  // Per-lane values that only edge tiles, the ragged last slice and the scale
  // copies need are recomputed from an opaque lane id at each call, so that
  // they occupy no VGPRs across the K loop.
  auto issue_scales = [&](const Tile &tl, int kb, int buf) {
    // wave 0 copies sA rows m0..m0+255; wave 1 copies sB columns n0.. (row-scaled
    // B) or the tile's two block scales (block-scaled B)
    if (w > 1) return;
    const uint32_t ls = lds_s0 + buf * 2 * kBM * 4;
    int ln = __lane_id();
    asm volatile("" : "+v"(ln));
    const bool full = tl.rows_a == kBM && tl.rows_b == BN;
    if (full && (g.M & 3) == 0 && (!kRowScaledB || (g.N & 3) == 0) && (w == 0 || kRowScaledB)) {
      // 16-byte-aligned rows: lane l brings the scales of rows (columns) 4l .. 4l+3
      const float *src = w == 0 ? g.sa + (int64_t)kb * g.M + tl.m0 : g.sb + (int64_t)kb * g.N + tl.n0;
      if (w == 0 || BN == kBM || ln < BN / 4) dma16_s(src, (uint32_t)ln * 16, ls + (w == 0 ? 0 : kBM * 4));
      return;
    }
    if (w == 0) {
      const float *src = g.sa + (int64_t)kb * g.M + tl.m0;
#pragma unroll
      for (int j = 0; j < 4; ++j) dma4_s(src, (uint32_t)min(ln + 64 * j, tl.rows_a - 1) * 4, ls + 256 * j);
    } else if constexpr (kRowScaledB) {
      const float *src = g.sb + (int64_t)kb * g.N + tl.n0;
#pragma unroll
      for (int j = 0; j < BN / 64; ++j) dma4_s(src, (uint32_t)min(ln + 64 * j, tl.rows_b - 1) * 4, ls + kBM * 4 + 256 * j);
    } else if constexpr (kGlu) {
      // lane 0 brings the scale of the tile's gate block, lane 1 that of its up block
      const float *src = g.sb + (int64_t)(tl.n0 / kBK) * g.nk + kb;
      dma4_s(src, (uint32_t)(ln == 1 ? g.I / kBK : 0) * (uint32_t)g.nk * 4, ls + kBM * 4);
    } else {
      // lane l brings sb[n-block nb0 + l][kb] (clamped); lanes 0 and 1 cover
      // the tile's two 128-column blocks
      const int nb0 = tl.n0 / kBK;
      const int nb_last = (int)((g.N - 1) / kBK) - nb0;
      const float *src = g.sb + (int64_t)nb0 * g.nk + kb;
      dma4_s(src, (uint32_t)min(ln, nb_last) * (uint32_t)g.nk * 4, ls + kBM * 4);
    }
  };

  // Fused SwiGLU: tile row r of B (r = 8j + i, i < 8) is gate row n0 + 4j + i
  // for i < 4 and up row I + n0 + 4j + i - 4 otherwise, so that n-blocks 2p
  // and 2p+1 give each lane the gate and up values of the same 4 h columns.
  auto glu_brow = [&](int r) -> int64_t {
    const int i = r & 7;
    return (int64_t)(4 * (r >> 3)) + (i < 4 ? i : g.I + i - 4);
  };
  auto issue_slice_kt = [&](const Tile &tl, int kb, int buf) {
    const uint32_t la = lds0 + buf * 2 * kSliceBytes;
    const int64_t k0 = (int64_t)kb * kBK + 16 * w;             // first token row of the wave's copies
    if (tl.rows_a == kBM && tl.rows_b == BN && !(ktail && kb == g.nk - 1)) {
      const uint8_t *pa = g.a + k0 * g.M + tl.m0;
      const uint8_t *pb = g.b + k0 * g.N + tl.n0;
      dma_slice8kt(pa, pa + 4 * g.M, pa + 8 * g.M, pa + 12 * g.M, pb, pb + 4 * g.N, pb + 8 * g.N, pb + 12 * g.N,
                   voff0, voff1, voff2, voff3, la + w * 4096);
    } else {
      // edge tiles and the ragged last slice: chunks past M / N and rows past K read a zero page
      int ln = __lane_id();
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kr = 4 * j + (ln >> 4);
        const int64_t kg = k0 + kr;
        const int c = (ln & 15) ^ ((kr & 7) | (((w >> 1) & 1) << 3));
        const bool kin = kg < g.K;
        const uint8_t *pa = kin && 16 * c < tl.rows_a ? g.a + kg * g.M + tl.m0 + 16 * c : g_zero16;
        const uint8_t *pb = kin && 16 * c < tl.rows_b ? g.b + kg * g.N + tl.n0 + 16 * c : g_zero16;
        dma16_v(pa, la + w * 4096 + j * 1024);
        dma16_v(pb, la + kSliceBytes + w * 4096 + j * 1024);
      }
    }
    issue_scales(tl, kb, buf);
  };
  auto issue_slice = [&](const Tile &tl, int kb, int buf) {
    if constexpr (kKT) {
      issue_slice_kt(tl, kb, buf);
      return;
    }
    const int kofs = kb * kBK;
    const uint32_t la = lds0 + buf * 2 * kSliceBytes;
    const uint8_t *a_tile = g.a + (int64_t)tl.m0 * g.K;
    const uint8_t *b_tile = g.b + (int64_t)tl.n0 * g.K;
    if (tl.rows_a == kBM && tl.rows_b == BN && !(ktail && kb == g.nk - 1)) {
      if constexpr (kNB != 8) {
        dma_slice_narrow<NGB>(a_tile + (int64_t)(w * 32) * g.K + kofs, b_tile + (int64_t)(w * 8 * NGB) * g.K + kofs,
                              voff0, voff1, voff2, voff3, vb, la + w * 4096, la + kSliceBytes + w * (1024 * NGB));
      } else if constexpr (kGlu) {
        // the wave's row groups 4w .. 4w+3 start at gate row n0 + 16w
        int ln = __lane_id();
        asm volatile("" : "+v"(ln));
        const uint32_t rb = (uint32_t)glu_brow(ln >> 3) * (uint32_t)K;
        dma_slice8ab(a_tile + (int64_t)(w * 32) * g.K + kofs, b_tile + (int64_t)(w * 16) * g.K + kofs, voff0, voff1,
                     voff2, voff3, rb + (uint32_t)dma_chunk(ln, 0), rb + (uint32_t)(4 * K + dma_chunk(ln, 1)),
                     rb + (uint32_t)(8 * K + dma_chunk(ln, 2)), rb + (uint32_t)(12 * K + dma_chunk(ln, 3)),
                     la + w * 4096);
      } else {
        dma_slice8(a_tile + (int64_t)(w * 32) * g.K + kofs, b_tile + (int64_t)(w * 32) * g.K + kofs, voff0,
                   voff1, voff2, voff3, la + w * 4096);
      }
    } else {
      // edge tiles and the ragged last slice: chunks at or past K read a zero page
      const uint32_t lb = la + kSliceBytes;
      int ln = __lane_id();
      asm volatile("" : "+v"(ln));
      const int rg = ln >> 3;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int grp = w * 4 + j;
        const int r = grp * 8 + rg;
        const int kc = dma_chunk(ln, j);
        const bool kin = kofs + kc < K;
        const uint8_t *pa = kin ? a_tile + kofs + (r < tl.rows_a ? (int64_t)r * K : 0) + kc : g_zero16;
        dma16_v(pa, la + grp * 1024);
        if constexpr (kNB == 8) {
          const int64_t br = kGlu ? glu_brow(r) : (r < tl.rows_b ? (int64_t)r : 0);
          const uint8_t *pb = kin ? b_tile + kofs + br * K + kc : g_zero16;
          dma16_v(pb, lb + grp * 1024);
        }
      }
      if constexpr (kNB != 8) {
#pragma unroll
        for (int j = 0; j < NGB; ++j) {
          const int grp = NGB * w + j;
          const int r = grp * 8 + rg;
          const int kc = ((ln & 7) ^ (((rg >> 1) & 1) | ((((rg >> 2) ^ (grp >> 1)) & 1) << 2))) * 16;
          const bool kin = kofs + kc < K;
          const uint8_t *pb = kin ? b_tile + kofs + (r < tl.rows_b ? (int64_t)r * K : 0) + kc : g_zero16;
          dma16_v(pb, lb + grp * 1024);
        }
      }
    }
    issue_scales(tl, kb, buf);
  };

  // ---- fragment read plan: lane reads logical chunks 2q and 2q+1 (q = lane
  // / 16) of one row per 16-row block: A row fr (= lane % 16) of its m-block.
  // The MFMAs take the B fragment as their first operand, so each 16x16 result
  // is (n, m): lane (q, fr) holds output row fr of the m-block at the 4 output
  // columns of B-fragment rows 4q .. 4q+3.  B-fragment row i of n-block nb is
  // B row  wn*128 + 32*(nb/2) + 4*(nb%2) + 8*(i/4) + i%4,  so that n-blocks 2p
  // and 2p+1 give lane (q, fr) the 8 consecutive output columns
  // wn*128 + 32p + 8q .. +7 (one 16-byte bf16 store).
  const int fr = lane & 15;
  const int q = lane >> 4;
  // Byte offsets of chunk 2q of a lane's fragment row; chunk 2q+1 is at ^16.
  // The swizzle of A row wm*64 + 16mb + fr depends on fr and mb%2; that of B
  // row wn*128 + 32*(nb/2) + 4*(nb%2) + cfr on fr and nb%2.
  const int cfr = 8 * (fr >> 2) + (fr & 3);                      // B row of fragment row fr, within its group
  auto swz_a = [&](int t) { return ((fr >> 1) & 1) | ((((fr >> 2) ^ t) & 1) << 2); };
  auto swz_b = [&](int t) { return ((fr >> 1) & 1) | (((t ^ (fr >> 3)) & 1) << 2); };
  const uint32_t aoff0 = (uint32_t)(fr * kBK + ((2 * q) ^ swz_a(0)) * 16);
  const uint32_t aoff1 = (uint32_t)(fr * kBK + ((2 * q) ^ swz_a(1)) * 16);
  const uint32_t boff0 = (uint32_t)(cfr * kBK + ((2 * q) ^ swz_b(0)) * 16);
  const uint32_t boff1 = (uint32_t)(cfr * kBK + ((2 * q) ^ swz_b(1)) * 16);

  v4f acc[4][kNB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = (v4f){0.f, 0.f, 0.f, 0.f};

  auto frag = [](const uint8_t *row_base, uint32_t off) -> v8i {
    const v4i lo = *reinterpret_cast<const v4i *>(row_base + off);
    const v4i hi = *reinterpret_cast<const v4i *>(row_base + (off ^ 16u));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // A fragment of m-block mb, B fragment of n-block nb (compile-time after unrolling)
  // Token-major tiles: a transposing LDS read (ds_read_b64_tr_b8) lets a group
  // of 16 lanes supply 16 rows of 8 bytes and gives lane i byte i % 8 of rows
  // 2r + i / 8 (r < 8).  With row 2r + h = 8 bytes of token 8s + r at columns
  // r0 + 8h .., lane (q, fr) receives tokens 32q + 8s .. +7 of column r0 + fr:
  // four reads (s = 0..3) make the 32 bytes of K that the MFMA takes from it.
  const uint32_t tr_lane = (uint32_t)((32 * q + (fr >> 1)) * 256 + 8 * (fr & 1));
  const uint32_t tr_swz = (uint32_t)((fr >> 1) | ((q & 1) << 3));     // kt_swz of the lane's rows
  typedef int v2i __attribute__((ext_vector_type(2)));
  auto frag_tr = [&](const uint8_t *tile, int r0) -> v8i {
    const uint32_t a = lds_addr(tile) + tr_lane + ((((uint32_t)r0 >> 4) ^ tr_swz) << 4);
    v8i out;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i *)(a + 2048u * s2));
      out[2 * s2] = v.x;
      out[2 * s2 + 1] = v.y;
    }
    return out;
  };
  auto load_fragA = [&](const uint8_t *base, int mb) -> v8i {
    if constexpr (kKT) return frag_tr(base, wm * 64 + mb * 16);
    return frag(base + (wm * 64 + mb * 16) * kBK, (mb & 1) ? aoff1 : aoff0);
  };
  auto load_fragB = [&](const uint8_t *base, int nb) -> v8i {
    if constexpr (kKT) return frag_tr(base, wn * WN + nb * 16);
    return frag(base + (wn * WN + 32 * (nb >> 1) + 4 * (nb & 1)) * kBK, (nb & 1) ? boff1 : boff0);
  };
  // first B-fragment column of n-block nb seen by lane (q, fr), relative to the wave's 128
  // (token-major tiles: the 16 fragment rows are 16 consecutive columns)
  auto colB = [&](int nb) { return kKT ? 16 * nb + 4 * q : 32 * (nb >> 1) + 4 * (nb & 1) + 8 * q; };

  // ---- K loop.  Slice s of the stream is computed from buffer s & 1 while
  // slice s+1 is copied into the other one.  The barrier that publishes slice
  // s+1 sits before the last n-block step of slice s, so that the reads of
  // slice s+1's A fragments, first B fragment and scales overlap the MFMAs of
  // that step instead of stalling every wave at the start of the slice.
  v8i af[4];                 // A fragments of the wave's 4 m-blocks
  v8i bf[2];                 // B fragments of n-blocks nb (in use) and nb+1 (landing)
  float sa[4];               // row scale sA of the lane's row in each m-block
  v4f sbn0 = {1.f, 1.f, 1.f, 1.f};   // row-scaled B: column scales of the coming slice's n-block 0
  float sbk = 1.0f;          // block-scaled B: the coming slice's scale of the wave's 128 columns
  float sbu = 1.0f;          // fused SwiGLU: sbk is the gate block's scale, sbu the up block's
  auto load_scales = [&](int buf) {
    const float *lsa = sscale[buf][0];
    const float *lsb = sscale[buf][1];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) sa[mb] = lsa[wm * 64 + mb * 16 + fr];
    if constexpr (kRowScaledB) sbn0 = *reinterpret_cast<const v4f *>(&lsb[wn * WN + colB(0)]);
    else if constexpr (kGlu) {
      sbk = lsb[0];
      sbu = lsb[1];
    } else sbk = lsb[wn];
  };

  // One slice from buffer `buf`.  Step nb issues the 4 MFMAs of n-block nb;
  // the partial of n-block nb-1 is promoted into the accumulators from P[mb]
  // right before MFMA (nb, mb) overwrites it, and the B fragment of n-block
  // nb+1 is read one step ahead.  kNext: slice kb_next of item `nxt` follows.
  auto slice = [&](int buf, const Tile &nxt, int kb_next, auto next_c, auto preload_c, auto first_c) {
    constexpr bool kNext = decltype(next_c)::value;           // a slice follows: copy it now
    constexpr bool kPre = kNext && decltype(preload_c)::value; // read its fragments in the last step
    constexpr bool kFirst = decltype(first_c)::value;          // first slice of an item: accumulators start at 0
    const uint8_t *Bs = smem[buf][1];
    const float *lsb = sscale[buf][1];
    v4f P[4];
    v4f sbv[kNB];              // row-scaled B: column scales of each n-block
    sbv[0] = sbn0;
    float sc[4];               // block-scaled B: promotion factors sA * sB
    float scu[4];              // fused SwiGLU: those of the up n-blocks (odd nb)
    // The buffer of the previous slice was released by the barrier inside it.
    // kSpread (every tile interior, K a multiple of 128): the scales go out
    // now and the operand copies one A/B row-group pair per n-block step over
    // steps 0-3, so that no wave stalls behind a burst of eight copies.
    if constexpr (kNext && !kSpread) issue_slice(nxt, kb_next, buf ^ 1);
    if constexpr (kNext && kSpread) issue_scales(nxt, kb_next, buf ^ 1);
    // token-major slices: 16 token rows per wave, copy j the rows 4j .. 4j+3 of them
    const uint8_t *spa = kKT ? g.a + ((int64_t)kb_next * kBK + 16 * w) * g.M + nxt.m0
                             : g.a + (int64_t)(nxt.m0 + w * 32) * g.K + kb_next * kBK;
    const uint8_t *spb = kKT ? g.b + ((int64_t)kb_next * kBK + 16 * w) * g.N + nxt.n0
                             : g.b + (int64_t)(nxt.n0 + w * 32) * g.K + kb_next * kBK;
    const uint32_t sla = lds0 + (buf ^ 1) * 2 * kSliceBytes + w * 4096;
    auto promote = [&](int pb, int mb) {
      const v4f prev = kFirst ? (v4f){0.f, 0.f, 0.f, 0.f} : acc[mb][pb];
      if constexpr (kRowScaledB) {
        // the scale products sA * sB need no MFMA result: only the FMA waits for P
        acc[mb][pb] = __builtin_elementwise_fma(P[mb], sbv[pb] * (v4f)sa[mb], prev);
      } else {
        acc[mb][pb] = __builtin_elementwise_fma(P[mb], (v4f)((kGlu && (pb & 1)) ? scu[mb] : sc[mb]), prev);
      }
    };
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      __builtin_amdgcn_sched_barrier(0);
      if (nb == kNB - 1) {
        // Every wave holds its n-block 7 fragment (lgkmcnt) and has landed its
        // share of the next slice (vmcnt): past the barrier the next slice is
        // readable and nothing reads this slice's buffer any more.
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kNext && kSpread && nb < 4) {
        if constexpr (kKT)
          dma_pair_ab(spa + (int64_t)(4 * nb) * g.M, spb + (int64_t)(4 * nb) * g.N, (nb & 1) ? voff1 : voff0,
                      (nb & 1) ? voff3 : voff2, sla + 1024 * nb);
        else
          dma_pair(spa, spb, nb == 0 ? voff0 : nb == 1 ? voff1 : nb == 2 ? voff2 : voff3, sla + 1024 * nb);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kRowScaledB && nb + 1 < kNB) sbv[nb + 1] = *reinterpret_cast<const v4f *>(&lsb[wn * WN + colB(nb + 1)]);
      if (nb + 1 < kNB) bf[(nb + 1) & 1] = load_fragB(Bs, nb + 1);
      if (nb == kNB - 1 && kPre) bf[0] = load_fragB(smem[buf ^ 1][1], 0);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (nb > 0) promote(nb - 1, mb);
        P[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bf[nb & 1], af[mb], (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        if (nb == kNB - 1 && kPre) af[mb] = load_fragA(smem[buf ^ 1][0], mb);
        if (nb == 0 && !kRowScaledB) sc[mb] = sa[mb] * sbk;
        if (nb == 0 && kGlu) scu[mb] = sa[mb] * sbu;
      }
      // issue order within the step: LDS reads first (a whole step to land),
      // then VALU groups between the MFMAs
      constexpr int kV = kRowScaledB ? 8 : 4;
      constexpr int kS = kRowScaledB ? 1 : 0;
      constexpr int kF = 2;  // LDS reads per group (also for the 4-read token-major fragments: it schedules better)
      if (nb == 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, kF + kS, 0);               // LDS reads
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
          if (!kRowScaledB) __builtin_amdgcn_sched_group_barrier(0x002, kGlu ? 2 : 1, 0);  // VALU
        }
      } else if (nb < kNB - 1) {
        __builtin_amdgcn_sched_group_barrier(0x100, kF + kS, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      } else {
        if (kPre) __builtin_amdgcn_sched_group_barrier(0x100, kF, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (kPre) __builtin_amdgcn_sched_group_barrier(0x100, kF, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) promote(kNB - 1, mb);
    if constexpr (kPre) load_scales(buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Output of one item straight from the accumulators: lane (q, fr) holds,
  // for m-block mb and n-block pair p, row m0 + wm*64 + 16mb + fr at the 8
  // columns n0 + wn*128 + 32p + 8q .. +7 (n-block 2p: the first 4, 2p+1: the
  // last 4): one 16-byte store of bf16, two of fp32.
  // Fused SwiGLU epilogue.  Lane (q, fr) holds, for m-block mb and pair p,
  // row m0 + wm*64 + 16mb + fr at h columns n0 + wn*64 + 16p + 4q .. +3: the
  // gate values in acc[mb][2p] and the up values in acc[mb][2p+1].  Both are
  // rounded to bf16 (the gate/up output), h = SwiGLU(g, u) in bf16, and each
  // row's 128 h columns (this wave's 64 and the partner wave's, wn ^ 1) form
  // one 1x128 tile: scale from the tile's max |h|, codes h / s.
  auto glu_store = [&](const Tile &tl) {
    const int hc = tl.n0 + wn * 64 + 4 * q;
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    typedef float v2f __attribute__((ext_vector_type(2)));
    auto pk2 = [](float a, float b) -> uint32_t {     // the bf16 output's conversion (RNE)
      return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
    };
    u32x2 gp[4][4], up[4][4], hp[4][4];   // packed bf16 gate, up and h of (mb, p)
    uint64_t slow = 0;                    // bit 16mb + 4p + e: element e of (mb, p) needs fp64
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const v4f ga = acc[mb][2 * p], ua = acc[mb][2 * p + 1];
        gp[mb][p] = (u32x2){pk2(ga[0], ga[1]), pk2(ga[2], ga[3])};
        up[mb][p] = (u32x2){pk2(ua[0], ua[1]), pk2(ua[2], ua[3])};
        uint32_t hb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t gw = gp[mb][p][e >> 1], uw = up[mb][p][e >> 1];
          bool sl;
          hb[e] = swiglu_fast((e & 1) ? bf16hi(gw) : bf16lo(gw), (e & 1) ? bf16hi(uw) : bf16lo(uw), sl);
          slow |= (uint64_t)sl << (16 * mb + 4 * p + e);
        }
        hp[mb][p] = (u32x2){(hb[0] & 0xffffu) | hb[1] << 16, (hb[2] & 0xffffu) | hb[3] << 16};
      }
    if (g.out != nullptr) {
      uint16_t *gu = reinterpret_cast<uint16_t *>(g.out);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int m = tl.m0 + wm * 64 + mb * 16 + fr;
        if (m >= g.M) continue;
        uint16_t *row = gu + (int64_t)m * 2 * g.I + hc;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          *reinterpret_cast<u32x2 *>(row + 16 * p) = gp[mb][p];
          *reinterpret_cast<u32x2 *>(row + g.I + 16 * p) = up[mb][p];
        }
      }
    }
    // rare elements near a bf16 rounding midpoint, or with |g| > 64: fp64,
    // one element per iteration, picked out of the packed words by selects
    while (slow) {
      const int i = __builtin_ctzll(slow);
      slow &= slow - 1;
      const int wi = i >> 1;
      uint32_t gw = 0, uw = 0;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const bool hit = wi == (4 * mb + p) * 2 + hh;
            gw = hit ? gp[mb][p][hh] : gw;
            uw = hit ? up[mb][p][hh] : uw;
          }
      const bool odd = i & 1;
      const uint32_t h = swiglu_f64(odd ? bf16hi(gw) : bf16lo(gw), odd ? bf16hi(uw) : bf16lo(uw));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const uint32_t w0 = hp[mb][p][hh];
            const uint32_t merged = odd ? ((w0 & 0xffffu) | (h << 16)) : ((w0 & 0xffff0000u) | h);
            hp[mb][p][hh] = wi == (4 * mb + p) * 2 + hh ? merged : w0;
          }
    }
    // row maxima of |h|: the lane's 16 values, the 4 lanes q of the row, then
    // the partner wave through LDS
    uint32_t am[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      uint32_t mx = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t w0 = hp[mb][p][hh];
          mx = max(mx, max(w0 & 0x7fffu, (w0 >> 16) & 0x7fffu));
        }
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
      am[mb] = mx;
      if (q == 0) xamax[wn * kBM + wm * 64 + mb * 16 + fr] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = tl.m0 + wm * 64 + mb * 16 + fr;
      const TileQ tq = make_tileq(mag_to_float(max(am[mb], xamax[(wn ^ 1) * kBM + wm * 64 + mb * 16 + fr])));
      if (m >= g.M) continue;
      uint8_t *row = g.hq + (int64_t)m * g.I + hc;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const u32x2 w0 = hp[mb][p];
        *reinterpret_cast<uint32_t *>(row + 16 * p) =
            pack4_e4m3(quot(bf16lo(w0.x), tq), quot(bf16hi(w0.x), tq), quot(bf16lo(w0.y), tq), quot(bf16hi(w0.y), tq));
      }
      if (wn == 0 && q == 0) g.hs[(int64_t)(tl.n0 / kBK) * g.M + m] = tq.s;
    }
  };

  // fp32 pair (a0: columns c .. c+3, a1: c+4 .. c+7 of row fr) stored as whole 128-byte
  // row segments: lane pairs (fr, fr ^ 1) trade 16 bytes through a DPP swap (moved as
  // integer dwords), so that one store covers 32 columns of 8 rows (even rows, then odd
  // rows) -- 8 whole cache lines.  rowx / rowy: the element offsets of rows fr & ~1 and
  // fr | 1, plus column c + 4 (fr & 1).
  auto store_f32_pair = [&](float *base, int64_t rowx, int64_t rowy, v4f a0, v4f a1) {
    const bool odd = fr & 1;
    const u32x4 e = __builtin_bit_cast(u32x4, odd ? a0 : a1);
    u32x4 swu;
#pragma unroll
    for (int j = 0; j < 4; ++j) swu[j] = (uint32_t)__builtin_amdgcn_mov_dpp((int)e[j], 0xB1, 0xF, 0xF, false);
    const v4f sw = __builtin_bit_cast(v4f, swu);
    *reinterpret_cast<v4f *>(base + rowx) = odd ? sw : a0;
    *reinterpret_cast<v4f *>(base + rowy) = odd ? a1 : sw;
  };

  auto store_item = [&](const Tile &tl) {
    if constexpr (kGlu) {
      glu_store(tl);
      return;
    }
    const int64_t wbase = (int64_t)(tl.m0 + wm * 64) * g.N + tl.n0 + wn * WN;
    const int64_t loff = (int64_t)fr * g.N + 8 * q;
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    auto pk = [](v4f v, int h) -> uint32_t {
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(h ? __builtin_shufflevector(v, v, 2, 3)
                                                                    : __builtin_shufflevector(v, v, 0, 1), v2bf));
    };
    if constexpr (kToWs) {
      // split-K partial: the tile's own 256 x 256 fp32 block of the workspace,
      // [split][tile within the launch][row][column], written whole (rows and
      // columns past M / N hold finite values the reduction never reads)
      float *o = g.ws + ((int64_t)tl.split * g.ntiles + tl.local) * (kBM * BN) + (wm * 64) * BN + wn * WN;
      if constexpr (!kKT) {
        const int cx = 8 * q + 4 * (fr & 1);
        const int rx = (fr & ~1) * BN + cx, ry = (fr | 1) * BN + cx;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int pp = 0; pp < kNB / 2; ++pp)
            store_f32_pair(o + (mb * 16) * BN + 32 * pp, rx, ry, acc[mb][2 * pp], acc[mb][2 * pp + 1]);
        return;
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        float *ob = o + (mb * 16 + fr) * BN;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) *reinterpret_cast<v4f *>(ob + colB(nb)) = acc[mb][nb];
      }
      return;
    }
    if constexpr (kKT) {
      // token-major tiles: lane (q, fr) holds columns 16nb + 4q .. +3 of n-block nb
      if (kSpread || (tl.rows_a == kBM && tl.rows_b == BN && (g.N & 3) == 0)) {
        const int64_t lk = (int64_t)fr * g.N + 4 * q;
        if constexpr (kBf16Out && !kToWs) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            uint16_t *ob = reinterpret_cast<uint16_t *>(g.out) + wbase + (int64_t)(mb * 16) * g.N + lk;
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb)
              *reinterpret_cast<u32x2 *>(ob + 16 * nb) = (u32x2){pk(acc[mb][nb], 0), pk(acc[mb][nb], 1)};
          }
        } else {
          float *o = reinterpret_cast<float *>(g.out) + wbase;
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            float *ob = o + (int64_t)(mb * 16) * g.N + lk;
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
              v4f *p0 = reinterpret_cast<v4f *>(ob + 16 * nb);
              if constexpr (kAcc) {
                const v4f o0 = *p0;
                *p0 = o0 + acc[mb][nb];
              } else {
                *p0 = acc[mb][nb];
              }
            }
          }
        }
        return;
      }
    }
    if constexpr (kBf16Out && !kToWs) {
      const bool fast = kSpread || (!kKT && tl.rows_a == kBM && tl.rows_b == BN && (g.N & 7) == 0);
      if (fast && kNB % 4 == 0) {
        // whole 128-byte row segments: lane pairs (fr, fr ^ 1) trade 16 bytes so that
        // one store covers 64 columns of 8 rows (even rows, then odd rows)
        const bool odd = fr & 1;
        const int64_t cx = 8 * (q + 4 * (fr & 1));
        const int64_t offx = (int64_t)(fr & ~1) * g.N + cx, offy = (int64_t)(fr | 1) * g.N + cx;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          uint16_t *ob = reinterpret_cast<uint16_t *>(g.out) + wbase + (int64_t)(mb * 16) * g.N;
#pragma unroll
          for (int t = 0; t < kNB / 4; ++t) {
            const u32x4 d0 = (u32x4){pk(acc[mb][4 * t], 0), pk(acc[mb][4 * t], 1), pk(acc[mb][4 * t + 1], 0),
                                     pk(acc[mb][4 * t + 1], 1)};
            const u32x4 d1 = (u32x4){pk(acc[mb][4 * t + 2], 0), pk(acc[mb][4 * t + 2], 1), pk(acc[mb][4 * t + 3], 0),
                                     pk(acc[mb][4 * t + 3], 1)};
            const u32x4 e = odd ? d0 : d1;
            u32x4 sw;
#pragma unroll
            for (int j = 0; j < 4; ++j) sw[j] = (uint32_t)__builtin_amdgcn_mov_dpp((int)e[j], 0xB1, 0xF, 0xF, false);
            *reinterpret_cast<u32x4 *>(ob + offx + 64 * t) = odd ? sw : d0;
            *reinterpret_cast<u32x4 *>(ob + offy + 64 * t) = odd ? d1 : sw;
          }
        }
      } else if (fast) {
        // 192-column tiles (an odd number of n-block pairs): half segments
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          uint16_t *ob = reinterpret_cast<uint16_t *>(g.out) + wbase + (int64_t)(mb * 16) * g.N;
#pragma unroll
          for (int pp = 0; pp < kNB / 2; ++pp) {
            const v4f a0 = acc[mb][2 * pp], a1 = acc[mb][2 * pp + 1];
            *reinterpret_cast<u32x4 *>(ob + loff + 32 * pp) = (u32x4){pk(a0, 0), pk(a0, 1), pk(a1, 0), pk(a1, 1)};
          }
        }
      } else {
        // edge tiles: lane values from an opaque lane id (none stays live across the K loop)
        int ln = __lane_id();
        asm volatile("" : "+v"(ln));
        const int efr = ln & 15, eq = ln >> 4;
        auto ecol = [&](int nb) { return kKT ? 16 * nb + 4 * eq : 32 * (nb >> 1) + 4 * (nb & 1) + 8 * eq; };
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int m = tl.m0 + wm * 64 + mb * 16 + efr;
          if (m >= g.M) continue;
          uint16_t *ob = reinterpret_cast<uint16_t *>(g.out) + wbase + (int64_t)(mb * 16 + efr) * g.N;
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const int n = tl.n0 + wn * WN + ecol(nb);
            const uint32_t lo = pk(acc[mb][nb], 0), hi = pk(acc[mb][nb], 1);
            const uint16_t h[4] = {(uint16_t)(lo & 0xffffu), (uint16_t)(lo >> 16), (uint16_t)(hi & 0xffffu),
                                   (uint16_t)(hi >> 16)};
            uint16_t *d = ob + ecol(nb);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < g.N) d[e] = h[e];
          }
        }
      }
    } else {
      float *o = reinterpret_cast<float *>(g.out) + wbase;
      const bool fast = kSpread || (!kKT && tl.rows_a == kBM && tl.rows_b == BN && (g.N & 3) == 0);
      if (fast && !kAcc) {
        const int64_t cx = 8 * q + 4 * (fr & 1);
        const int64_t rx = (int64_t)(fr & ~1) * g.N + cx, ry = (int64_t)(fr | 1) * g.N + cx;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int pp = 0; pp < kNB / 2; ++pp)
            store_f32_pair(o + (int64_t)(mb * 16) * g.N + 32 * pp, rx, ry, acc[mb][2 * pp], acc[mb][2 * pp + 1]);
      } else if (fast) {
        // accumulate mode: read, add, write back in the accumulators' own layout
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          float *ob = o + (int64_t)(mb * 16) * g.N;
#pragma unroll
          for (int pp = 0; pp < kNB / 2; ++pp) {
            v4f *p0 = reinterpret_cast<v4f *>(ob + loff + 32 * pp);
            v4f *p1 = reinterpret_cast<v4f *>(ob + loff + 32 * pp + 4);
            const v4f o0 = *p0, o1 = *p1;
            *p0 = o0 + acc[mb][2 * pp];
            *p1 = o1 + acc[mb][2 * pp + 1];
          }
        }
      } else {
        int ln = __lane_id();
        asm volatile("" : "+v"(ln));
        const int efr = ln & 15, eq = ln >> 4;
        auto ecol = [&](int nb) { return kKT ? 16 * nb + 4 * eq : 32 * (nb >> 1) + 4 * (nb & 1) + 8 * eq; };
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int m = tl.m0 + wm * 64 + mb * 16 + efr;
          if (m >= g.M) continue;
          float *ob = o + (int64_t)(mb * 16 + efr) * g.N;
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const int n = tl.n0 + wn * WN + ecol(nb);
            float *d = ob + ecol(nb);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < g.N) d[e] = kAcc ? d[e] + acc[mb][nb][e] : acc[mb][nb][e];
          }
        }
      }
    }
  };

  Tile cur = tile_of(g, item, kGlu);
  issue_slice(cur, kb_at(cur, 0), 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  bf[0] = load_fragB(smem[0][1], 0);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) af[mb] = load_fragA(smem[0][0], mb);
  load_scales(0);

  int buf = 0;
  for (;;) {
    // The first slice of an item writes the accumulators instead of adding to
    // them; an item of one slice starts from cleared accumulators instead.
    if (cur.kb_end - cur.kb_begin > 1) {
      slice(buf, cur, kb_at(cur, 1), std::true_type{}, std::true_type{}, std::true_type{});
      buf ^= 1;
    } else {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
    for (int i = 1; i + 1 < cur.kb_end - cur.kb_begin; ++i) {
      slice(buf, cur, kb_at(cur, i + 1), std::true_type{}, std::true_type{}, std::false_type{});
      buf ^= 1;
    }
    // Last slice of the item: the first slice of the next item is copied and
    // its fragments read meanwhile.  After the last item this re-reads the
    // item's own first slice, which keeps a single code path (a separate
    // final-slice variant costs the register allocator its accumulators).
    const int next_item = item + (int)gridDim.x;
    const bool more = next_item < total_items;
    const Tile nxt = tile_of(g, more ? next_item : item, kGlu);
    // (the SwiGLU epilogue needs the registers of the next item's fragments:
    // those are read after it)
    slice(buf, nxt, kb_at(nxt, 0), std::true_type{}, std::bool_constant<!kGlu>{}, std::false_type{});
    buf ^= 1;
    store_item(cur);
    if constexpr (kGlu) {
      bf[0] = load_fragB(smem[buf][1], 0);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) af[mb] = load_fragA(smem[buf][0], mb);
      load_scales(buf);
    }
    if (!more) break;
    item = next_item;
    cur = nxt;
  }
}

// out[o .. o+W-1] = the sum of the split-K partials ws[s*stride + w ..] in
// increasing split order (then added to the fp32 output in accumulate mode);
// W = 4 (16-byte accesses) when kVec, else 1.
template <bool kBf16Out, bool kAcc, bool kVec>
__device__ __forceinline__ void reduce_at(const float *ws, void *out, int64_t w, int64_t o, int64_t stride, int splits) {
  if constexpr (kVec) {
    v4f v = *reinterpret_cast<const v4f *>(ws + w);
    for (int s = 1; s < splits; ++s) v += *reinterpret_cast<const v4f *>(ws + (int64_t)s * stride + w);
    if constexpr (kBf16Out) {
      *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(out) + o) =
          (u32x2){f32_to_bf16_rne(v[0]) | f32_to_bf16_rne(v[1]) << 16, f32_to_bf16_rne(v[2]) | f32_to_bf16_rne(v[3]) << 16};
    } else {
      v4f *d = reinterpret_cast<v4f *>(reinterpret_cast<float *>(out) + o);
      if constexpr (kAcc) *d = *d + v;
      else *d = v;
    }
  } else {
    float v = ws[w];
    for (int s = 1; s < splits; ++s) v += ws[(int64_t)s * stride + w];
    if constexpr (kBf16Out)
      reinterpret_cast<uint16_t *>(out)[o] = (uint16_t)f32_to_bf16_rne(v);
    else if constexpr (kAcc)
      reinterpret_cast<float *>(out)[o] += v;
    else
      reinterpret_cast<float *>(out)[o] = v;
  }
}

// Sum of the split-K partials of output tiles tile0 .. tile0 + ntiles - 1
// (tiles of 256 x bn).  The workspace holds one 256 x bn fp32 block per split
// and tile, [split][tile - tile0][row][column].  With W elements per thread,
// index e covers row (e / (bn/W)) % 256, columns W * (e % (bn/W)) .. +W-1 of
// tile tile0 + e / (256 bn / W).  kVec needs N % 4 == 0 (a group of 4 columns
// is then either wholly inside the output or wholly past its last column).
template <bool kBf16Out, bool kAcc, bool kVec>
__global__ __launch_bounds__(256) void splitk_reduce_tiles_kernel(const float *ws, void *out, int64_t M, int64_t N,
                                                                  int tiles_m, int tile0, int ntiles, int splits,
                                                                  int bn, int banded) {
  static_assert(!kAcc || !kBf16Out, "accumulate mode is fp32 only");
  constexpr int W = kVec ? 4 : 1;
  const int row_items = bn / W;
  const int64_t tile_elems = (int64_t)kBM * bn;
  const int64_t stride = (int64_t)ntiles * tile_elems;
  const int64_t total = (int64_t)ntiles * kBM * row_items;
  const int64_t gstride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += gstride) {
    const int t = (int)(e / (kBM * row_items));
    const int tile = tile0 + t;
    const int r = (int)((e / row_items) % kBM), c = (int)(e % row_items) * W;
    int tm = tile % tiles_m, tn = tile / tiles_m;
    if (banded) band_tile(tile, tiles_m, tm, tn);
    const int64_t m = (int64_t)tm * kBM + r, n = (int64_t)tn * bn + c;
    if (m >= M || n >= N) continue;
    reduce_at<kBf16Out, kAcc, kVec>(ws, out, (int64_t)t * tile_elems + (int64_t)r * bn + c, m * N + n, stride, splits);
  }
}

template <bool kBf16Out>
__global__ __launch_bounds__(256) void fill_zero_kernel(void *out, int64_t MN) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += stride) {
    if constexpr (kBf16Out)
      reinterpret_cast<uint16_t *>(out)[i] = 0;
    else
      reinterpret_cast<float *>(out)[i] = 0.0f;
  }
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *p, int64_t n, uint32_t v) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// ---------------------------------------------------------------- planning

// Estimated time of one plan: rounds of 256 work items, each of its slices
// plus about 2 slices of fixed cost (first copy, epilogue) at about 1.9 us per
// 256 x 256 slice (a narrower tile's slice takes its share of that, times the
// cost of its extra copies per flop), plus the workspace traffic (every split
// writes an fp32 partial of its tiles and the reduction reads it back) at
// about 4 TB/s.
struct PlanCost {
  double slice_us;     // one slice of one tile
  double tile_bytes;   // fp32 partial of one tile
};

static PlanCost plan_cost(int bn) {
  // per-slice times relative to a 256 x 256 tile's, measured on MI355X at the
  // layer's weight-gradient shapes (a narrow tile copies more bytes per flop,
  // so its slices cost more than its share of the work: 0.86 for 3/4 of it,
  // 0.68 for half)
  const double rel = bn == 256 ? 1.0 : bn == 192 ? 0.86 : 0.68;
  return PlanCost{1.9e-6 * rel, 4.0 * kBM * bn};
}

static void plan_splits(GemmPlan &p, int64_t M, int64_t N, double &best) {
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  const PlanCost c = plan_cost(p.bn);
  const double bw = 4.0e12;
  p.splits = 1;
  p.whole = 0;
  best = 0.0;
  // Split the K loop when the output tiles fill the 256 compute units poorly
  // (a last round of tiles that leaves units idle, or fewer tiles than units).
  // Two forms:
  //  - every tile split s ways;
  //  - when the tiles fill w >= 1 whole rounds and leave r more, the first
  //    256w tiles computed whole by a first launch (direct stores, no
  //    workspace) and only the last r split s ways by a second one (about
  //    3 us more for the extra launch).
  // Splitting must win by 3%; at least 4 slices per split.
  for (int s = 1; s <= 8; ++s) {
    const int spl = (p.nk + s - 1) / s;
    if (s > 1 && (spl < 4 || (p.nk + spl - 1) / spl != s)) continue;
    const double t = (double)((tiles * s + 255) / 256) * (spl + 2) * c.slice_us +
                     (s > 1 ? 2.0 * s * (double)tiles * c.tile_bytes / bw : 0.0);
    if (s == 1 || t < best * 0.97) {
      best = t;
      p.splits = s;
    }
  }
  const int64_t w = tiles / 256, r = tiles % 256;
  for (int s = 2; w > 0 && r > 0 && s <= 8; ++s) {
    const int spl = (p.nk + s - 1) / s;
    if (spl < 4 || (p.nk + spl - 1) / spl != s) continue;
    const double t = (double)w * (p.nk + 2) * c.slice_us + (double)((r * s + 255) / 256) * (spl + 2) * c.slice_us +
                     2.0 * s * (double)r * c.tile_bytes / bw + 3.0e-6;
    if (t < best * 0.97) {
      best = t;
      p.splits = s;
      p.whole = (int)(w * 256);
    }
  }
  (void)M;
  (void)N;
}

GemmPlan plan_gemm(int mode, int64_t M, int64_t N, int64_t K) {
  GemmPlan p{};
  p.nk = (int)((K + kBK - 1) / kBK);
  p.tiles_m = (int)((M + kBM - 1) / kBM);
  p.bn = kBN;
  p.tiles_n = (int)((N + kBN - 1) / kBN);
  p.splits = 1;
  p.whole = 0;
  if (p.tiles_m > 0 && p.tiles_n > 0 && p.nk > 0) {
    double best = 0.0;
    plan_splits(p, M, N, best);
    // The weight gradient (row-scaled B, in both operand layouts) also has
    // tiles 192 and 128 wide; a narrower tile must win by 3% too.
    if (mode == 2 || mode == 3) {
      for (int bn : {192, 128}) {
        GemmPlan q = p;
        q.bn = bn;
        q.tiles_n = (int)((N + bn - 1) / bn);
        double t = 0.0;
        plan_splits(q, M, N, t);
        if (t < best * 0.97) {
          best = t;
          p = q;
        }
      }
    }
  }
  p.spl = (p.nk + p.splits - 1) / p.splits;
  if (p.spl > 0) p.splits = (p.nk + p.spl - 1) / p.spl;
  if (p.splits == 1) p.whole = 0;
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  // one 256 x bn fp32 block per split of each split tile
  p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)(tiles - p.whole) * kBM * p.bn * sizeof(float) : 0;
  return p;
}

// Compute units of the current device (one persistent workgroup each),
// queried once per device; callers on several host threads may race to fill
// an entry, which is harmless since they all store the same count.
static int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// One kernel of the family for a mode (RB: row-scaled B; KT: token-major
// operands; NB: n-blocks per wave, the tile width over 32).
template <bool RB, bool KT, int NB = 8>
static void launch_mode(const dim3 &grid, hipStream_t stream, const GemmArgs &g, bool to_ws, bool acc, bool bf16) {
  if (to_ws)
    hipLaunchKernelGGL((gemm_fp8_bw_kernel<RB, false, true, false, false, KT, NB>), grid, dim3(kThreads), 0, stream, g);
  else if (acc)
    hipLaunchKernelGGL((gemm_fp8_bw_kernel<RB, false, false, true, false, KT, NB>), grid, dim3(kThreads), 0, stream, g);
  else if (bf16)
    hipLaunchKernelGGL((gemm_fp8_bw_kernel<RB, true, false, false, false, KT, NB>), grid, dim3(kThreads), 0, stream, g);
  else
    hipLaunchKernelGGL((gemm_fp8_bw_kernel<RB, false, false, false, false, KT, NB>), grid, dim3(kThreads), 0, stream, g);
}

hipError_t run_gemm(int mode, const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                    void *out, bool bf16_out, bool accumulate, int64_t M, int64_t N, int64_t K, void *ws,
                    hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t MN = M * N;
  if (K == 0) {
    if (accumulate) return hipSuccess;            // out + 0
    const int blocks = (int)std::min<int64_t>((MN + 255) / 256, 65536);
    if (bf16_out) hipLaunchKernelGGL(fill_zero_kernel<true>, dim3(blocks), dim3(256), 0, stream, out, MN);
    else hipLaunchKernelGGL(fill_zero_kernel<false>, dim3(blocks), dim3(256), 0, stream, out, MN);
    return hipGetLastError();
  }
  const GemmPlan p = plan_gemm(mode, M, N, K);
  GemmArgs g{};
  g.a = a; g.sa = sa; g.b = b; g.sb = sb; g.out = out; g.ws = (float *)ws;
  g.M = M; g.N = N; g.K = K;
  g.nk = p.nk; g.tiles_m = p.tiles_m; g.tiles_n = p.tiles_n; g.bn = p.bn;
  const int tiles = p.tiles_m * p.tiles_n;
  const bool row_b = mode == 2 || mode == 3;
  // 8 column tiles and an A operand larger than half the 256 MB MALL (so the
  // row-tile walk's second read of each A panel comes from HBM): the tiles
  // are numbered in row bands (band_tile) by every launch of the GEMM and by
  // its reduction.  Each tile's K order still depends on its row tile alone.
  // Where A fits the MALL the walk measured faster.
  const int banded = p.tiles_n == 8 && p.bn == kBN && M * K > (int64_t(128) << 20);
  // one persistent launch over tiles [tile0, tile0 + ntiles), each split s ways
  auto launch = [&](int tile0, int ntiles, int s, int spl, bool to_ws) {
    g.tile0 = tile0; g.ntiles = ntiles; g.splits = s; g.spl = spl;
    // weight gradients over the whole tile grid in whole rounds of 256 items:
    // the blocked item order (a function of the plan alone, so both operand
    // layouts sum every output in the same order)
    g.blocked = row_b && tile0 == 0 && ntiles == tiles && p.tiles_m % 4 == 0 && p.tiles_n % 8 == 0 &&
                (int64_t)ntiles * s % 256 == 0;
    g.banded = !g.blocked && banded;
    const dim3 grid((unsigned)std::min<int64_t>((int64_t)ntiles * s, compute_units()));
    // every tile interior and no ragged K slice: the spread-copy kernels
    const bool interior = p.bn == kBN && M % kBM == 0 && N % kBN == 0 && K % kBK == 0;
    auto spread_rb = [&](auto kt_c) {                // row-scaled B: partials, accumulate or plain fp32
      constexpr bool KT = decltype(kt_c)::value;
      if (to_ws)
        hipLaunchKernelGGL((gemm_fp8_bw_kernel<true, false, true, false, false, KT, 8, true>), grid, dim3(kThreads), 0,
                           stream, g);
      else if (accumulate)
        hipLaunchKernelGGL((gemm_fp8_bw_kernel<true, false, false, true, false, KT, 8, true>), grid, dim3(kThreads), 0,
                           stream, g);
      else
        hipLaunchKernelGGL((gemm_fp8_bw_kernel<true, false, false, false, false, KT, 8, true>), grid, dim3(kThreads), 0,
                           stream, g);
    };
    if (row_b && interior && (to_ws || !bf16_out)) {
      if (mode == 3) spread_rb(std::true_type{});
      else spread_rb(std::false_type{});
    }
    else if (mode == 3 && p.bn == 192) launch_mode<true, true, 6>(grid, stream, g, to_ws, accumulate, bf16_out);
    else if (mode == 3 && p.bn == 128) launch_mode<true, true, 4>(grid, stream, g, to_ws, accumulate, bf16_out);
    else if (mode == 3) launch_mode<true, true>(grid, stream, g, to_ws, accumulate, bf16_out);
    else if (row_b && p.bn == 192) launch_mode<true, false, 6>(grid, stream, g, to_ws, accumulate, bf16_out);
    else if (row_b && p.bn == 128) launch_mode<true, false, 4>(grid, stream, g, to_ws, accumulate, bf16_out);
    else if (row_b) launch_mode<true, false>(grid, stream, g, to_ws, accumulate, bf16_out);
    else if (!row_b && interior && bf16_out && !to_ws && !accumulate)
      hipLaunchKernelGGL((gemm_fp8_bw_kernel<false, true, false, false, false, false, 8, true>), grid, dim3(kThreads), 0,
                         stream, g);
    else launch_mode<false, false>(grid, stream, g, to_ws, accumulate, bf16_out);
    return hipGetLastError();
  };
  hipError_t err = hipSuccess;
  if (p.whole > 0 && (err = launch(0, p.whole, 1, p.nk, false)) != hipSuccess) return err;
  const bool to_ws = p.splits > 1;
  err = launch(p.whole, tiles - p.whole, p.splits, p.spl, to_ws);
  if (err != hipSuccess || !to_ws) return err;
  const float *w = (const float *)ws;
  const int nt = tiles - p.whole;
  auto reduce = [&](auto bf16_c, auto acc_c, auto vec_c) {
    constexpr bool kB = decltype(bf16_c)::value, kA = decltype(acc_c)::value, kV = decltype(vec_c)::value;
    constexpr int W = kV ? 4 : 1;
    const int64_t n = (int64_t)nt * kBM * p.bn / W;
    const int blocks = (int)std::min<int64_t>((n + 255) / 256, 8192);
    hipLaunchKernelGGL((splitk_reduce_tiles_kernel<kB, kA, kV>), dim3(blocks), dim3(256), 0, stream, w, out, M, N,
                       p.tiles_m, p.whole, nt, p.splits, p.bn, g.banded);   // the split launch's numbering
  };
  using T = std::true_type;
  using F = std::false_type;
  const bool vec = N % 4 == 0;
  if (bf16_out) vec ? reduce(T{}, F{}, T{}) : reduce(T{}, F{}, F{});
  else if (accumulate) vec ? reduce(F{}, T{}, T{}) : reduce(F{}, T{}, F{});
  else vec ? reduce(F{}, F{}, T{}) : reduce(F{}, F{}, F{});
  return hipGetLastError();
}

// ---------------------------------------------------------------- allocation-free entry

// Split-K scratch of run_gemm_noalloc: device memory owned by the library, one
// copy per GPU (each device that loads the library holds it until the process
// ends).  kScratchBytes is the largest workspace any GEMM of the layer at 16384
// tokens plans.  In host code `scratch` only names the symbol: its device
// address comes from hipGetSymbolAddress, per device.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up once per device
// (concurrent first calls store the same address).
static hipError_t scratch_address(void **ptr) {
  static std::atomic<void *> cached[64];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void *p = cached[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    cached[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t run_gemm_noalloc(int mode, const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                            void *out, bool bf16_out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  void *ws = nullptr;
  if (K > 0 && plan_gemm(mode, M, N, K).ws_bytes > 0) {
    if (plan_gemm(mode, M, N, K).ws_bytes > kScratchBytes) return hipErrorInvalidValue;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
  }
  return run_gemm(mode, a, sa, b, sb, out, bf16_out, false, M, N, K, ws, stream);
}

// Fused gate/up fprop + SwiGLU + 1x128 quantizer.  One work item per 256
// rows x 128 h columns (its 128 gate and 128 up rows of B); no split-K.  The
// results are those of the bf16 fprop followed by the SwiGLU quantizer.
hipError_t run_gemm_swiglu_quant(const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                                 uint16_t *gu, uint8_t *hq, float *hs, int64_t M, int64_t I, int64_t K,
                                 hipStream_t stream) {
  if (M == 0 || I == 0) return hipSuccess;
  if (K == 0) {
    // g = u = 0: h = 0, every tile scale 1, codes +0
    auto fill = [&](void *p, int64_t words, uint32_t v) {
      const int blocks = (int)std::min<int64_t>((words + 255) / 256, 65536);
      hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, stream, (uint32_t *)p, words, v);
    };
    if (gu) fill(gu, M * I, 0u);
    fill(hq, M * I / 4, 0u);
    fill(hs, I / kBK * M, 0x3f800000u);
    return hipGetLastError();
  }
  GemmArgs g{};
  g.a = a; g.sa = sa; g.b = b; g.sb = sb; g.out = gu; g.ws = nullptr;
  g.M = M; g.N = 2 * I; g.K = K;
  g.nk = (int)((K + kBK - 1) / kBK);
  g.tiles_m = (int)((M + kBM - 1) / kBM);
  g.tiles_n = (int)(I / kBK);
  g.bn = kBN;
  g.splits = 1; g.spl = g.nk;
  g.tile0 = 0; g.ntiles = g.tiles_m * g.tiles_n;
  g.I = I; g.hq = hq; g.hs = hs;
  const dim3 grid((unsigned)std::min<int64_t>((int64_t)g.tiles_m * g.tiles_n, compute_units()));
  hipLaunchKernelGGL((gemm_fp8_bw_kernel<false, true, false, false, true>), grid, dim3(kThreads), 0, stream, g);
  return hipGetLastError();
}

}  // namespace puro
