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
//    one of two buffers while the other is consumed: 128 KB of the 160 KB LDS;
//  - one v_mfma_f32_16x16x128_f8f6f4 covers exactly one 16x16 block of one
//    slice, so its result is the slice partial P_kb; it is promoted at once:
//    acc = fma(P, sA*sB, acc);
//  - the barrier that publishes slice kb+1 sits before the last of slice kb's
//    eight n-block steps, so the next slice's fragment and scale reads overlap
//    MFMAs instead of stalling all waves at once at the slice boundary;
//  - LDS rows are 128 B; the 16-byte chunk c of row r sits at chunk
//    c ^ ((r & 7) ^ ((r >> 3) & 1)), which makes the fragment reads (16 lanes
//    reading one chunk column of 16 consecutive rows) bank-conflict free;
//  - rows past M or N are read from clamped (valid) rows and never stored;
//    K chunks past K read a 16-byte zero page, so a ragged last slice adds 0;
//  - optional split-K writes fp32 partials to a workspace that a second
//    kernel sums in a fixed order (deterministic).
#include "device_common.h"
#include "launch.h"

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
};

__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

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

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Writes the 256x256 fp32 accumulator tile (distributed over the 8 waves in
// the MFMA output layout) to out[M][N] as T (fp32, or bf16 rounded to nearest
// even), staging rows through LDS so that global stores are 16-byte chunks.
// `lds` must hold 128 KB and be free; the call begins with a barrier.
template <typename T>
__device__ __forceinline__ void store_tile(const v4f (&acc)[4][8], T *out, const GemmArgs &g, int64_t m0,
                                           int64_t n0, uint8_t *lds, int wm, int wn, int q, int fr) {
  constexpr int kRowsPerPass = sizeof(T) == 2 ? 128 : 64;     // a multiple of a wave's 64 rows
  constexpr int kStride = kBN * (int)sizeof(T) + 16;          // padded LDS row (bytes)
  static_assert(kRowsPerPass * kStride <= 2 * 2 * kSliceBytes, "staging must fit the operand buffers");
  constexpr int kChunk = 16 / (int)sizeof(T);                  // elements per 16-byte chunk
  constexpr int kChunksPerRow = kBN / kChunk;
  const int t = threadIdx.x;
  const bool vec_ok = (g.N % kChunk) == 0;                      // rows of out are 16-byte aligned
#pragma unroll
  for (int pass = 0; pass < kBM / kRowsPerPass; ++pass) {
    __syncthreads();
    const int r_lo = pass * kRowsPerPass;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int rb = wm * 64 + mb * 16 + 4 * q;
      if (rb < r_lo || rb >= r_lo + kRowsPerPass) continue;    // uniform per wave: a wave's 64 rows lie in one pass
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int c = wn * 128 + nb * 16 + fr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[mb][nb][e];
          T *dst = reinterpret_cast<T *>(lds + (rb + e - r_lo) * kStride + c * (int)sizeof(T));
          if constexpr (sizeof(T) == 2) *dst = (T)f32_to_bf16_rne(v);
          else *dst = v;
        }
      }
    }
    __syncthreads();
    constexpr int kChunksPerPass = kRowsPerPass * kChunksPerRow;
#pragma unroll
    for (int i = 0; i < kChunksPerPass / kThreads; ++i) {
      const int chunk = t + i * kThreads;
      const int r = chunk / kChunksPerRow;
      const int cc = chunk % kChunksPerRow;
      const int64_t m = m0 + r_lo + r;
      const int64_t n = n0 + cc * kChunk;
      if (m >= g.M || n >= g.N) continue;
      const u32x4 d = *reinterpret_cast<const u32x4 *>(lds + r * kStride + cc * 16);
      T *dst = out + m * g.N + n;
      if (vec_ok && n + kChunk <= g.N) {
        *reinterpret_cast<u32x4 *>(dst) = d;
      } else {
        const T *src = reinterpret_cast<const T *>(&d);
        for (int k = 0; k < kChunk && n + k < g.N; ++k) dst[k] = src[k];
      }
    }
  }
}

template <bool kRowScaledB, bool kBf16Out, bool kToWs>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_bw_kernel(GemmArgs g) {
  // [buf][A/B][256 rows x 128 B] operand slices; [buf][sA/sB][256] scales
  __shared__ __align__(1024) uint8_t smem[2][2][kSliceBytes];
  __shared__ __align__(16) float sscale[2][2][kBM];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1;

  const int total_tiles = g.tiles_m * g.tiles_n;
  const int bid = blockIdx.x;
  const int split = bid / total_tiles;
  const int tile = bid - split * total_tiles;
  const int tm = tile % g.tiles_m;       // consecutive workgroups walk down M: they share B
  const int tn = tile / g.tiles_m;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
  const int kb_begin = split * g.spl;
  const int kb_end = min(g.nk, kb_begin + g.spl);
  const int K = (int)g.K;

  // ---- global -> LDS copy plan.  Wave w fills LDS row groups grp = 4w + j
  // (j = 0..3) of 8 rows; lane -> row grp*8 + (lane/8), physical chunk lane%8,
  // whose logical chunk is (lane%8) ^ (lane/8) ^ (j&1).  Rows past M / N are
  // redirected to the tile's first row (finite codes whose products are
  // never stored).
  const int rig = lane >> 3;
  const int kc0 = ((lane & 7) ^ rig) * 16;     // even j
  const int kc1 = kc0 ^ 16;                     // odd j
  const uint8_t *a_tile = g.a + m0 * g.K;
  const uint8_t *b_tile = g.b + n0 * g.K;
  const int rows_a = (int)min<int64_t>(g.M - m0, kBM);   // valid rows in this tile
  const int rows_b = (int)min<int64_t>(g.N - n0, kBN);
  const uint32_t lds0 = lds_addr(&smem[0][0][0]);
  const uint32_t lds_s0 = lds_addr(&sscale[0][0][0]);
  const bool ktail = (K & (kBK - 1)) != 0;
  const int64_t nb0 = n0 / kBK;                               // first 128-column block of B in this tile
  const int nb_last = (int)((g.N - 1) / kBK - nb0);           // last valid block, relative to nb0
  // Interior tiles: lane offsets (row group j, row rig, logical chunk) are
  // shared by A and B; the wave's first row group and the K slice go into the
  // scalar bases.  Scales travel as one 16-byte-per-lane copy when their rows
  // are 16-byte aligned.
  const uint32_t voff0 = (uint32_t)(rig * K + kc0);
  const uint32_t voff1 = (uint32_t)((8 + rig) * K + kc1);
  const uint32_t voff2 = (uint32_t)((16 + rig) * K + kc0);
  const uint32_t voff3 = (uint32_t)((24 + rig) * K + kc1);
  const bool full_rows = rows_a == kBM && rows_b == kBN;
  const bool scale_x4 = full_rows && (g.M & 3) == 0 && (!kRowScaledB || (g.N & 3) == 0);
  const uint8_t *a_wave = a_tile + (int64_t)(w * 32) * g.K;
  const uint8_t *b_wave = b_tile + (int64_t)(w * 32) * g.K;

  // Per-lane values that only edge tiles, the ragged last slice and the scale
  // copies need are recomputed from an opaque lane id at each call, so that
  // they occupy no VGPRs across the K loop.
  auto issue_scales = [&](int kb, int buf) {
    // wave 0 copies sA rows m0..m0+255; wave 1 copies sB columns n0.. (row-scaled
    // B) or the tile's two block scales (block-scaled B)
    if (w > 1) return;
    const uint32_t ls = lds_s0 + buf * 2 * kBM * 4;
    int ln = __lane_id();
    asm volatile("" : "+v"(ln));
    if (scale_x4 && (w == 0 || kRowScaledB)) {
      // lane l brings the 4 scales of rows (or columns) 4l .. 4l+3
      const float *src = w == 0 ? g.sa + (int64_t)kb * g.M + m0 : g.sb + (int64_t)kb * g.N + n0;
      dma16_s(src, (uint32_t)ln * 16, ls + (w == 0 ? 0 : kBM * 4));
      return;
    }
    if (w == 0) {
      const float *src = g.sa + (int64_t)kb * g.M + m0;
#pragma unroll
      for (int j = 0; j < 4; ++j) dma4_s(src, (uint32_t)min(ln + 64 * j, rows_a - 1) * 4, ls + 256 * j);
    } else if constexpr (kRowScaledB) {
      const float *src = g.sb + (int64_t)kb * g.N + n0;
#pragma unroll
      for (int j = 0; j < 4; ++j) dma4_s(src, (uint32_t)min(ln + 64 * j, rows_b - 1) * 4, ls + kBM * 4 + 256 * j);
    } else {
      // lane l brings sb[n-block nb0 + l][kb] (clamped); lanes 0 and 1 cover
      // the tile's two 128-column blocks
      const float *src = g.sb + nb0 * g.nk + kb;
      dma4_s(src, (uint32_t)min(ln, nb_last) * (uint32_t)g.nk * 4, ls + kBM * 4);
    }
  };

  auto issue_slice = [&](int kb, int buf) {
    const int kofs = kb * kBK;
    const uint32_t la = lds0 + buf * 2 * kSliceBytes;
    const uint32_t lb = la + kSliceBytes;
    if (full_rows && !(ktail && kb == g.nk - 1)) {
      dma_slice8(a_wave + kofs, b_wave + kofs, voff0, voff1, voff2, voff3, la + w * 4096);
    } else {
      // edge tiles and the ragged last slice: chunks at or past K read a zero page
      int ln = __lane_id();
      asm volatile("" : "+v"(ln));
      const int rg = ln >> 3;
      const int k0 = ((ln & 7) ^ rg) * 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int grp = w * 4 + j;
        const int r = grp * 8 + rg;
        const int kc = (j & 1) ? (k0 ^ 16) : k0;
        const bool kin = kofs + kc < K;
        const uint8_t *pa = kin ? a_tile + kofs + (r < rows_a ? (int64_t)r * K : 0) + kc : g_zero16;
        const uint8_t *pb = kin ? b_tile + kofs + (r < rows_b ? (int64_t)r * K : 0) + kc : g_zero16;
        dma16_v(pa, la + grp * 1024);
        dma16_v(pb, lb + grp * 1024);
      }
    }
    issue_scales(kb, buf);
  };

  // ---- fragment read plan: lane reads row (lane % 16) of each 16-row block,
  // logical chunks 2q and 2q+1 (q = lane / 16).
  const int fr = lane & 15;
  const int q = lane >> 4;
  const int p0 = (2 * q) ^ lds_swz(fr);
  const int p1 = p0 ^ 1;

  v4f acc[4][8];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = (v4f){0.f, 0.f, 0.f, 0.f};

  auto load_frag = [&](const uint8_t *base, int r) -> v8i {
    const v4i lo = *reinterpret_cast<const v4i *>(base + r * kBK + p0 * 16);
    const v4i hi = *reinterpret_cast<const v4i *>(base + r * kBK + p1 * 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // ---- K loop.  Slice kb is computed from buffer (kb - kb_begin) & 1 while
  // slice kb+1 is copied into the other one.  The barrier that publishes slice
  // kb+1 sits before the last n-block step of slice kb, so that the reads of
  // slice kb+1's A fragments, first B fragment and scales overlap the MFMAs of
  // that step instead of stalling every wave at the start of the slice.
  v8i af[4];                 // A fragments of the wave's 4 m-blocks
  v8i bf[2];                 // B fragments of n-blocks nb (in use) and nb+1 (landing)
  v4f sa[4];                 // row scales sA of the lane's 4 rows in each m-block
  float sbn0 = 1.0f;         // row-scaled B: column scale of the coming slice's n-block 0
  float sbk = 1.0f;          // block-scaled B: the coming slice's scale of the wave's 128 columns
  auto load_scales = [&](int buf) {
    const float *lsa = sscale[buf][0];
    const float *lsb = sscale[buf][1];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) sa[mb] = *reinterpret_cast<const v4f *>(&lsa[wm * 64 + mb * 16 + 4 * q]);
    if constexpr (kRowScaledB) sbn0 = lsb[wn * 128 + fr];
    else sbk = lsb[wn];
  };

  if (kb_begin < kb_end) {
    issue_slice(kb_begin, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    bf[0] = load_frag(smem[0][1], wn * 128 + fr);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) af[mb] = load_frag(smem[0][0], wm * 64 + mb * 16 + fr);
    load_scales(0);
  }

  // One slice.  Step nb issues the 4 MFMAs of n-block nb; the partial of
  // n-block nb-1 is promoted into the accumulators from P[mb] right before
  // MFMA (nb, mb) overwrites it, and the B fragment of n-block nb+1 is read
  // one step ahead.  kNext: a slice follows in this work item.
  auto slice = [&](int kb, auto next_c) {
    constexpr bool kNext = decltype(next_c)::value;
    const int buf = (kb - kb_begin) & 1;
    const uint8_t *Bs = smem[buf][1];
    const float *lsb = sscale[buf][1];
    v4f P[4];
    float sbv[8];              // row-scaled B: column scale of each n-block
    sbv[0] = sbn0;
    v4f sc[4];                 // block-scaled B: promotion factors sA * sB
    // the buffer of slice kb-1 was released by the barrier inside slice kb-1
    if constexpr (kNext) issue_slice(kb + 1, buf ^ 1);
    auto promote = [&](int pb, int mb) {
      if constexpr (kRowScaledB) {
        const v4f ps = P[mb] * sbv[pb];                          // column scale first, in place
        acc[mb][pb] = __builtin_elementwise_fma(ps, sa[mb], acc[mb][pb]);
      } else {
        acc[mb][pb] = __builtin_elementwise_fma(P[mb], sc[mb], acc[mb][pb]);
      }
    };
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      __builtin_amdgcn_sched_barrier(0);
      if (nb == 7) {
        // Every wave holds its n-block 7 fragment (lgkmcnt) and has landed its
        // share of slice kb+1 (vmcnt): past the barrier slice kb+1 is readable
        // and nothing reads slice kb's buffer any more.
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kRowScaledB && nb + 1 < 8) sbv[nb + 1] = lsb[wn * 128 + (nb + 1) * 16 + fr];
      if (nb + 1 < 8) bf[(nb + 1) & 1] = load_frag(Bs, wn * 128 + (nb + 1) * 16 + fr);
      if (nb == 7 && kNext) bf[0] = load_frag(smem[buf ^ 1][1], wn * 128 + fr);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (nb > 0) promote(nb - 1, mb);
        P[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af[mb], bf[nb & 1], (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        if (nb == 7 && kNext) af[mb] = load_frag(smem[buf ^ 1][0], wm * 64 + mb * 16 + fr);
        if (nb == 0 && !kRowScaledB) sc[mb] = sa[mb] * sbk;
      }
      // issue order within the step: LDS reads first (a whole step to land),
      // then VALU groups between the MFMAs
      constexpr int kV = kRowScaledB ? 8 : 4;
      constexpr int kS = kRowScaledB ? 1 : 0;
      if (nb == 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2 + kS, 0);                // LDS reads
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
          if (!kRowScaledB) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
        }
      } else if (nb < 7) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2 + kS, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      } else {
        if (kNext) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (kNext) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) promote(7, mb);
    if constexpr (kNext) load_scales(buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
  };

  {
    int kb = kb_begin;
    for (; kb + 1 < kb_end; ++kb) slice(kb, std::true_type{});
    if (kb < kb_end) slice(kb, std::false_type{});
  }

  // ---- epilogue.  Lane holds rows wm*64 + mb*16 + 4q + e, columns
  // wn*128 + nb*16 + fr of the tile.  The tile is staged through the (now
  // idle) LDS in row-major order and leaves as 16-byte row chunks: bf16 in two
  // passes of 128 rows, fp32 in four passes of 64 rows.
  if constexpr (kToWs) {
    store_tile<float>(acc, g.ws + (int64_t)split * g.M * g.N, g, m0, n0, &smem[0][0][0], wm, wn, q, fr);
  } else if constexpr (kBf16Out) {
    store_tile<uint16_t>(acc, reinterpret_cast<uint16_t *>(g.out), g, m0, n0, &smem[0][0][0], wm, wn, q, fr);
  } else {
    store_tile<float>(acc, reinterpret_cast<float *>(g.out), g, m0, n0, &smem[0][0][0], wm, wn, q, fr);
  }
}

// Sum of the split-K partials in increasing split order.
template <bool kBf16Out>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *ws, void *out, int64_t MN, int splits) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += stride) {
    float v = ws[i];
    for (int s = 1; s < splits; ++s) v += ws[(int64_t)s * MN + i];
    if constexpr (kBf16Out)
      reinterpret_cast<uint16_t *>(out)[i] = (uint16_t)f32_to_bf16_rne(v);
    else
      reinterpret_cast<float *>(out)[i] = v;
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

// ---------------------------------------------------------------- planning

GemmPlan plan_gemm(int mode, int64_t M, int64_t N, int64_t K) {
  GemmPlan p{};
  p.nk = (int)((K + kBK - 1) / kBK);
  p.tiles_m = (int)((M + kBM - 1) / kBM);
  p.tiles_n = (int)((N + kBN - 1) / kBN);
  p.splits = 1;
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  // Split the K loop when the output tiles fill the 256 compute units poorly
  // (a last round of tiles that leaves units idle, or fewer tiles than units).
  // Estimated time with s splits: rounds of 256 work items, each of ceil(nk/s)
  // slices plus about 2 slices of fixed cost (first copy, epilogue) at about
  // 1.9 us per slice, plus the workspace traffic (every split writes an fp32
  // partial of the output and the reduction reads it back) at about 4 TB/s.
  // More splits must win by 3%; at least 4 slices per split.
  if (tiles > 0 && p.nk > 0) {
    double best = 0.0;
    for (int s = 1; s <= 8; ++s) {
      const int spl = (p.nk + s - 1) / s;
      if (s > 1 && (spl < 4 || (p.nk + spl - 1) / spl != s)) continue;
      const double rounds = (double)((tiles * s + 255) / 256);
      const double t = rounds * (spl + 2) * 1.9e-6 +
                       (s > 1 ? 2.0 * s * (double)M * (double)N * 4.0 / 4.0e12 : 0.0);
      if (s == 1 || t < best * 0.97) {
        best = t;
        p.splits = s;
      }
    }
  }
  p.spl = (p.nk + p.splits - 1) / p.splits;
  if (p.spl > 0) p.splits = (p.nk + p.spl - 1) / p.spl;
  p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
  (void)mode;
  return p;
}

hipError_t run_gemm(int mode, const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                    void *out, bool bf16_out, int64_t M, int64_t N, int64_t K, void *ws,
                    hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t MN = M * N;
  if (K == 0) {
    const int blocks = (int)std::min<int64_t>((MN + 255) / 256, 65536);
    if (bf16_out) hipLaunchKernelGGL(fill_zero_kernel<true>, dim3(blocks), dim3(256), 0, stream, out, MN);
    else hipLaunchKernelGGL(fill_zero_kernel<false>, dim3(blocks), dim3(256), 0, stream, out, MN);
    return hipGetLastError();
  }
  const GemmPlan p = plan_gemm(mode, M, N, K);
  GemmArgs g{};
  g.a = a; g.sa = sa; g.b = b; g.sb = sb; g.out = out; g.ws = (float *)ws;
  g.M = M; g.N = N; g.K = K;
  g.nk = p.nk; g.tiles_m = p.tiles_m; g.tiles_n = p.tiles_n;
  g.splits = p.splits; g.spl = p.spl;
  const dim3 grid((unsigned)((int64_t)p.tiles_m * p.tiles_n * p.splits));
  const bool row_b = mode == 2;
  const bool to_ws = p.splits > 1;
#define PURO_LAUNCH(RB, BF, WS) \
  hipLaunchKernelGGL((gemm_fp8_bw_kernel<RB, BF, WS>), grid, dim3(kThreads), 0, stream, g)
  if (to_ws) {
    if (row_b) PURO_LAUNCH(true, false, true); else PURO_LAUNCH(false, false, true);
  } else if (bf16_out) {
    if (row_b) PURO_LAUNCH(true, true, false); else PURO_LAUNCH(false, true, false);
  } else {
    if (row_b) PURO_LAUNCH(true, false, false); else PURO_LAUNCH(false, false, false);
  }
#undef PURO_LAUNCH
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !to_ws) return err;
  const int blocks = (int)std::min<int64_t>((MN + 255) / 256, 8192);
  if (bf16_out)
    hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3(blocks), dim3(256), 0, stream, (const float *)ws, out, MN, p.splits);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3(blocks), dim3(256), 0, stream, (const float *)ws, out, MN, p.splits);
  return hipGetLastError();
}

}  // namespace puro
