// Blockwise FP8 quantizers for gfx950: 1x128 activation tiles, 128x128
// weight blocks, and the transposed 128x1 / 128x128 variants for the backward
// operands (optionally writing the row-wise codes in the same pass).
//
// The pages (en.roboind.com article on Puro-2B, section "FP8 takes advantage
// of the RTX 5090's low precision efficiency") name fine-grained block
// quantization after DeepSeek-V3 for the main linear layers; the tile shapes
// and the scale/code rule are this library's reading (see device_common.h).
//
// Design.  These kernels are bound by HBM bandwidth: each element is read
// once as bf16 (2 B) and written once or twice as a code (1 B), plus one fp32
// scale per tile.  One workgroup of 256 threads owns one 128x128 block of the
// input.  Thread t owns 8 consecutive rows (rg = t/16) x 8 consecutive columns
// (cc = t%16): every load is 16 B and the 16 lanes of a DPP row read 256
// contiguous bytes of one input row, so reads are coalesced.  All eight loads
// are issued before any arithmetic.  Row maxima reduce across the 16 lanes of
// a DPP row; column and block maxima go through LDS.  Scales and their
// reciprocals are computed once per tile by one thread and shared through
// LDS.  Transposed codes are assembled in LDS (8-byte slots XOR-swizzled by
// the column group, so both the 8-byte writes and the 16-byte reads are free
// of bank conflicts) and leave as 128-byte row segments.  The token-major form
// of the 128x1 codes skips the transpose: they leave in the input's layout,
// 8 bytes per row of the thread's block, like the row-wise codes.
#include "device_common.h"
#include "launch.h"

namespace puro {

struct QuantArgs {
  const uint16_t *x;
  int64_t R, C;
  int64_t ld;              // row stride of x in elements (C, or 2C for the gate/up input)
  int64_t ni, nj;          // ceil(R/128), ceil(C/128)
  uint8_t *q;              // row-major codes [R][C] (or null)
  float *s;                // scales of the row-major codes
  uint8_t *qt;             // transposed codes [C][R] (or null)
  float *st;               // scales of the transposed codes
  uint16_t *h;             // SwiGLU output [R][C] in bf16 (or null)
  int64_t band;            // launch order: workgroups walk down bands of `band` block rows (1: row-major)
};

// Transposed codes of one 128x128 block, staged in LDS, to global memory.
// LDS row c (a column of the block, an output row) holds 16 slots of 8 codes
// (8 input rows each); logical slot g is stored at physical slot g ^ (c / 8),
// so that the 8-byte slot writes of 16 consecutive column groups and the
// 16-byte chunk reads below are both free of bank conflicts.  Each of the 256
// threads writes four 16-byte chunks; a run of 8 threads covers one 128-byte
// output row segment.  kStream: non-temporal stores (the requantizer);
// otherwise plain ones (see the row codes' stores in quant_block).
__device__ __forceinline__ void put_transposed_slot(uint8_t *lds_t, int lc, int g, u32x2 codes) {
  *reinterpret_cast<u32x2 *>(&lds_t[lc * kTile + ((g ^ (lc >> 3)) * 8)]) = codes;
}

template <bool kStream>
__device__ __forceinline__ void flush_transposed(const uint8_t *lds_t, uint8_t *qt, int64_t R, int64_t C,
                                                 int64_t bi, int64_t bj, int t) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int chunk = t + 256 * u;
    const int lc = chunk >> 3;          // block column = output row
    const int p = chunk & 7;            // physical 16-byte chunk in the LDS row
    const int xs = (lc >> 3) & 15;      // swizzle of this LDS row
    u32x4 d = *reinterpret_cast<const u32x4 *>(&lds_t[lc * kTile + p * 16]);
    if (xs & 1) d = (u32x4){d.z, d.w, d.x, d.y};
    const int l = p ^ (xs >> 1);        // logical 16-byte chunk = rows 16l .. 16l+15
    const int64_t orow = bj * kTile + lc;
    const int64_t ocol = bi * kTile + l * 16;
    if (orow < C && ocol < R) {
      if constexpr (kStream) __builtin_nontemporal_store(d, reinterpret_cast<u32x4 *>(qt + orow * R + ocol));
      else *reinterpret_cast<u32x4 *>(qt + orow * R + ocol) = d;
    }
  }
}

// kRow:    1x128 scales (per row of the block)       -> row-major output
// kCol:    128x1 scales (per column of the block)    -> transposed output
// kBlock:  one 128x128 scale                         -> row-major and/or transposed output
// kSwiGLU: the block's values are h = SwiGLU(gate, up) of a [R][2C] gate/up
//          input (gate = first C columns), computed in registers
// kTRow: the 128x1 codes (kCol) leave in the input's own [R][C] layout
// instead of transposed, for a wgrad that reads its operands token-major.
// The work of one workgroup on block `bid` (row-major block index) of a.
template <bool kRow, bool kCol, bool kBlock, bool kWriteRow, bool kWriteT, bool kSwiGLU, bool kTRow>
__device__ __forceinline__ void quant_block(const QuantArgs &a, int64_t bid) {
  static_assert(!kTRow || (kCol && kWriteT), "the untransposed form is that of the 128x1 codes");
  __shared__ float lds_part[16 * kTile];                 // column partial maxima [rg][c]
  __shared__ float lds_rowamax[kTile];
  __shared__ __align__(16) float lds_rows[kTile], lds_rowr[kTile];
  __shared__ __align__(16) float lds_cols[kTile], lds_colr[kTile];
  __shared__ float lds_wmax[4];
  __shared__ __align__(16) uint8_t lds_t[kWriteT && !kTRow ? kTile * kTile : 16];

  const int t = threadIdx.x;
  const int cc = t & 15, rg = t >> 4;
  const int64_t bi = bid / a.nj, bj = bid - bi * a.nj;
  const int64_t r0 = bi * kTile + rg * 8;
  const int64_t c0 = bj * kTile + cc * 8;
  const bool cvalid = c0 < a.C;

  // ---- load 8 rows x 8 columns (16 B per row), all in flight at once
  u32x4 raw[8];
  if constexpr (kSwiGLU) {
    // gate and up words of the same 8 x 8 block, then h in registers
    u32x4 gw[8], uw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t r = r0 + k;
      if (cvalid && r < a.R) {
        gw[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.x + r * a.ld + c0));
        uw[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.x + r * a.ld + a.C + c0));
      } else {
        gw[k] = (u32x4){0u, 0u, 0u, 0u};
        uw[k] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
    uint64_t slow = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bool s0, s1;
        const uint32_t h0 = swiglu_fast(bf16lo(gw[k][j]), bf16lo(uw[k][j]), s0);
        const uint32_t h1 = swiglu_fast(bf16hi(gw[k][j]), bf16hi(uw[k][j]), s1);
        raw[k][j] = (h0 & 0xffffu) | (h1 << 16);
        slow |= ((uint64_t)s0 << (k * 8 + 2 * j)) | ((uint64_t)s1 << (k * 8 + 2 * j + 1));
      }
    }
    // rare elements near a bf16 rounding midpoint, or with |g| > 64: fp64,
    // one element at a time (reloaded; the lines are still cached)
    while (slow) {
      const int i = __builtin_ctzll(slow);
      slow &= slow - 1;
      const int k = i >> 3, c = i & 7;
      const int64_t off = (r0 + k) * a.ld + c0 + c;
      const uint32_t hb = swiglu_f64(bf16lo(a.x[off]), bf16lo(a.x[off + a.C]));
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = raw[kk][j];
          const uint32_t merged = (c & 1) ? ((w & 0xffffu) | (hb << 16)) : ((w & 0xffff0000u) | hb);
          raw[kk][j] = (kk == k && j == (c >> 1)) ? merged : w;
        }
    }
    if (a.h != nullptr) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t r = r0 + k;
        if (cvalid && r < a.R)
          __builtin_nontemporal_store(raw[k], reinterpret_cast<u32x4 *>(a.h + r * a.C + c0));
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t r = r0 + k;
      if (cvalid && r < a.R)
        raw[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.x + r * a.ld + c0));
      else
        raw[k] = (u32x4){0u, 0u, 0u, 0u};
    }
  }
  // Hide the packed words from the optimizer between phases so that unpacked
  // values are recomputed in each phase instead of staying live across it.
  auto refresh = [&]() {
#pragma unroll
    for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(raw[k]));
  };

  // element (k, c) of the thread's 8x8 block, unpacked where it is used (the
  // packed words are all that stays live, which keeps occupancy up)
  auto el = [&](int k, int c) -> float {
    const uint32_t wd = raw[k][c >> 1];
    return (c & 1) ? bf16hi(wd) : bf16lo(wd);
  };

  // ---- maxima, on the packed magnitude bits (see bf16_mags)
  uint32_t rbits[8];                 // row maxima of this thread's 8 columns
  u16x2 cbits[4];                    // column maxima over this thread's 8 rows (column pairs)
#pragma unroll
  for (int j = 0; j < 4; ++j) cbits[j] = (u16x2){0, 0};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const u16x2 m0 = bf16_mags(raw[k].x), m1 = bf16_mags(raw[k].y);
    const u16x2 m2 = bf16_mags(raw[k].z), m3 = bf16_mags(raw[k].w);
    rbits[k] = hmax16(max16x2(max16x2(m0, m1), max16x2(m2, m3)));
    if constexpr (kCol) {
      cbits[0] = max16x2(cbits[0], m0);
      cbits[1] = max16x2(cbits[1], m1);
      cbits[2] = max16x2(cbits[2], m2);
      cbits[3] = max16x2(cbits[3], m3);
    }
  }

  TileQ tb;                      // block tile (kBlock)
  if constexpr (kBlock) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = max(m, rbits[k]);
    m = wave_max_u32(m);
    if ((t & 63) == 0) lds_wmax[t >> 6] = mag_to_float(m);
  }
  if constexpr (kRow) {
#pragma unroll
    for (int k = 0; k < 8; ++k) rbits[k] = row16_max_u32(rbits[k]);
    if (cc == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) lds_rowamax[rg * 8 + k] = mag_to_float(rbits[k]);
    }
  }
  if constexpr (kCol) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lds_part[rg * kTile + cc * 8 + 2 * j] = mag_to_float(cbits[j].x);
      lds_part[rg * kTile + cc * 8 + 2 * j + 1] = mag_to_float(cbits[j].y);
    }
  }
  __syncthreads();

  // ---- scales: one thread per row (threads 0..127) / per column (128..255)
  if constexpr (kRow) {
    if (t < kTile) {
      const TileQ q = make_tileq(lds_rowamax[t]);
      lds_rows[t] = q.s;
      lds_rowr[t] = q.r;
      const int64_t r = bi * kTile + t;
      if (r < a.R) a.s[bj * a.R + r] = q.s;
    }
  }
  if constexpr (kCol) {
    if (t >= kTile) {
      const int c = t - kTile;
      float m = 0.0f;
#pragma unroll
      for (int g = 0; g < 16; ++g) m = fmaxf(m, lds_part[g * kTile + c]);
      const TileQ q = make_tileq(m);
      lds_cols[c] = q.s;
      lds_colr[c] = q.r;
      const int64_t cg = bj * kTile + c;
      if (cg < a.C) a.st[bi * a.C + cg] = q.s;
    }
  }
  if constexpr (kBlock) {
    const float m = fmaxf(fmaxf(lds_wmax[0], lds_wmax[1]), fmaxf(lds_wmax[2], lds_wmax[3]));
    tb = make_tileq(m);
    if (t == 0) {
      if constexpr (kWriteRow) a.s[bi * a.nj + bj] = tb.s;
      if constexpr (kWriteT) a.st[bj * a.ni + bi] = tb.s;
    }
  }
  if constexpr (kRow || kCol) __syncthreads();

  // ---- row-major codes
  if constexpr (kWriteRow) {
    float rs[8], rr[8];
    if constexpr (kRow) {
      const f32x4 s0 = *reinterpret_cast<const f32x4 *>(&lds_rows[rg * 8]);
      const f32x4 s1 = *reinterpret_cast<const f32x4 *>(&lds_rows[rg * 8 + 4]);
      const f32x4 q0 = *reinterpret_cast<const f32x4 *>(&lds_rowr[rg * 8]);
      const f32x4 q1 = *reinterpret_cast<const f32x4 *>(&lds_rowr[rg * 8 + 4]);
      rs[0] = s0.x; rs[1] = s0.y; rs[2] = s0.z; rs[3] = s0.w;
      rs[4] = s1.x; rs[5] = s1.y; rs[6] = s1.z; rs[7] = s1.w;
      rr[0] = q0.x; rr[1] = q0.y; rr[2] = q0.z; rr[3] = q0.w;
      rr[4] = q1.x; rr[5] = q1.y; rr[6] = q1.z; rr[7] = q1.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) { rs[k] = tb.s; rr[k] = tb.r; }
    }
    bool fast = true;
#pragma unroll
    for (int k = 0; k < 8; ++k) fast &= rs[k] >= kFastDivMinScale;
    refresh();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float v[8];
      if (fast) {
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = quot_fast(el(k, c), rs[k], rr[k]);
      } else {
        const bool fk = rs[k] >= kFastDivMinScale;
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = fk ? quot_fast(el(k, c), rs[k], rr[k]) : el(k, c) / rs[k];
      }
      u32x2 o;
      o.x = pack4_e4m3(v[0], v[1], v[2], v[3]);
      o.y = pack4_e4m3(v[4], v[5], v[6], v[7]);
      const int64_t r = r0 + k;
      // plain (cached) stores for every code output: the codes stay in L2
      // and leave it while the GEMM that reads them computes.  Non-temporal
      // stores made the layer's quantizers 8% slower for a 0.7% faster GEMM
      // sum, and plain input loads made them slower too.
      if (cvalid && r < a.R) *reinterpret_cast<u32x2 *>(a.q + r * a.C + c0) = o;
    }
  }

  // ---- transposed codes
  if constexpr (kWriteT) {
    float cs[8], cr[8];
    if constexpr (kCol) {
      const f32x4 s0 = *reinterpret_cast<const f32x4 *>(&lds_cols[cc * 8]);
      const f32x4 s1 = *reinterpret_cast<const f32x4 *>(&lds_cols[cc * 8 + 4]);
      const f32x4 q0 = *reinterpret_cast<const f32x4 *>(&lds_colr[cc * 8]);
      const f32x4 q1 = *reinterpret_cast<const f32x4 *>(&lds_colr[cc * 8 + 4]);
      cs[0] = s0.x; cs[1] = s0.y; cs[2] = s0.z; cs[3] = s0.w;
      cs[4] = s1.x; cs[5] = s1.y; cs[6] = s1.z; cs[7] = s1.w;
      cr[0] = q0.x; cr[1] = q0.y; cr[2] = q0.z; cr[3] = q0.w;
      cr[4] = q1.x; cr[5] = q1.y; cr[6] = q1.z; cr[7] = q1.w;
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) { cs[c] = tb.s; cr[c] = tb.r; }
    }
    bool fast = true;
#pragma unroll
    for (int c = 0; c < 8; ++c) fast &= cs[c] >= kFastDivMinScale;
    refresh();
    if constexpr (kTRow) {
      // row k of the thread's 8x8 block with its 8 column scales: one 8-byte
      // store per row, like the row-wise codes
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float v[8];
        if (fast) {
#pragma unroll
          for (int c = 0; c < 8; ++c) v[c] = quot_fast(el(k, c), cs[c], cr[c]);
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) v[c] = cs[c] >= kFastDivMinScale ? quot_fast(el(k, c), cs[c], cr[c]) : el(k, c) / cs[c];
        }
        u32x2 o;
        o.x = pack4_e4m3(v[0], v[1], v[2], v[3]);
        o.y = pack4_e4m3(v[4], v[5], v[6], v[7]);
        const int64_t r = r0 + k;
        if (cvalid && r < a.R) *reinterpret_cast<u32x2 *>(a.qt + r * a.C + c0) = o;
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v[8];
      if (fast) {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = quot_fast(el(k, c), cs[c], cr[c]);
      } else {
        const bool fc = cs[c] >= kFastDivMinScale;
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = fc ? quot_fast(el(k, c), cs[c], cr[c]) : el(k, c) / cs[c];
      }
      u32x2 col;
      col.x = pack4_e4m3(v[0], v[1], v[2], v[3]);
      col.y = pack4_e4m3(v[4], v[5], v[6], v[7]);
      put_transposed_slot(lds_t, cc * 8 + c, rg, col);
    }
    __syncthreads();
    flush_transposed<false>(lds_t, a.qt, a.R, a.C, bi, bj, t);
  }
}

// Workgroup b takes the blocks of a band of `band` block rows in column order
// (block row fastest), the bands one after another; the last band may be
// shorter.
template <bool kRow, bool kCol, bool kBlock, bool kWriteRow, bool kWriteT, bool kSwiGLU = false, bool kTRow = false>
__global__ __launch_bounds__(256) void quant_block_kernel(QuantArgs a) {
  int64_t bid = blockIdx.x;
  if (a.band > 1) {
    const int64_t per = a.band * a.nj;
    const int64_t band = bid / per, local = bid - band * per;
    const int64_t h = min(a.band, a.ni - band * a.band);
    bid = (band * a.band + local % h) * a.nj + local / h;
  }
  quant_block<kRow, kCol, kBlock, kWriteRow, kWriteT, kSwiGLU, kTRow>(a, bid);
}

// Several weights quantized by one launch (128x128 blocks, row-major and/or
// transposed outputs): a small weight alone fills only part of the chip for a
// few microseconds, while the layer's weights together make thousands of
// workgroups.  Workgroup b works on tensor i, block b - first[i], where
// first[i] <= b < first[i + 1].
constexpr int kMaxGroup = 8;
struct QuantGroupArgs {
  QuantArgs t[kMaxGroup];
  int64_t first[kMaxGroup + 1];
  int count;
};

template <bool kWriteRow, bool kWriteT>
__global__ __launch_bounds__(256) void quant_weights_kernel(QuantGroupArgs g) {
  const int64_t b = blockIdx.x;
  int i = 0;
#pragma unroll
  for (int k = 1; k < kMaxGroup; ++k) i += (k < g.count && b >= g.first[k]) ? 1 : 0;
  quant_block<false, false, true, kWriteRow, kWriteT, false, false>(g.t[i], b - g.first[i]);
}

// Requantization of saved 1x128 activation codes into transposed 128x1 tiles:
// each code is dequantized to fp32 with its row tile's scale (one IEEE
// multiply, so the exact product rounded once), then quantized again with
// the 128x1 rule: per column of the block, st = amax/448 and
// qt = e4m3(fp32(d / st)).
//
// Division.  d is an arbitrary fp32 value here, not a bf16 one, so the
// one-step reciprocal of the bf16 kernels is not used.  For a column scale b
// in [2^-60, 2^60] the quotient is formed from a two-word reciprocal
// rh + rl = 1/b (rh the rounded reciprocal, rl the rounded residual times
// rh): y = fma(d, rh, d * rl) is then a faithful quotient, and one residual
// correction z = fma(fma(-y, b, d), rh, y) (Markstein) rounds it correctly.
// No step underflows while |d / b| >= 2^-12; below that both z and the true
// quotient lie under 2^-10 and take the zero code of d's sign.  A thread with
// a column scale outside that range uses the IEEE division.  Five operations per
// element instead of the IEEE division's dozen, which left the kernel bound
// by the vector ALU rather than by memory.
//
// One workgroup of 256 threads owns one 128x128 block of the code matrix.
// Within a block all 128 columns belong to one 1x128 tile column, so each row
// has a single input scale.  Thread t owns 8 rows (rg = t/16) x 8 columns
// (cc = t%16): 8-byte code loads, so the 16 lanes of a DPP row read one
// 128-byte row segment, and two 16-byte loads of its 8 row scales.  Rows and
// columns are multiples of 16, so a thread's 8 rows and 8 columns are either
// all inside the matrix or all outside it.
//
// Memory order.  Consecutive workgroups walk down a block column (block row
// index fastest), so the blocks in flight together write adjacent 128-byte
// segments of the same output rows; loads and stores are non-temporal.
// Measured on MI355X with inputs rotated over 1.2 GB (so that the 256 MB
// last-level cache cannot serve them), a 16384 x 6144 input takes 42 us this
// way against 48 us with workgroups walking along block rows; a plain device
// copy of the same bytes takes 38 us.  The partial column maxima share the
// LDS buffer of the transposed codes (they are dead before the codes are
// staged), which leaves room for more resident workgroups.
struct RequantArgs {
  const uint8_t *q;        // saved codes [R][C]
  const float *s;          // their 1x128 scales [nj][R]
  int64_t R, C;
  int64_t ni, nj;
  uint8_t *qt;             // transposed codes [C][R]
  float *st;               // 128x1 scales [ni][C]
};

constexpr float kRequantFastMin = 0x1p-60f;
constexpr float kRequantFastMax = 0x1p60f;

// fp32(d / b) from b, rh = fp32(1/b) and rl = fp32((1 - b*rh) * rh); exact
// (see above) for b in [kRequantFastMin, kRequantFastMax] and |d/b| >= 2^-12.
__device__ __forceinline__ float quot_2w(float d, float b, float rh, float rl) {
  const float y = __builtin_fmaf(d, rh, d * rl);
  const float e = __builtin_fmaf(-y, b, d);
  const float z = __builtin_fmaf(e, rh, y);
  return __builtin_copysignf(z, d);
}

__global__ __launch_bounds__(256) void requant_t_kernel(RequantArgs a) {
  __shared__ __align__(16) uint8_t lds_t[kTile * kTile];  // transposed codes; first the partial maxima
  __shared__ __align__(16) float lds_cols[kTile];        // column scales b
  __shared__ __align__(16) float lds_colh[kTile];        // rh = fp32(1 / b)
  __shared__ __align__(16) float lds_coll[kTile];        // rl = fp32((1 - b rh) rh)
  float *lds_part = reinterpret_cast<float *>(lds_t);    // column partial maxima [rg][c] (8 KB)

  const int t = threadIdx.x;
  const int cc = t & 15, rg = t >> 4;
  const int64_t bid = blockIdx.x;
  const int64_t bj = bid / a.ni, bi = bid - bj * a.ni;
  const int64_t r0 = bi * kTile + rg * 8;
  const int64_t c0 = bj * kTile + cc * 8;
  const bool valid = r0 < a.R && c0 < a.C;

  u32x2 raw[8];
  f32x4 s0 = (f32x4){0.f, 0.f, 0.f, 0.f}, s1 = s0;
  if (valid) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      raw[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(a.q + (r0 + k) * a.C + c0));
    s0 = *reinterpret_cast<const f32x4 *>(a.s + bj * a.R + r0);
    s1 = *reinterpret_cast<const f32x4 *>(a.s + bj * a.R + r0 + 4);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) raw[k] = (u32x2){0u, 0u};
  }
  const float sr[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};

  // dequantized elements: hardware e4m3 -> fp32 decode (exact), times the
  // row scale
  float d[8][8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[k].x, false);
    const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[k].x, true);
    const auto p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[k].y, false);
    const auto p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[k].y, true);
    d[k][0] = p0[0] * sr[k]; d[k][1] = p0[1] * sr[k];
    d[k][2] = p1[0] * sr[k]; d[k][3] = p1[1] * sr[k];
    d[k][4] = p2[0] * sr[k]; d[k][5] = p2[1] * sr[k];
    d[k][6] = p3[0] * sr[k]; d[k][7] = p3[1] * sr[k];
  }

  // column maxima of |d| over this thread's 8 rows (finite values: the
  // absolute values are free source modifiers of the max instructions)
  float cm[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = __builtin_fmaxf(m, __builtin_fabsf(d[k][c]));
    cm[c] = m;
  }
  *reinterpret_cast<f32x4 *>(&lds_part[rg * kTile + cc * 8]) = (f32x4){cm[0], cm[1], cm[2], cm[3]};
  *reinterpret_cast<f32x4 *>(&lds_part[rg * kTile + cc * 8 + 4]) = (f32x4){cm[4], cm[5], cm[6], cm[7]};
  __syncthreads();

  if (t < kTile) {
    float m = 0.0f;
#pragma unroll
    for (int g = 0; g < 16; ++g) m = fmaxf(m, lds_part[g * kTile + t]);
    const float sc = tile_scale(m);
    const float rh = 1.0f / sc;
    lds_cols[t] = sc;
    lds_colh[t] = rh;
    lds_coll[t] = __builtin_fmaf(-rh, sc, 1.0f) * rh;
    const int64_t cg = bj * kTile + t;
    if (cg < a.C) a.st[bi * a.C + cg] = sc;
  }
  __syncthreads();

  bool fast = true;
  {
    const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&lds_cols[cc * 8]);
    const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&lds_cols[cc * 8 + 4]);
    const float cs[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) fast &= cs[c] >= kRequantFastMin && cs[c] <= kRequantFastMax;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float b = lds_cols[cc * 8 + c], rh = lds_colh[cc * 8 + c], rl = lds_coll[cc * 8 + c];
    float v[8];
    if (fast) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = quot_2w(d[k][c], b, rh, rl);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = d[k][c] / b;
    }
    u32x2 col;
    col.x = pack4_e4m3(v[0], v[1], v[2], v[3]);
    col.y = pack4_e4m3(v[4], v[5], v[6], v[7]);
    put_transposed_slot(lds_t, cc * 8 + c, rg, col);
  }
  __syncthreads();
  flush_transposed<true>(lds_t, a.qt, a.R, a.C, bi, bj, t);
}

template <bool kRow, bool kCol, bool kBlock, bool kWriteRow, bool kWriteT, bool kSwiGLU = false, bool kTRow = false>
static hipError_t launch_quant(const QuantArgs &a, hipStream_t stream) {
  const int64_t blocks = a.ni * a.nj;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((quant_block_kernel<kRow, kCol, kBlock, kWriteRow, kWriteT, kSwiGLU, kTRow>),
                     dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

static QuantArgs make_args(const uint16_t *x, int64_t R, int64_t C) {
  QuantArgs a{};
  a.x = x;
  a.R = R;
  a.C = C;
  a.ld = C;
  a.ni = (R + kTile - 1) / kTile;
  a.nj = (C + kTile - 1) / kTile;
  // Inputs at least 64 blocks wide go in bands of 8 block rows: measured on
  // the 16384 x 12288 gradient's dual quantizer, 0.172-0.173 ms against
  // 0.187-0.188 ms row-major (column-major: 0.195 ms); narrower inputs gain
  // nothing from it.
  a.band = a.nj >= 64 ? 8 : 1;
  return a;
}

hipError_t run_quant_act_1x128(const uint16_t *x, int64_t R, int64_t C, uint8_t *q, float *s,
                               hipStream_t stream) {
  QuantArgs a = make_args(x, R, C);
  a.q = q;
  a.s = s;
  return launch_quant<true, false, false, true, false>(a, stream);
}

hipError_t run_quant_w_128x128(const uint16_t *w, int64_t R, int64_t C, uint8_t *q, float *s,
                               hipStream_t stream) {
  QuantArgs a = make_args(w, R, C);
  a.q = q;
  a.s = s;
  return launch_quant<false, false, true, true, false>(a, stream);
}

hipError_t run_quant_t_act(const uint16_t *x, int64_t R, int64_t C, uint8_t *qt, float *st,
                           uint8_t *q, float *s, hipStream_t stream) {
  QuantArgs a = make_args(x, R, C);
  a.qt = qt;
  a.st = st;
  a.q = q;
  a.s = s;
  if (q) return launch_quant<true, true, false, true, true>(a, stream);
  return launch_quant<false, true, false, false, true>(a, stream);
}

hipError_t run_quant_act_128x1(const uint16_t *x, int64_t R, int64_t C, uint8_t *qc, float *sc, uint8_t *q,
                               float *s, hipStream_t stream) {
  QuantArgs a = make_args(x, R, C);
  a.qt = qc;          // [R][C]: the 128x1 codes in x's layout
  a.st = sc;
  a.q = q;
  a.s = s;
  if (q) return launch_quant<true, true, false, true, true, false, true>(a, stream);
  return launch_quant<false, true, false, false, true, false, true>(a, stream);
}

hipError_t run_quant_t_w(const uint16_t *w, int64_t R, int64_t C, uint8_t *qt, float *st,
                         uint8_t *q, float *s, hipStream_t stream) {
  QuantArgs a = make_args(w, R, C);
  a.qt = qt;
  a.st = st;
  a.q = q;
  a.s = s;
  if (q) return launch_quant<false, false, true, true, true>(a, stream);
  return launch_quant<false, false, true, false, true>(a, stream);
}

hipError_t run_quant_weights(int count, const WeightQuant *w, hipStream_t stream) {
  QuantGroupArgs g{};
  g.count = count;
  int64_t blocks = 0;
  bool row = false, tr = false;
  for (int i = 0; i < count; ++i) {
    QuantArgs a = make_args(w[i].w, w[i].R, w[i].C);
    a.q = w[i].q;
    a.s = w[i].s;
    a.qt = w[i].qt;
    a.st = w[i].st;
    row = a.q != nullptr;
    tr = a.qt != nullptr;
    g.t[i] = a;
    g.first[i] = blocks;
    blocks += a.ni * a.nj;
  }
  g.first[count] = blocks;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  if (row && tr) hipLaunchKernelGGL((quant_weights_kernel<true, true>), grid, dim3(256), 0, stream, g);
  else if (tr) hipLaunchKernelGGL((quant_weights_kernel<false, true>), grid, dim3(256), 0, stream, g);
  else hipLaunchKernelGGL((quant_weights_kernel<true, false>), grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t run_swiglu_quant(const uint16_t *gu, int64_t R, int64_t I, uint8_t *q, float *s, uint8_t *qt,
                            float *st, uint16_t *h, hipStream_t stream) {
  QuantArgs a = make_args(gu, R, I);
  a.ld = 2 * I;
  a.q = q;
  a.s = s;
  a.qt = qt;
  a.st = st;
  a.h = h;
  if (qt) return launch_quant<true, true, false, true, true, true>(a, stream);
  return launch_quant<true, false, false, true, false, true>(a, stream);
}

hipError_t run_requant_act_t(const uint8_t *q, const float *s, int64_t R, int64_t C, uint8_t *qt,
                             float *st, hipStream_t stream) {
  RequantArgs a{};
  a.q = q;
  a.s = s;
  a.R = R;
  a.C = C;
  a.ni = (R + kTile - 1) / kTile;
  a.nj = (C + kTile - 1) / kTile;
  a.qt = qt;
  a.st = st;
  const int64_t blocks = a.ni * a.nj;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(requant_t_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace puro
