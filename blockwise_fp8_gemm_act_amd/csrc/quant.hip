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
// of bank conflicts) and leave as 128-byte row segments.
#include "device_common.h"
#include "launch.h"

namespace puro {

struct QuantArgs {
  const uint16_t *x;
  int64_t R, C;
  int64_t ni, nj;          // ceil(R/128), ceil(C/128)
  uint8_t *q;              // row-major codes [R][C] (or null)
  float *s;                // scales of the row-major codes
  uint8_t *qt;             // transposed codes [C][R] (or null)
  float *st;               // scales of the transposed codes
};

// kRow:   1x128 scales (per row of the block)       -> row-major output
// kCol:   128x1 scales (per column of the block)    -> transposed output
// kBlock: one 128x128 scale                         -> row-major and/or transposed output
template <bool kRow, bool kCol, bool kBlock, bool kWriteRow, bool kWriteT>
__global__ __launch_bounds__(256) void quant_block_kernel(QuantArgs a) {
  __shared__ float lds_part[16 * kTile];                 // column partial maxima [rg][c]
  __shared__ float lds_rowamax[kTile];
  __shared__ __align__(16) float lds_rows[kTile], lds_rowr[kTile];
  __shared__ __align__(16) float lds_cols[kTile], lds_colr[kTile];
  __shared__ float lds_wmax[4];
  __shared__ __align__(16) uint8_t lds_t[kWriteT ? kTile * kTile : 16];

  const int t = threadIdx.x;
  const int cc = t & 15, rg = t >> 4;
  const int64_t bid = blockIdx.x;
  const int64_t bi = bid / a.nj, bj = bid - bi * a.nj;
  const int64_t r0 = bi * kTile + rg * 8;
  const int64_t c0 = bj * kTile + cc * 8;
  const bool cvalid = c0 < a.C;

  // ---- load 8 rows x 8 columns (16 B per row), all in flight at once
  u32x4 raw[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t r = r0 + k;
    if (cvalid && r < a.R)
      raw[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.x + r * a.C + c0));
    else
      raw[k] = (u32x4){0u, 0u, 0u, 0u};
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
      if (cvalid && r < a.R) __builtin_nontemporal_store(o, reinterpret_cast<u32x2 *>(a.q + r * a.C + c0));
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
    // LDS row c (a column of the block) holds 16 slots of 8 codes (8 rows);
    // slot rg is stored at physical slot rg ^ (c / 8).
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
      const int lc = cc * 8 + c;
      *reinterpret_cast<u32x2 *>(&lds_t[lc * kTile + ((rg ^ cc) * 8)]) = col;
    }
    __syncthreads();
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
      if (orow < a.C && ocol < a.R)
        __builtin_nontemporal_store(d, reinterpret_cast<u32x4 *>(a.qt + orow * a.R + ocol));
    }
  }
}

template <bool kRow, bool kCol, bool kBlock, bool kWriteRow, bool kWriteT>
static hipError_t launch_quant(const QuantArgs &a, hipStream_t stream) {
  const int64_t blocks = a.ni * a.nj;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((quant_block_kernel<kRow, kCol, kBlock, kWriteRow, kWriteT>),
                     dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

static QuantArgs make_args(const uint16_t *x, int64_t R, int64_t C) {
  QuantArgs a{};
  a.x = x;
  a.R = R;
  a.C = C;
  a.ni = (R + kTile - 1) / kTile;
  a.nj = (C + kTile - 1) / kTile;
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

}  // namespace puro
