// Device helpers shared by the gfx950 kernels: bf16 unpacking, the e4m3 tile
// scale and code rule, DPP reductions, the SwiGLU value.
//
// Quantization rule (the pages name DeepSeek-V3's fine-grained block
// quantization for the main linear layers -- en.roboind.com article on
// Puro-2B, section "FP8 takes advantage of the RTX 5090's low precision
// efficiency"; the rule itself is this library's reading):
//   s = fp32(amax / 448), or 1 when amax == 0
//   q = e4m3_rne_saturating(fp32(x / s))
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace puro {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 128;          // tile edge (elements)
constexpr float kE4m3Max = 448.0f;  // largest finite OCP E4M3FN value

// Tiles whose scale is at least this take the reciprocal path for x / s; the
// rest divide.  For every pair of bf16 values (x, amax) with |x| <= amax and
// amax >= 2^-104, the reciprocal path yields the same fp32 quotient as an
// IEEE division whenever |x / s| >= 2^-12, and a value of the same sign below
// 2^-10 otherwise -- hence the same e4m3 code (checked exhaustively over all
// such pairs).  s >= 2^-73 implies amax > 2^-65, a wide margin.
constexpr float kFastDivMinScale = 0x1p-73f;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Scale of a tile from its absolute maximum (IEEE division, no fast-math).
__device__ __forceinline__ float tile_scale(float amax) {
  return amax == 0.0f ? 1.0f : amax / kE4m3Max;
}

// Per-tile constants for quantizing: the scale, its correctly rounded
// reciprocal, and whether the reciprocal path is valid for this tile.
struct TileQ {
  float s;
  float r;
  bool fast;
};

__device__ __forceinline__ TileQ make_tileq(float amax) {
  TileQ t;
  t.s = tile_scale(amax);
  t.r = 1.0f / t.s;
  t.fast = t.s >= kFastDivMinScale;
  return t;
}

// fp32(x / s), exactly, via the reciprocal: y = x*r is within a few ulp of
// the quotient; one residual step (Markstein) rounds it correctly.  The sign
// is restored explicitly so that -0 stays -0.
__device__ __forceinline__ float quot_fast(float x, float s, float r) {
  float y = x * r;
  float e = __builtin_fmaf(-y, s, x);
  float z = __builtin_fmaf(e, r, y);
  return __builtin_copysignf(z, x);
}

__device__ __forceinline__ float quot(float x, const TileQ &t) {
  return t.fast ? quot_fast(x, t.s, t.r) : x / t.s;
}

// Four fp32 values (already divided by the scale, |v| <= 448 up to one ulp)
// to four e4m3 codes packed little-endian in one dword.  The hardware
// conversion rounds to nearest even (OCP E4M3FN on gfx950).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Max over the 16 lanes of a DPP row (lanes 16k .. 16k+15); every lane of the
// row gets the result.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));  // row_ror:8
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));  // row_ror:4
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false)));  // row_ror:2
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false)));  // row_ror:1
  return v;
}

// Magnitude bits of the two bf16 values packed in a word.  For finite values
// the magnitude bits order exactly like the magnitudes, so maxima can be taken
// on them as 16-bit integers (packed max) and turned into a float at the end:
// the fp32 value of a bf16 magnitude m is the bit pattern m << 16.
__device__ __forceinline__ u16x2 bf16_mags(uint32_t w) {
  return __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
}
__device__ __forceinline__ u16x2 max16x2(u16x2 a, u16x2 b) { return __builtin_elementwise_max(a, b); }
__device__ __forceinline__ uint32_t hmax16(u16x2 a) { return a.x > a.y ? a.x : a.y; }
__device__ __forceinline__ float mag_to_float(uint32_t m) { return __uint_as_float(m << 16); }

// Max over the 16 lanes of a DPP row of non-negative integers.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));  // row_ror:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));  // row_ror:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false));  // row_ror:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false));  // row_ror:1
  return v;
}

// Max over a whole wave of 64 lanes of non-negative integers, returned uniformly.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row16_max_u32(v);
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

// Max over a whole wave of 64 lanes, returned uniformly.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// fp32 -> bf16 bits, round to nearest even (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// SwiGLU of one gate/up pair, h = bf16(silu(g) * u), silu(g) = g / (1 + e^-g).
// The value is defined as the fp64 evaluation of that expression, rounded
// once to bf16 (round to nearest even).
//
// Fast path, fp32: s = g * rcp(1 + expf(-g)) is within 2.94 * 2^-24 of
// silu(g) (relative) for every bf16 g with |g| <= 64, measured exhaustively
// on gfx950 against fp64; with the rounding of p = s * u, p is within 3.44
// fp32 ulps of the exact product.  So unless p's low 16 bits lie within 5
// ulps of the bf16 rounding midpoint (0x8000), rounding p gives the bf16 of
// the exact value, which the fp64 value rounds to as well.  Otherwise, or for
// |g| > 64, the element takes the fp64 evaluation (swiglu_f64).
__device__ __forceinline__ uint32_t swiglu_fast(float g, float u, bool &slow) {
  const float e = expf(-g);
  const float sg = g * __builtin_amdgcn_rcpf(1.0f + e);
  const float p = sg * u;
  const uint32_t b = __float_as_uint(p);
  slow = ((b & 0xffffu) - 0x7ffbu) <= 10u || !(__builtin_fabsf(g) <= 64.0f);
  return (b + 0x8000u) >> 16;
}

// bf16 bits of v, round to nearest even (from fp64: one rounding).
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double v) {
  const uint32_t sign = signbit(v) ? 0x8000u : 0u;
  const double a = fabs(v);
  if (a == 0.0) return sign;
  if (a < 0x1p-126) return sign | (uint32_t)rint(ldexp(a, 133));   // 2^-133 grid
  int e = ilogb(a);
  double n = rint(ldexp(a, 7 - e));                                 // 128 .. 256
  if (n == 256.0) { n = 128.0; ++e; }
  if (e > 127) return sign | 0x7f80u;
  return sign | ((uint32_t)(e + 127) << 7) | ((uint32_t)n - 128u);
}

__device__ __forceinline__ uint32_t swiglu_f64(float g, float u) {
  const double gd = g, ud = u;
  return f64_to_bf16_bits(gd / (1.0 + exp(-gd)) * ud);
}

}  // namespace puro
