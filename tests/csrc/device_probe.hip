// Test-only probes of device code that the kernels rely on (built by the
// package's build step into tests/csrc/libdevprobe.so; loaded by the GPU tests
// only, never by the library).
//
//  - probe_pack_e4m3: the quantizers' fp32 -> e4m3 conversion (pack4_e4m3 of
//    device_common.h, the hardware round-to-nearest-even pack) applied to every
//    fp32 bit pattern of a range, so that a test can compare it with the
//    oracle's encoder over all values a quantizer can hand it;
//  - probe_mfma32_slice: one 128-deep slice of a 32x32 output block through
//    v_mfma_f32_32x32x64_f8f6f4 (two instructions, the second accumulating
//    onto the first), to measure that instruction's summation precision next
//    to the 16x16x128 form the GEMM uses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Thread i converts the values of bit patterns (start + 4i + j) | sign, j < 4,
// and stores the codes of those below `count`.
__global__ __launch_bounds__(256) void pack_e4m3_kernel(uint32_t start, uint32_t count, uint32_t sign, uint8_t *out) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  const uint32_t e0 = 4u * i;
  if (e0 >= count) return;
  float f[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(((start + e0 + j) | sign));
  const uint32_t w = puro::pack4_e4m3(f[0], f[1], f[2], f[3]);
  if (e0 + 4 <= count) {
    *reinterpret_cast<uint32_t *>(out + e0) = w;     // out is 4-byte aligned and count-sized
  } else {
    for (uint32_t j = 0; e0 + j < count; ++j) out[e0 + j] = (uint8_t)(w >> (8 * j));
  }
}

// One wave.  Lane l supplies row l % 32 of A and of B at k = 32 (l / 32) .. +31
// of each 64-deep half; lane l receives out[m][n] for n = l % 32 and
// m = 8j + 4 (l / 32) + v (j, v < 4).
__global__ __launch_bounds__(64) void mfma32_slice_kernel(const uint8_t *a, const uint8_t *b, float *out) {
  const int l = threadIdx.x;
  const int r = l & 31, h = l >> 5;
  const v8i a0 = *reinterpret_cast<const v8i *>(a + r * 128 + 32 * h);
  const v8i a1 = *reinterpret_cast<const v8i *>(a + r * 128 + 64 + 32 * h);
  const v8i b0 = *reinterpret_cast<const v8i *>(b + r * 128 + 32 * h);
  const v8i b1 = *reinterpret_cast<const v8i *>(b + r * 128 + 64 + 32 * h);
  v16f c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, (v16f){}, 0, 0, 0, 0, 0, 0);
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, c, 0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) out[(8 * j + 4 * h + v) * 32 + r] = c[4 * j + v];
}

extern "C" {

// out: `count` bytes of device memory, 4-byte aligned.
int probe_pack_e4m3(uint32_t start, uint32_t count, uint32_t sign, uint8_t *out, hipStream_t stream) {
  if (count == 0) return 0;
  const uint32_t threads = (count + 3u) / 4u;
  hipLaunchKernelGGL(pack_e4m3_kernel, dim3((threads + 255u) / 256u), dim3(256), 0, stream, start, count, sign, out);
  return (int)hipGetLastError();
}

// a, b: [32][128] e4m3 codes (device, 32-byte aligned); out: [32][32] fp32 (device).
int probe_mfma32_slice(const uint8_t *a, const uint8_t *b, float *out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma32_slice_kernel, dim3(1), dim3(64), 0, stream, a, b, out);
  return (int)hipGetLastError();
}
}
