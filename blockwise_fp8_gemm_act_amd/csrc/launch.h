// Internal launchers behind the C ABI (host side).  Arguments are already
// validated by the ABI layer when these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace puro {

hipError_t run_quant_act_1x128(const uint16_t *x, int64_t R, int64_t C, uint8_t *q, float *s,
                               hipStream_t stream);
hipError_t run_quant_w_128x128(const uint16_t *w, int64_t R, int64_t C, uint8_t *q, float *s,
                               hipStream_t stream);
hipError_t run_quant_t_act(const uint16_t *x, int64_t R, int64_t C, uint8_t *qt, float *st,
                           uint8_t *q, float *s, hipStream_t stream);
// 128x1 codes of x in x's own layout (qc [R][C], sc [ceil(R/128)][C]); q, s
// optional 1x128 codes from the same read.
hipError_t run_quant_act_128x1(const uint16_t *x, int64_t R, int64_t C, uint8_t *qc, float *sc, uint8_t *q,
                               float *s, hipStream_t stream);
hipError_t run_quant_t_w(const uint16_t *w, int64_t R, int64_t C, uint8_t *qt, float *st,
                         uint8_t *q, float *s, hipStream_t stream);
// One launch over several weights (at most 8), each as run_quant_t_w / run_quant_w_128x128:
// every entry has the same outputs (row-wise q, s and/or transposed qt, st).
struct WeightQuant {
  const uint16_t *w;
  int64_t R, C;
  uint8_t *q;
  float *s;
  uint8_t *qt;
  float *st;
};
hipError_t run_quant_weights(int count, const WeightQuant *w, hipStream_t stream);
hipError_t run_swiglu_quant(const uint16_t *gu, int64_t R, int64_t I, uint8_t *q, float *s, uint8_t *qt,
                            float *st, uint16_t *h, hipStream_t stream);
hipError_t run_requant_act_t(const uint8_t *q, const float *s, int64_t R, int64_t C, uint8_t *qt,
                             float *st, hipStream_t stream);

struct GemmPlan {
  int nk;          // 128-deep K slices
  int tiles_m, tiles_n;
  int splits;      // K-loop splits
  int spl;         // slices per split
  int whole;       // > 0: tiles 0 .. whole-1 run unsplit in a first launch, only the rest split
  int bn;          // tile width: 256, or 192 / 128 (weight gradient)
  size_t ws_bytes; // fp32 split-K partials
};

// Deterministic launch plan of a GEMM shape (host only, no device access).
GemmPlan plan_gemm(int mode, int64_t M, int64_t N, int64_t K);

// accumulate: out (fp32) = out + GEMM instead of out = GEMM.
hipError_t run_gemm(int mode, const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                    void *out, bool bf16_out, bool accumulate, int64_t M, int64_t N, int64_t K, void *ws,
                    hipStream_t stream);

// The GEMM with its split-K partials in the library's own device scratch
// (kScratchBytes, one per device) instead of a caller's workspace: no device
// allocation.  Shapes whose plan needs more scratch are refused
// (hipErrorInvalidValue; the ABI layer checks this first).  Calls that overlap
// on one device share the scratch and race.
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t run_gemm_noalloc(int mode, const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                            void *out, bool bf16_out, int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Fused fprop of a gate/up projection (B = [gate rows; up rows], 2I x K,
// 128x128 block scales) with the SwiGLU quantizer as its epilogue: gu (bf16
// [M][2I], optional), hq / hs (1x128 codes and scales of h).  I % 128 == 0.
hipError_t run_gemm_swiglu_quant(const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                                 uint16_t *gu, uint8_t *hq, float *hs, int64_t M, int64_t I, int64_t K,
                                 hipStream_t stream);

}  // namespace puro
