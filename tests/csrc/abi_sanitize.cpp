// Host-only driver of the C ABI's validation layer (blockwise_fp8_gemm_act_amd/
// csrc/abi.cpp), built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_abi_sanitized.py.  Tests only.
//
// The HIP runtime calls that abi.cpp makes and the launchers behind it are
// replaced by stubs: the device query reports one gfx950, and every launcher
// records its arguments instead of enqueueing a kernel.  No pointer is ever
// dereferenced by the layer, so the buffers are fake, well separated
// addresses.  The driver checks that
//   - every entry point reaches its own launcher with the caller's arguments
//     when the call is valid;
//   - every error path returns its status and reaches no launcher;
//   - shapes at the limits of the contract evaluate without undefined
//     behaviour (signed overflow in the size arithmetic stops the program).
// Exit status 0 and the line "abi under sanitizers: ok" when every check holds.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "launch.h"
#include "puro.h"

// ---------------------------------------------------------------- HIP stubs
hipError_t hipGetDevice(int *dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_t *prop, int) {
  std::memset(prop, 0, sizeof(*prop));
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }

// ---------------------------------------------------------------- launcher stubs
namespace {
struct Call {
  std::string name;
  const void *p[10];
  int64_t n[4];
  int mode;
  bool flag[2];
  int calls = 0;
};
Call g_last;

void record(const char *name, std::initializer_list<const void *> ptrs, std::initializer_list<int64_t> sizes,
            int mode = -1, bool f0 = false, bool f1 = false) {
  g_last.name = name;
  int i = 0;
  for (const void *p : ptrs) g_last.p[i++] = p;
  for (; i < 10; ++i) g_last.p[i] = nullptr;
  i = 0;
  for (int64_t v : sizes) g_last.n[i++] = v;
  for (; i < 4; ++i) g_last.n[i] = -1;
  g_last.mode = mode;
  g_last.flag[0] = f0;
  g_last.flag[1] = f1;
  ++g_last.calls;
}
}  // namespace

namespace puro {
hipError_t run_quant_act_1x128(const uint16_t *x, int64_t R, int64_t C, uint8_t *q, float *s, hipStream_t st) {
  record("act_1x128", {x, q, s, st}, {R, C});
  return hipSuccess;
}
hipError_t run_quant_w_128x128(const uint16_t *w, int64_t R, int64_t C, uint8_t *q, float *s, hipStream_t st) {
  record("w_128x128", {w, q, s, st}, {R, C});
  return hipSuccess;
}
hipError_t run_quant_t_act(const uint16_t *x, int64_t R, int64_t C, uint8_t *qt, float *st, uint8_t *q, float *s,
                           hipStream_t stream) {
  record("t_act", {x, qt, st, q, s, stream}, {R, C});
  return hipSuccess;
}
hipError_t run_quant_act_128x1(const uint16_t *x, int64_t R, int64_t C, uint8_t *qc, float *sc, uint8_t *q,
                               float *s, hipStream_t stream) {
  record("act_128x1", {x, qc, sc, q, s, stream}, {R, C});
  return hipSuccess;
}
hipError_t run_quant_t_w(const uint16_t *w, int64_t R, int64_t C, uint8_t *qt, float *st, uint8_t *q, float *s,
                         hipStream_t stream) {
  record("t_w", {w, qt, st, q, s, stream}, {R, C});
  return hipSuccess;
}
hipError_t run_quant_weights(int count, const WeightQuant *w, hipStream_t stream) {
  record("weights", {count > 0 ? w[0].w : nullptr, count > 0 ? w[0].q : nullptr, count > 0 ? w[0].qt : nullptr,
                     stream},
         {count, count > 0 ? w[0].R : -1, count > 0 ? w[0].C : -1});
  return hipSuccess;
}
hipError_t run_swiglu_quant(const uint16_t *gu, int64_t R, int64_t I, uint8_t *q, float *s, uint8_t *qt, float *st,
                            uint16_t *h, hipStream_t stream) {
  record("swiglu", {gu, q, s, qt, st, h, stream}, {R, I});
  return hipSuccess;
}
hipError_t run_requant_act_t(const uint8_t *q, const float *s, int64_t R, int64_t C, uint8_t *qt, float *st,
                             hipStream_t stream) {
  record("requant", {q, s, qt, st, stream}, {R, C});
  return hipSuccess;
}
// A stand-in planner: two splits (fp32 partials of the whole output) when K is
// long against the tile count, none otherwise.
GemmPlan plan_gemm(int, int64_t M, int64_t N, int64_t K) {
  GemmPlan p{};
  p.nk = (int)((K + 127) / 128);
  p.tiles_m = (int)((M + 255) / 256);
  p.tiles_n = (int)((N + 255) / 256);
  p.bn = 256;
  p.splits = ((int64_t)p.tiles_m * p.tiles_n < 256 && p.nk >= 8) ? 2 : 1;
  p.spl = (p.nk + p.splits - 1) / p.splits;
  p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * 4 : 0;
  return p;
}
hipError_t run_gemm(int mode, const uint8_t *a, const float *sa, const uint8_t *b, const float *sb, void *out,
                    bool bf16_out, bool accumulate, int64_t M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
  record("gemm", {a, sa, b, sb, out, ws, stream}, {M, N, K}, mode, bf16_out, accumulate);
  return hipSuccess;
}
hipError_t run_gemm_noalloc(int mode, const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                            void *out, bool bf16_out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  record("gemm_noalloc", {a, sa, b, sb, out, stream}, {M, N, K}, mode, bf16_out);
  return hipSuccess;
}
hipError_t run_gemm_swiglu_quant(const uint8_t *a, const float *sa, const uint8_t *b, const float *sb, uint16_t *gu,
                                 uint8_t *hq, float *hs, int64_t M, int64_t I, int64_t K, hipStream_t stream) {
  record("gemm_swiglu", {a, sa, b, sb, gu, hq, hs, stream}, {M, I, K});
  return hipSuccess;
}
}  // namespace puro

// ---------------------------------------------------------------- driver
namespace {
int g_fail = 0;

// Buffer i: a 16-byte-aligned fake address 2^42 bytes from its neighbours, so
// that no two buffers overlap at any size the contract allows.
template <typename T>
T *buf(int i, int64_t byte_offset = 0) {
  return reinterpret_cast<T *>((uintptr_t(i + 1) << 42) + (uintptr_t)byte_offset);
}
puro_stream_t kStream = reinterpret_cast<puro_stream_t>(uintptr_t(0x5150));

void expect(bool ok, const std::string &what) {
  if (!ok) {
    std::printf("FAIL: %s\n", what.c_str());
    ++g_fail;
  }
}

// A call that must launch `name` (status OK) and pass the listed pointers and sizes.
void launches(puro_status st, const char *name, std::initializer_list<const void *> ptrs,
              std::initializer_list<int64_t> sizes, const std::string &what) {
  expect(st == PURO_OK, what + ": status " + std::to_string(st));
  expect(g_last.name == name, what + ": launcher " + g_last.name + ", expected " + name);
  int i = 0;
  for (const void *p : ptrs) {
    expect(g_last.p[i] == p, what + ": pointer argument " + std::to_string(i));
    ++i;
  }
  i = 0;
  for (int64_t v : sizes) {
    expect(g_last.n[i] == v, what + ": size argument " + std::to_string(i));
    ++i;
  }
}

// A call that must return `want` and launch nothing.
void refuses(puro_status st, puro_status want, const std::string &what) {
  expect(st == want, what + ": status " + std::to_string(st) + ", expected " + std::to_string(want));
  expect(g_last.calls == 0, what + ": a launcher ran");
}

void reset() { g_last = Call{}; }

void quantizers() {
  const int64_t R = 272, C = 400;   // ragged: one partial tile in each direction
  // puro_quant_act_1x128
  reset();
  launches(puro_quant_act_1x128(buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(2), kStream), "act_1x128",
           {buf<uint16_t>(0), buf<uint8_t>(1), buf<float>(2), kStream}, {R, C}, "act_1x128 valid");
  reset();
  refuses(puro_quant_act_1x128(buf<uint16_t>(0), R, C + 8, buf<uint8_t>(1), buf<float>(2), kStream), PURO_ERR_SHAPE,
          "act_1x128 cols % 16");
  reset();
  refuses(puro_quant_act_1x128(buf<uint16_t>(0), -1, C, buf<uint8_t>(1), buf<float>(2), kStream), PURO_ERR_SHAPE,
          "act_1x128 negative rows");
  reset();
  refuses(puro_quant_act_1x128(nullptr, R, C, buf<uint8_t>(1), buf<float>(2), kStream), PURO_ERR_NULL,
          "act_1x128 null input");
  reset();
  refuses(puro_quant_act_1x128(buf<uint16_t>(0), R, C, buf<uint8_t>(1, 8), buf<float>(2), kStream), PURO_ERR_ALIGN,
          "act_1x128 misaligned codes");
  reset();
  refuses(puro_quant_act_1x128(buf<uint16_t>(0), R, C, buf<uint8_t>(0, 1024), buf<float>(2), kStream),
          PURO_ERR_ALIAS, "act_1x128 codes inside the input");
  reset();
  refuses(puro_quant_act_1x128(nullptr, 0, C, nullptr, nullptr, kStream), PURO_OK, "act_1x128 empty");
  // the limits: rows at 2^31 - 1 with 16 columns, and the largest element count
  reset();
  launches(puro_quant_act_1x128(buf<uint16_t>(0), (int64_t(1) << 31) - 1, 16, buf<uint8_t>(1), buf<float>(2),
                                kStream),
           "act_1x128", {}, {(int64_t(1) << 31) - 1, 16}, "act_1x128 at the row limit");
  reset();
  launches(puro_quant_act_1x128(buf<uint16_t>(0), int64_t(1) << 24, int64_t(1) << 16, buf<uint8_t>(1),
                                buf<float>(2), kStream),
           "act_1x128", {}, {int64_t(1) << 24, int64_t(1) << 16}, "act_1x128 at the element limit");
  reset();
  refuses(puro_quant_act_1x128(buf<uint16_t>(0), (int64_t(1) << 24) + 1, int64_t(1) << 16, buf<uint8_t>(1),
                               buf<float>(2), kStream),
          PURO_ERR_SHAPE, "act_1x128 past the element limit");
  reset();
  refuses(puro_quant_act_1x128(buf<uint16_t>(0), INT64_MAX, INT64_MAX - 15, buf<uint8_t>(1), buf<float>(2), kStream),
          PURO_ERR_SHAPE, "act_1x128 INT64_MAX shape");

  // puro_quant_w_128x128
  reset();
  launches(puro_quant_w_128x128(buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(2), kStream), "w_128x128",
           {buf<uint16_t>(0), buf<uint8_t>(1), buf<float>(2), kStream}, {R, C}, "w_128x128 valid");
  reset();
  refuses(puro_quant_w_128x128(buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(1, R * C - 16), kStream),
          PURO_ERR_ALIAS, "w_128x128 scales overlapping the codes' last 16 bytes");
  reset();
  launches(puro_quant_w_128x128(buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(1, R * C), kStream), "w_128x128",
           {buf<uint16_t>(0), buf<uint8_t>(1), buf<float>(1, R * C), kStream}, {R, C},
           "w_128x128 scales right after the codes");

  // puro_quant_transpose: both kinds, single and dual
  reset();
  launches(puro_quant_transpose(PURO_T_ACT, buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(2), buf<uint8_t>(3),
                                buf<float>(4), kStream),
           "t_act", {buf<uint16_t>(0), buf<uint8_t>(1), buf<float>(2), buf<uint8_t>(3), buf<float>(4), kStream},
           {R, C}, "transpose ACT dual");
  reset();
  launches(puro_quant_transpose(PURO_T_WEIGHT, buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(2), nullptr,
                                nullptr, kStream),
           "t_w", {buf<uint16_t>(0), buf<uint8_t>(1), buf<float>(2), nullptr, nullptr, kStream}, {R, C},
           "transpose WEIGHT single");
  reset();
  refuses(puro_quant_transpose((puro_t_kind)7, buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(2), nullptr,
                               nullptr, kStream),
          PURO_ERR_MODE, "transpose bad kind");
  reset();
  refuses(puro_quant_transpose(PURO_T_ACT, buf<uint16_t>(0), R + 1, C, buf<uint8_t>(1), buf<float>(2), nullptr,
                               nullptr, kStream),
          PURO_ERR_SHAPE, "transpose rows % 16");
  reset();
  refuses(puro_quant_transpose(PURO_T_ACT, buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(2), buf<uint8_t>(3),
                               nullptr, kStream),
          PURO_ERR_NULL, "transpose half of the dual pair");
  reset();
  refuses(puro_quant_transpose(PURO_T_ACT, buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(2), buf<uint8_t>(1),
                               buf<float>(4), kStream),
          PURO_ERR_ALIAS, "transpose outputs sharing a buffer");

  // puro_quant_act_128x1
  reset();
  launches(puro_quant_act_128x1(buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(2), buf<uint8_t>(3),
                                buf<float>(4), kStream),
           "act_128x1", {buf<uint16_t>(0), buf<uint8_t>(1), buf<float>(2), buf<uint8_t>(3), buf<float>(4), kStream},
           {R, C}, "act_128x1 dual");
  reset();
  refuses(puro_quant_act_128x1(buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(2, 4), nullptr, nullptr, kStream),
          PURO_ERR_ALIGN, "act_128x1 misaligned scales");

  // puro_swiglu_quant
  reset();
  launches(puro_swiglu_quant(buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(2), buf<uint8_t>(3), buf<float>(4),
                             buf<uint16_t>(5), kStream),
           "swiglu",
           {buf<uint16_t>(0), buf<uint8_t>(1), buf<float>(2), buf<uint8_t>(3), buf<float>(4), buf<uint16_t>(5), kStream},
           {R, C}, "swiglu dual with h");
  reset();
  refuses(puro_swiglu_quant(buf<uint16_t>(0), R, C, buf<uint8_t>(1), buf<float>(2), nullptr, nullptr,
                            buf<uint16_t>(0, R * C * 2), kStream),
          PURO_ERR_ALIAS, "swiglu h inside the up half of the input");
  reset();
  refuses(puro_swiglu_quant(buf<uint16_t>(0), R, (int64_t(1) << 30) + 16, buf<uint8_t>(1), buf<float>(2), nullptr,
                            nullptr, nullptr, kStream),
          PURO_ERR_SHAPE, "swiglu 2 x inter past the row limit");

  // puro_requant_act_t
  reset();
  launches(puro_requant_act_t(buf<uint8_t>(0), buf<float>(1), R, C, buf<uint8_t>(2), buf<float>(3), kStream),
           "requant", {buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3), kStream}, {R, C},
           "requant valid");
  reset();
  refuses(puro_requant_act_t(buf<uint8_t>(0), buf<float>(1), R, C, buf<uint8_t>(2), nullptr, kStream), PURO_ERR_NULL,
          "requant null scales out");

  // puro_quant_weights
  puro_weight ws[9];
  for (int i = 0; i < 9; ++i)
    ws[i] = puro_weight{buf<uint16_t>(10 + 5 * i), 256, 128, buf<uint8_t>(11 + 5 * i), buf<float>(12 + 5 * i),
                        buf<uint8_t>(13 + 5 * i), buf<float>(14 + 5 * i)};
  reset();
  launches(puro_quant_weights(4, ws, kStream), "weights", {ws[0].w, ws[0].q, ws[0].qt, kStream}, {4, 256, 128},
           "weights four");
  reset();
  refuses(puro_quant_weights(9, ws, kStream), PURO_ERR_SHAPE, "weights nine");
  puro_weight mixed[2] = {ws[0], ws[1]};
  mixed[1].qt = nullptr;
  mixed[1].st = nullptr;
  reset();
  refuses(puro_quant_weights(2, mixed, kStream), PURO_ERR_NULL, "weights with different outputs");
  puro_weight shared[2] = {ws[0], ws[1]};
  shared[1].q = ws[0].q;
  reset();
  refuses(puro_quant_weights(2, shared, kStream), PURO_ERR_ALIAS, "weights sharing a code buffer");
}

void gemms() {
  const int64_t M = 300, N = 520, K = 2064;   // ragged tiles, split by the stand-in planner
  const size_t need = puro_gemm_workspace_bytes(PURO_WGRAD, M, N, K);
  expect(need == 2 * (size_t)M * N * 4, "workspace bytes of a split plan");
  expect(puro_gemm_workspace_bytes((puro_gemm_mode)9, M, N, K) == 0, "workspace bytes of a bad mode");
  expect(puro_gemm_workspace_bytes(PURO_FPROP, M, N, int64_t(1) << 24) == 0, "workspace bytes past the K limit");
  for (int mode = PURO_FPROP; mode <= PURO_WGRAD_TM; ++mode) {
    const std::string m = "gemm mode " + std::to_string(mode);
    const int64_t Mm = mode == PURO_WGRAD_TM ? 304 : M, Nm = mode == PURO_WGRAD_TM ? 528 : N;
    const size_t w = puro_gemm_workspace_bytes((puro_gemm_mode)mode, Mm, Nm, K);
    reset();
    launches(puro_gemm_fp8_blockwise((puro_gemm_mode)mode, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2),
                                     buf<float>(3), buf<void>(4), PURO_OUT_BF16, Mm, Nm, K, buf<void>(5), w, kStream),
             "gemm",
             {buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3), buf<void>(4), buf<void>(5), kStream},
             {Mm, Nm, K}, m);
    expect(g_last.mode == mode && g_last.flag[0] && !g_last.flag[1], m + ": mode and flags");
    reset();
    launches(puro_gemm_fp8_blockwise_accumulate((puro_gemm_mode)mode, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2),
                                                buf<float>(3), buf<float>(4), Mm, Nm, K, buf<void>(5), w, kStream),
             "gemm", {}, {Mm, Nm, K}, m + " accumulate");
    expect(!g_last.flag[0] && g_last.flag[1], m + " accumulate: fp32 and accumulate flags");
    reset();
    launches(puro_gemm_fp8_blockwise_noalloc((puro_gemm_mode)mode, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2),
                                             buf<float>(3), buf<void>(4), PURO_OUT_F32, Mm, Nm, K, kStream),
             "gemm_noalloc", {buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3), buf<void>(4), kStream},
             {Mm, Nm, K}, m + " noalloc");
  }
  reset();
  refuses(puro_gemm_fp8_blockwise(PURO_WGRAD, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3),
                                  buf<void>(4), PURO_OUT_F32, M, N, K, buf<void>(5), need - 16, kStream),
          PURO_ERR_WORKSPACE, "gemm workspace too small");
  reset();
  refuses(puro_gemm_fp8_blockwise(PURO_WGRAD, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3),
                                  buf<void>(4), PURO_OUT_F32, M, N, K, nullptr, 0, kStream),
          PURO_ERR_WORKSPACE, "gemm workspace missing");
  reset();
  refuses(puro_gemm_fp8_blockwise(PURO_WGRAD, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3),
                                  buf<void>(4), PURO_OUT_F32, M, N, K, buf<void>(4, 64), need, kStream),
          PURO_ERR_ALIAS, "gemm workspace inside the output");
  reset();
  refuses(puro_gemm_fp8_blockwise(PURO_FPROP, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3),
                                  buf<void>(4), (puro_out_dtype)5, M, N, K, buf<void>(5), need, kStream),
          PURO_ERR_DTYPE, "gemm bad dtype");
  reset();
  refuses(puro_gemm_fp8_blockwise((puro_gemm_mode)9, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3),
                                  buf<void>(4), PURO_OUT_F32, M, N, K, buf<void>(5), need, kStream),
          PURO_ERR_MODE, "gemm bad mode");
  reset();
  refuses(puro_gemm_fp8_blockwise(PURO_FPROP, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3),
                                  buf<void>(4), PURO_OUT_F32, M, N, (int64_t(1) << 23) + 16, buf<void>(5), need, kStream),
          PURO_ERR_SHAPE, "gemm K past 2^23");
  reset();
  refuses(puro_gemm_fp8_blockwise(PURO_WGRAD_TM, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3),
                                  buf<void>(4), PURO_OUT_F32, M, N, K, buf<void>(5), need, kStream),
          PURO_ERR_SHAPE, "token-major wgrad with M % 16 != 0");
  reset();
  refuses(puro_gemm_fp8_blockwise(PURO_FPROP, nullptr, buf<float>(1), buf<uint8_t>(2), buf<float>(3), buf<void>(4),
                                  PURO_OUT_F32, M, N, K, buf<void>(5), need, kStream),
          PURO_ERR_NULL, "gemm null A");
  reset();
  refuses(puro_gemm_fp8_blockwise_noalloc(PURO_WGRAD, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3),
                                          buf<void>(4), PURO_OUT_F32, 3840, 3840, K, kStream),
          PURO_ERR_SCRATCH, "noalloc plan past the scratch");
  reset();
  refuses(puro_gemm_fp8_blockwise(PURO_FPROP, buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3),
                                  buf<void>(4), PURO_OUT_F32, INT64_MAX, INT64_MAX, INT64_MAX, nullptr, 0, kStream),
          PURO_ERR_SHAPE, "gemm INT64_MAX shape");
  // K = 0: the output is written (zeros), operands are not needed
  reset();
  launches(puro_gemm_fp8_blockwise(PURO_FPROP, nullptr, nullptr, nullptr, nullptr, buf<void>(4), PURO_OUT_BF16, M, N, 0,
                                   nullptr, 0, kStream),
           "gemm", {nullptr, nullptr, nullptr, nullptr, buf<void>(4)}, {M, N, 0}, "gemm K = 0");

  // the fused gate/up fprop with the SwiGLU quantizer as its epilogue
  const int64_t I = 384;
  reset();
  launches(puro_gemm_fp8_swiglu_quant(buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3), M, I, K,
                                      buf<uint16_t>(4), buf<uint8_t>(5), buf<float>(6), kStream),
           "gemm_swiglu",
           {buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3), buf<uint16_t>(4), buf<uint8_t>(5),
            buf<float>(6), kStream},
           {M, I, K}, "gemm_swiglu valid");
  reset();
  refuses(puro_gemm_fp8_swiglu_quant(buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3), M, I + 16, K,
                                     nullptr, buf<uint8_t>(5), buf<float>(6), kStream),
          PURO_ERR_SHAPE, "gemm_swiglu inter % 128");
  reset();
  refuses(puro_gemm_fp8_swiglu_quant(buf<uint8_t>(0), buf<float>(1), buf<uint8_t>(2), buf<float>(3), M, I, K,
                                     nullptr, buf<uint8_t>(5), buf<float>(5, 256), kStream),
          PURO_ERR_ALIAS, "gemm_swiglu scales inside the codes");
}
}  // namespace

int main() {
  expect(puro_abi_version() == PURO_ABI_VERSION, "abi version");
  for (int s = PURO_OK; s <= PURO_ERR_SCRATCH; ++s)
    expect(std::strcmp(puro_status_str((puro_status)s), "unknown status") != 0, "status string " + std::to_string(s));
  quantizers();
  gemms();
  if (g_fail) {
    std::printf("%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("abi under sanitizers: ok\n");
  return 0;
}
