// C ABI of the blockwise-FP8 library: argument validation on the host,
// device check, dispatch to the gfx950 kernels.  See include/puro.h for the
// contract of every call.
//
// Validation runs entirely on the host and before any HIP call, in this
// order: mode/kind/dtype, shapes, NULL pointers, alignment, overlaps,
// workspace; then the device is checked (gfx950) and the kernels are
// enqueued.  Nothing is enqueued when any check fails.
#include "puro.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "launch.h"

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kMaxGemmK = int64_t(1) << 23;    // 256 rows x K must index in 32 bits

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;   // [lo, hi)
};

Range rng(const void *p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Any output overlapping any input or another output.
bool any_alias(const Range *in, int nin, const Range *out, int nout) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(out[i], in[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(out[i], out[j])) return true;
  }
  return false;
}

bool shape_ok(int64_t r, int64_t c) {
  if (r < 0 || c < 0 || r > kMaxDim || c > kMaxDim) return false;
  if (r > 0 && c > kMaxElems / r) return false;
  return true;
}

// Per-device cache of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_dev_ok[64];

puro_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return PURO_ERR_DEVICE;
  }
  if (dev < 64) {
    const int c = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return PURO_OK;
    if (c == 2) return PURO_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return PURO_ERR_DEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? PURO_OK : PURO_ERR_DEVICE;
}

puro_status launched(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return PURO_ERR_LAUNCH;
  }
  return PURO_OK;
}

}  // namespace

extern "C" {

int puro_abi_version(void) { return PURO_ABI_VERSION; }

const char *puro_status_str(puro_status s) {
  switch (s) {
    case PURO_OK: return "ok";
    case PURO_ERR_NULL: return "a required pointer is NULL";
    case PURO_ERR_SHAPE: return "invalid shape (negative, not a multiple of 16 where required, or over the limits)";
    case PURO_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case PURO_ERR_MODE: return "unknown GEMM mode or transpose kind";
    case PURO_ERR_DTYPE: return "unknown output dtype";
    case PURO_ERR_WORKSPACE: return "workspace missing or too small";
    case PURO_ERR_DEVICE: return "no current device, or the device is not gfx950";
    case PURO_ERR_LAUNCH: return "the HIP runtime failed to enqueue a kernel";
    case PURO_ERR_ALIAS: return "an output overlaps an input or another output";
    case PURO_ERR_SCRATCH: return "the shape's split-K plan needs more than the library's 64 MiB device scratch";
  }
  return "unknown status";
}

puro_status puro_quant_act_1x128(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q, float *s,
                                 puro_stream_t stream) {
  if (!shape_ok(rows, cols) || cols % 16 != 0) return PURO_ERR_SHAPE;
  if (rows == 0 || cols == 0) return PURO_OK;
  if (!x || !q || !s) return PURO_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return PURO_ERR_ALIGN;
  const Range in[] = {rng(x, rows * cols * 2)};
  const Range out[] = {rng(q, rows * cols), rng(s, cdiv(cols, 128) * rows * 4)};
  if (any_alias(in, 1, out, 2)) return PURO_ERR_ALIAS;
  if (puro_status d = check_device()) return d;
  return launched(puro::run_quant_act_1x128(x, rows, cols, q, s, (hipStream_t)stream));
}

puro_status puro_quant_w_128x128(const uint16_t *w, int64_t rows, int64_t cols, uint8_t *q, float *s,
                                 puro_stream_t stream) {
  if (!shape_ok(rows, cols) || cols % 16 != 0) return PURO_ERR_SHAPE;
  if (rows == 0 || cols == 0) return PURO_OK;
  if (!w || !q || !s) return PURO_ERR_NULL;
  if (!aligned16(w) || !aligned16(q) || !aligned16(s)) return PURO_ERR_ALIGN;
  const Range in[] = {rng(w, rows * cols * 2)};
  const Range out[] = {rng(q, rows * cols), rng(s, cdiv(rows, 128) * cdiv(cols, 128) * 4)};
  if (any_alias(in, 1, out, 2)) return PURO_ERR_ALIAS;
  if (puro_status d = check_device()) return d;
  return launched(puro::run_quant_w_128x128(w, rows, cols, q, s, (hipStream_t)stream));
}

puro_status puro_quant_transpose(puro_t_kind kind, const uint16_t *x, int64_t rows, int64_t cols,
                                 uint8_t *qt, float *st, uint8_t *q_row, float *s_row,
                                 puro_stream_t stream) {
  if (kind != PURO_T_ACT && kind != PURO_T_WEIGHT) return PURO_ERR_MODE;
  if (!shape_ok(rows, cols) || cols % 16 != 0 || rows % 16 != 0) return PURO_ERR_SHAPE;
  if ((q_row == nullptr) != (s_row == nullptr)) return PURO_ERR_NULL;
  if (rows == 0 || cols == 0) return PURO_OK;
  if (!x || !qt || !st) return PURO_ERR_NULL;
  const bool dual = q_row != nullptr;
  if (!aligned16(x) || !aligned16(qt) || !aligned16(st)) return PURO_ERR_ALIGN;
  if (dual && (!aligned16(q_row) || !aligned16(s_row))) return PURO_ERR_ALIGN;
  const int64_t ni = cdiv(rows, 128), nj = cdiv(cols, 128);
  const int64_t st_elems = kind == PURO_T_ACT ? ni * cols : nj * ni;
  const int64_t s_elems = kind == PURO_T_ACT ? nj * rows : ni * nj;
  const Range in[] = {rng(x, rows * cols * 2)};
  const Range out[] = {rng(qt, rows * cols), rng(st, st_elems * 4),
                       rng(q_row, dual ? rows * cols : 0), rng(s_row, dual ? s_elems * 4 : 0)};
  if (any_alias(in, 1, out, 4)) return PURO_ERR_ALIAS;
  if (puro_status d = check_device()) return d;
  if (kind == PURO_T_ACT)
    return launched(puro::run_quant_t_act(x, rows, cols, qt, st, q_row, s_row, (hipStream_t)stream));
  return launched(puro::run_quant_t_w(x, rows, cols, qt, st, q_row, s_row, (hipStream_t)stream));
}

puro_status puro_quant_weights(int count, const puro_weight *weights, puro_stream_t stream) {
  constexpr int kMax = 8;
  if (count < 0 || count > kMax) return PURO_ERR_SHAPE;
  if (count == 0) return PURO_OK;
  if (!weights) return PURO_ERR_NULL;
  for (int i = 0; i < count; ++i) {
    const puro_weight &w = weights[i];
    if (!shape_ok(w.rows, w.cols) || w.cols % 16 != 0 || (w.qt && w.rows % 16 != 0)) return PURO_ERR_SHAPE;
  }
  // entries with no elements write nothing: their pointers are not looked at
  int first = -1;
  for (int i = 0; i < count && first < 0; ++i)
    if (weights[i].rows > 0 && weights[i].cols > 0) first = i;
  if (first < 0) return PURO_OK;
  const bool row = weights[first].q != nullptr, tr = weights[first].qt != nullptr;
  for (int i = 0; i < count; ++i) {
    const puro_weight &w = weights[i];
    if (w.rows == 0 || w.cols == 0) continue;
    if ((w.q == nullptr) != (w.s == nullptr) || (w.qt == nullptr) != (w.st == nullptr)) return PURO_ERR_NULL;
    if ((w.q != nullptr) != row || (w.qt != nullptr) != tr || (!row && !tr)) return PURO_ERR_NULL;
    if (!w.w) return PURO_ERR_NULL;
  }
  Range in[kMax], out[4 * kMax];
  int nin = 0, nout = 0;
  for (int i = 0; i < count; ++i) {
    const puro_weight &w = weights[i];
    if (w.rows == 0 || w.cols == 0) continue;
    if (!aligned16(w.w) || (row && (!aligned16(w.q) || !aligned16(w.s))) ||
        (tr && (!aligned16(w.qt) || !aligned16(w.st))))
      return PURO_ERR_ALIGN;
    const int64_t blocks = cdiv(w.rows, 128) * cdiv(w.cols, 128);
    in[nin++] = rng(w.w, w.rows * w.cols * 2);
    out[nout++] = rng(w.q, row ? w.rows * w.cols : 0);
    out[nout++] = rng(w.s, row ? blocks * 4 : 0);
    out[nout++] = rng(w.qt, tr ? w.rows * w.cols : 0);
    out[nout++] = rng(w.st, tr ? blocks * 4 : 0);
  }
  if (any_alias(in, nin, out, nout)) return PURO_ERR_ALIAS;
  int64_t total = 0;
  for (int i = 0; i < count; ++i) total += cdiv(weights[i].rows, 128) * cdiv(weights[i].cols, 128);
  if (total > kMaxDim) return PURO_ERR_SHAPE;
  if (puro_status d = check_device()) return d;
  puro::WeightQuant wq[kMax];
  int n = 0;
  for (int i = 0; i < count; ++i)
    if (weights[i].rows > 0 && weights[i].cols > 0)
      wq[n++] = puro::WeightQuant{weights[i].w, weights[i].rows, weights[i].cols, weights[i].q, weights[i].s,
                                  weights[i].qt, weights[i].st};
  return launched(puro::run_quant_weights(n, wq, (hipStream_t)stream));
}

puro_status puro_quant_act_128x1(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qc, float *sc,
                                 uint8_t *q_row, float *s_row, puro_stream_t stream) {
  if (!shape_ok(rows, cols) || cols % 16 != 0) return PURO_ERR_SHAPE;
  if ((q_row == nullptr) != (s_row == nullptr)) return PURO_ERR_NULL;
  if (rows == 0 || cols == 0) return PURO_OK;
  if (!x || !qc || !sc) return PURO_ERR_NULL;
  const bool dual = q_row != nullptr;
  if (!aligned16(x) || !aligned16(qc) || !aligned16(sc)) return PURO_ERR_ALIGN;
  if (dual && (!aligned16(q_row) || !aligned16(s_row))) return PURO_ERR_ALIGN;
  const Range in[] = {rng(x, rows * cols * 2)};
  const Range out[] = {rng(qc, rows * cols), rng(sc, cdiv(rows, 128) * cols * 4),
                       rng(q_row, dual ? rows * cols : 0), rng(s_row, dual ? cdiv(cols, 128) * rows * 4 : 0)};
  if (any_alias(in, 1, out, 4)) return PURO_ERR_ALIAS;
  if (puro_status d = check_device()) return d;
  return launched(puro::run_quant_act_128x1(x, rows, cols, qc, sc, q_row, s_row, (hipStream_t)stream));
}

puro_status puro_swiglu_quant(const uint16_t *gu, int64_t rows, int64_t inter, uint8_t *q, float *s,
                              uint8_t *qt, float *st, uint16_t *h, puro_stream_t stream) {
  if (inter > kMaxDim / 2 || !shape_ok(rows, 2 * inter) || inter % 16 != 0) return PURO_ERR_SHAPE;
  if ((qt == nullptr) != (st == nullptr)) return PURO_ERR_NULL;
  const bool dual = qt != nullptr;
  if (dual && rows % 16 != 0) return PURO_ERR_SHAPE;
  if (rows == 0 || inter == 0) return PURO_OK;
  if (!gu || !q || !s) return PURO_ERR_NULL;
  if (!aligned16(gu) || !aligned16(q) || !aligned16(s)) return PURO_ERR_ALIGN;
  if (dual && (!aligned16(qt) || !aligned16(st))) return PURO_ERR_ALIGN;
  if (h && !aligned16(h)) return PURO_ERR_ALIGN;
  const Range in[] = {rng(gu, rows * inter * 4)};
  const Range out[] = {rng(q, rows * inter), rng(s, cdiv(inter, 128) * rows * 4),
                       rng(qt, dual ? rows * inter : 0), rng(st, dual ? cdiv(rows, 128) * inter * 4 : 0),
                       rng(h, h ? rows * inter * 2 : 0)};
  if (any_alias(in, 1, out, 5)) return PURO_ERR_ALIAS;
  if (puro_status d = check_device()) return d;
  return launched(puro::run_swiglu_quant(gu, rows, inter, q, s, qt, st, h, (hipStream_t)stream));
}

puro_status puro_requant_act_t(const uint8_t *q, const float *s, int64_t rows, int64_t cols,
                               uint8_t *qt, float *st, puro_stream_t stream) {
  if (!shape_ok(rows, cols) || cols % 16 != 0 || rows % 16 != 0) return PURO_ERR_SHAPE;
  if (rows == 0 || cols == 0) return PURO_OK;
  if (!q || !s || !qt || !st) return PURO_ERR_NULL;
  if (!aligned16(q) || !aligned16(s) || !aligned16(qt) || !aligned16(st)) return PURO_ERR_ALIGN;
  const Range in[] = {rng(q, rows * cols), rng(s, cdiv(cols, 128) * rows * 4)};
  const Range out[] = {rng(qt, rows * cols), rng(st, cdiv(rows, 128) * cols * 4)};
  if (any_alias(in, 2, out, 2)) return PURO_ERR_ALIAS;
  if (puro_status d = check_device()) return d;
  return launched(puro::run_requant_act_t(q, s, rows, cols, qt, st, (hipStream_t)stream));
}

size_t puro_gemm_workspace_bytes(puro_gemm_mode mode, int64_t M, int64_t N, int64_t K) {
  if (mode != PURO_FPROP && mode != PURO_DGRAD && mode != PURO_WGRAD && mode != PURO_WGRAD_TM) return 0;
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxGemmK) return 0;
  return puro::plan_gemm((int)mode, M, N, K).ws_bytes;
}

}  // extern "C"

namespace {

// noalloc: the split-K partials go to the library's scratch (workspace unused).
puro_status gemm_call(puro_gemm_mode mode, const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                      void *out, puro_out_dtype out_dtype, bool accumulate, int64_t M, int64_t N, int64_t K,
                      void *workspace, size_t workspace_bytes, puro_stream_t stream, bool noalloc = false) {
  if (mode != PURO_FPROP && mode != PURO_DGRAD && mode != PURO_WGRAD && mode != PURO_WGRAD_TM) return PURO_ERR_MODE;
  if (out_dtype != PURO_OUT_F32 && out_dtype != PURO_OUT_BF16) return PURO_ERR_DTYPE;
  if (!shape_ok(M, K) || !shape_ok(N, K) || !shape_ok(M, N) || K % 16 != 0 || K > kMaxGemmK)
    return PURO_ERR_SHAPE;
  if (mode == PURO_WGRAD_TM && (M % 16 != 0 || N % 16 != 0 || M >= (int64_t(1) << 30) || N >= (int64_t(1) << 30)))
    return PURO_ERR_SHAPE;   // 16-byte code rows; 4 rows of either operand index in 32 bits
  if (M == 0 || N == 0) return PURO_OK;
  if (!out) return PURO_ERR_NULL;
  const int64_t osz = out_dtype == PURO_OUT_F32 ? 4 : 2;
  puro::GemmPlan plan{};
  if (K > 0) {
    plan = puro::plan_gemm((int)mode, M, N, K);
    if ((int64_t)plan.tiles_m * plan.tiles_n * plan.splits > kMaxDim) return PURO_ERR_SHAPE;
    if (!a || !sa || !b || !sb) return PURO_ERR_NULL;
    if (noalloc) {
      if (plan.ws_bytes > puro::kScratchBytes) return PURO_ERR_SCRATCH;
      plan.ws_bytes = 0;                     // no caller workspace to check
    } else if (plan.ws_bytes > 0 && !workspace) {
      return PURO_ERR_WORKSPACE;
    }
  }
  if (!aligned16(out)) return PURO_ERR_ALIGN;
  if (K > 0) {
    if (!aligned16(a) || !aligned16(sa) || !aligned16(b) || !aligned16(sb)) return PURO_ERR_ALIGN;
    if (plan.ws_bytes > 0 && !aligned16(workspace)) return PURO_ERR_ALIGN;
    const int64_t nk = cdiv(K, 128);
    const int64_t sb_elems = mode == PURO_WGRAD || mode == PURO_WGRAD_TM ? nk * N : cdiv(N, 128) * nk;
    const Range in[] = {rng(a, M * K), rng(sa, nk * M * 4), rng(b, N * K), rng(sb, sb_elems * 4)};
    const Range outs[] = {rng(out, M * N * osz), rng(workspace, (int64_t)plan.ws_bytes)};
    if (any_alias(in, 4, outs, 2)) return PURO_ERR_ALIAS;
    if (plan.ws_bytes > 0 && workspace_bytes < plan.ws_bytes) return PURO_ERR_WORKSPACE;
  }
  if (puro_status d = check_device()) return d;
  if (noalloc)
    return launched(puro::run_gemm_noalloc((int)mode, a, sa, b, sb, out, out_dtype == PURO_OUT_BF16, M, N, K,
                                           (hipStream_t)stream));
  return launched(puro::run_gemm((int)mode, a, sa, b, sb, out, out_dtype == PURO_OUT_BF16, accumulate, M, N, K,
                                 workspace, (hipStream_t)stream));
}

}  // namespace

extern "C" {

puro_status puro_gemm_fp8_blockwise(puro_gemm_mode mode, const uint8_t *a, const float *sa,
                                    const uint8_t *b, const float *sb, void *out,
                                    puro_out_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                                    void *workspace, size_t workspace_bytes, puro_stream_t stream) {
  return gemm_call(mode, a, sa, b, sb, out, out_dtype, false, M, N, K, workspace, workspace_bytes, stream);
}

puro_status puro_gemm_fp8_blockwise_noalloc(puro_gemm_mode mode, const uint8_t *a, const float *sa,
                                            const uint8_t *b, const float *sb, void *out,
                                            puro_out_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                                            puro_stream_t stream) {
  return gemm_call(mode, a, sa, b, sb, out, out_dtype, false, M, N, K, nullptr, 0, stream, true);
}

puro_status puro_gemm_fp8_swiglu_quant(const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                                       int64_t M, int64_t inter, int64_t K, uint16_t *gu, uint8_t *hq, float *hs,
                                       puro_stream_t stream) {
  if (inter < 0 || inter > kMaxDim / 2 || inter % 128 != 0) return PURO_ERR_SHAPE;
  if (!shape_ok(M, K) || !shape_ok(2 * inter, K) || !shape_ok(M, 2 * inter) || K % 16 != 0 || K > kMaxGemmK)
    return PURO_ERR_SHAPE;
  if ((inter + 16) * K >= (int64_t(1) << 32)) return PURO_ERR_SHAPE;      // B row offsets in 32 bits
  if (cdiv(M, 256) * (inter / 128) > kMaxDim) return PURO_ERR_SHAPE;
  if (M == 0 || inter == 0) return PURO_OK;
  if (!hq || !hs) return PURO_ERR_NULL;
  if (K > 0 && (!a || !sa || !b || !sb)) return PURO_ERR_NULL;
  if (!aligned16(hq) || !aligned16(hs) || (gu && !aligned16(gu))) return PURO_ERR_ALIGN;
  if (K > 0 && (!aligned16(a) || !aligned16(sa) || !aligned16(b) || !aligned16(sb))) return PURO_ERR_ALIGN;
  const int64_t nk = cdiv(K, 128);
  const Range in[] = {rng(a, M * K), rng(sa, nk * M * 4), rng(b, 2 * inter * K), rng(sb, 2 * inter / 128 * nk * 4)};
  const Range outs[] = {rng(gu, gu ? M * 2 * inter * 2 : 0), rng(hq, M * inter), rng(hs, inter / 128 * M * 4)};
  if (any_alias(in, K > 0 ? 4 : 0, outs, 3)) return PURO_ERR_ALIAS;
  if (puro_status d = check_device()) return d;
  return launched(puro::run_gemm_swiglu_quant(a, sa, b, sb, gu, hq, hs, M, inter, K, (hipStream_t)stream));
}

puro_status puro_gemm_fp8_blockwise_accumulate(puro_gemm_mode mode, const uint8_t *a, const float *sa,
                                               const uint8_t *b, const float *sb, float *out,
                                               int64_t M, int64_t N, int64_t K,
                                               void *workspace, size_t workspace_bytes, puro_stream_t stream) {
  return gemm_call(mode, a, sa, b, sb, out, PURO_OUT_F32, true, M, N, K, workspace, workspace_bytes, stream);
}

}  // extern "C"
