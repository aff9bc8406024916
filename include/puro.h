/*
 * puro.h -- C ABI of the blockwise-FP8 quantizers and the blockwise-scaled
 * FP8 GEMM for AMD Instinct MI355X (gfx950).
 *
 * What the calls compute.  The pages on Puro-2B (en.roboind.com article,
 * section "FP8 takes advantage of the RTX 5090's low precision efficiency")
 * put the matrix multiplications of the main linear layers on an FP8 path
 * that follows DeepSeek-V3's fine-grained block quantization, and keep the
 * numerically sensitive operations and the training state in BF16/FP32; the
 * ainews.surl.tw article adds that training uses blockwise FP8 to cut compute
 * and memory.  The pages give no formulas; this library fixes them as:
 *
 *   tile scale   s = amax / 448 (IEEE fp32 division), s = 1 for an all-zero tile
 *   code         q = e4m3(fp32(x / s)): OCP E4M3FN, round to nearest even,
 *                saturating at +-448; -0 and negative values that round to zero
 *                give 0x80
 *   1x128 tile   128 consecutive elements of one row (activations)
 *   128x128 tile 128 rows x 128 columns (weights)
 *   128x1 tile   128 consecutive rows of one column (the transposed wgrad
 *                operands, quantized from the bf16 original)
 *   GEMM         out[m][n] = sum_k deq(a)[m][k] * deq(b)[n][k], with each
 *                128-deep slice of k summed in fp32 and added into an fp32
 *                accumulator after multiplying by the slice's two scales.
 *
 * Ragged shapes.  A row length that is not a multiple of 128 leaves a short
 * last tile that covers only the elements that exist.  Row lengths (the
 * contraction extent of every code tensor) must be multiples of 16; row
 * counts are free.  Sizes of 0 are allowed and enqueue nothing (a GEMM with
 * K = 0 writes zeros).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers, row-major, densely packed, and
 *     16-byte aligned.  bf16 tensors are passed as uint16_t bit patterns.
 *   - The caller allocates and frees every buffer (the library never allocates
 *     device memory), keeps them alive until the stream has passed the call,
 *     and must not let any output overlap any input or another output.
 *   - Every call validates its arguments on the host first.  On any error it
 *     enqueues nothing, touches no output and returns the error code.  Launch
 *     failures return PURO_ERR_LAUNCH.  No exception or abort crosses the ABI.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     and the call returns without waiting for it.
 *   - Inputs must be finite; non-finite inputs are outside the contract.
 *   - Calls are thread-safe and keep no per-call state.
 *   - Limits: every dimension < 2^31 and every tensor < 2^40 elements
 *     (PURO_ERR_SHAPE otherwise).
 */
#ifndef PURO_H
#define PURO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PURO_ABI_VERSION 8

/* Device scratch of puro_gemm_fp8_blockwise_noalloc, per GPU. */
#define PURO_SCRATCH_BYTES (64ull << 20)

typedef struct ihipStream_t *puro_stream_t;   /* = hipStream_t */

typedef enum {
    PURO_OK = 0,
    PURO_ERR_NULL = 1,        /* a required pointer is NULL */
    PURO_ERR_SHAPE = 2,       /* negative size, row length not a multiple of 16, or over the limits */
    PURO_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    PURO_ERR_MODE = 4,        /* unknown GEMM mode or transpose kind */
    PURO_ERR_DTYPE = 5,       /* unknown output dtype */
    PURO_ERR_WORKSPACE = 6,   /* workspace missing or smaller than puro_gemm_workspace_bytes() */
    PURO_ERR_DEVICE = 7,      /* the current device is not gfx950, or no device */
    PURO_ERR_LAUNCH = 8,      /* the HIP runtime reported an error while enqueueing */
    PURO_ERR_ALIAS = 9,       /* an output overlaps an input or another output */
    PURO_ERR_SCRATCH = 10     /* puro_gemm_fp8_blockwise_noalloc: the shape needs more split-K
                                 scratch than the library holds (PURO_SCRATCH_BYTES) */
} puro_status;

typedef enum {
    PURO_FPROP = 0,   /* Y  = X  W^T : a = act codes of X  [T][K_in],      b = weight codes of W [N_out][K_in] */
    PURO_DGRAD = 1,   /* dX = dY W   : a = act codes of dY [T][N_out],     b = transposed weight codes [K_in][N_out] */
    PURO_WGRAD = 2,   /* dW = dY^T X : a = 128x1 codes of dY [N_out][T],   b = 128x1 codes of X [K_in][T] */
    PURO_WGRAD_TM = 3 /* dW = dY^T X from token-major codes: a = 128x1 codes of dY [T][N_out],
                         b = 128x1 codes of X [T][K_in], as puro_quant_act_128x1 writes them */
} puro_gemm_mode;

typedef enum { PURO_OUT_F32 = 0, PURO_OUT_BF16 = 1 } puro_out_dtype;

typedef enum { PURO_T_ACT = 0, PURO_T_WEIGHT = 1 } puro_t_kind;

/*
 * puro_quant_act_1x128 -- activation quantization, one scale per 1x128 tile.
 *   x     [rows][cols] bf16 (input)
 *   q     [rows][cols] uint8 e4m3 codes (output)
 *   s     [ceil(cols/128)][rows] fp32 (output): s[j][r] is the scale of the
 *         tile x[r][128j .. min(128j+128, cols)-1]
 * cols must be a multiple of 16.
 */
puro_status puro_quant_act_1x128(const uint16_t *x, int64_t rows, int64_t cols,
                                 uint8_t *q, float *s, puro_stream_t stream);

/*
 * puro_quant_w_128x128 -- weight quantization, one scale per 128x128 block.
 *   w     [rows][cols] bf16 (input)
 *   q     [rows][cols] uint8 codes (output)
 *   s     [ceil(rows/128)][ceil(cols/128)] fp32 (output), block (i, j) covers
 *         rows 128i.. and columns 128j.. (short at a ragged edge)
 * cols must be a multiple of 16.
 */
puro_status puro_quant_w_128x128(const uint16_t *w, int64_t rows, int64_t cols,
                                 uint8_t *q, float *s, puro_stream_t stream);

/*
 * puro_quant_transpose -- transposed (re)quantization for the backward pass,
 * from the bf16 original, in one read of x.
 *   kind == PURO_T_ACT: 128x1 tiles (128 consecutive rows of one column).
 *     qt [cols][rows] uint8: qt[c][r] is the code of x[r][c]
 *     st [ceil(rows/128)][cols] fp32: st[i][c] is the scale of x[128i..][c]
 *     q_row, s_row (optional, both NULL or both set): the same pass also
 *       writes exactly what puro_quant_act_1x128(x) writes.
 *   kind == PURO_T_WEIGHT: 128x128 blocks, stored transposed.
 *     qt [cols][rows] uint8: the transpose of puro_quant_w_128x128's codes
 *     st [ceil(cols/128)][ceil(rows/128)] fp32: st[j][i] = scale of block (i, j)
 *     q_row, s_row (optional): exactly what puro_quant_w_128x128(x) writes.
 * Both rows and cols must be multiples of 16.
 */
puro_status puro_quant_transpose(puro_t_kind kind, const uint16_t *x, int64_t rows, int64_t cols,
                                 uint8_t *qt, float *st, uint8_t *q_row, float *s_row,
                                 puro_stream_t stream);

/*
 * puro_quant_weights -- several weights quantized in 128x128 blocks by one
 * launch.  Each entry gets exactly what puro_quant_w_128x128 (q, s) and
 * puro_quant_transpose(PURO_T_WEIGHT) (qt, st) write for it; a training step
 * quantizes all of a layer's weights at once, and one launch over all of them
 * keeps the chip busy where a small weight alone would not.
 *   count    0 .. 8 entries (0 enqueues nothing)
 *   weights  [count] descriptors (host memory, read during the call only):
 *     w            bf16 [rows][cols] (input)
 *     q, s         [rows][cols] codes, [ceil(rows/128)][ceil(cols/128)] scales,
 *                  or both NULL
 *     qt, st       [cols][rows] transposed codes, [ceil(cols/128)][ceil(rows/128)]
 *                  scales, or both NULL
 *   Every entry must request the same outputs (q, s and/or qt, st; at least
 *   one pair).  cols must be a multiple of 16, and rows too when qt is
 *   requested.  No output may overlap any input or output of any entry.  An
 *   entry with rows or cols 0 writes nothing and its pointers are not used.
 */
typedef struct {
    const uint16_t *w;
    int64_t rows, cols;
    uint8_t *q;
    float *s;
    uint8_t *qt;
    float *st;
} puro_weight;

puro_status puro_quant_weights(int count, const puro_weight *weights, puro_stream_t stream);

/*
 * puro_quant_act_128x1 -- the 128x1 tiles of puro_quant_transpose(PURO_T_ACT)
 * (128 consecutive rows of one column share a scale), with the codes left in
 * x's own layout instead of transposed: the wgrad operand in the token-major
 * form that puro_gemm_fp8_blockwise(PURO_WGRAD_TM) reads.  Writing the codes
 * untransposed keeps every store a row segment.
 *   qc [rows][cols] uint8: qc[r][c] = the 128x1 code of x[r][c]
 *      (= qt[c][r] of puro_quant_transpose(PURO_T_ACT))
 *   sc [ceil(rows/128)][cols] fp32: sc[i][c] is the scale of x[128i..][c]
 *   q_row, s_row (optional, both NULL or both set): the same pass also writes
 *      exactly what puro_quant_act_1x128(x) writes.
 * cols must be a multiple of 16; rows is free.
 */
puro_status puro_quant_act_128x1(const uint16_t *x, int64_t rows, int64_t cols,
                                 uint8_t *qc, float *sc, uint8_t *q_row, float *s_row,
                                 puro_stream_t stream);

/*
 * puro_requant_act_t -- transposed 128x1 codes rebuilt from saved 1x128 codes
 * (for a backward pass that kept only the FP8 copy of an activation).  Where
 * puro_quant_transpose quantizes the bf16 original along the other axis, this
 * call dequantizes each saved code and quantizes the result again in 128x1
 * tiles:
 *   d[r][c]  = fp32(dec(q[r][c]) * s[c/128][r])      (exact product, one rounding)
 *   st[i][c] = amax over rows 128i.. of |d[.][c]| / 448 (1 for an all-zero tile)
 *   qt[c][r] = e4m3(fp32(d[r][c] / st[r/128][c]))    (IEEE division)
 *   q    [rows][cols] uint8 codes (input), as puro_quant_act_1x128 writes them
 *   s    [ceil(cols/128)][rows] fp32 scales (input), as puro_quant_act_1x128
 *        writes them; every scale must be a positive normal fp32 value
 *        (>= 2^-126), which the quantizer gives for every tile whose maximum is
 *        0 or at least 2^-117; smaller scales and NaN codes are outside the
 *        contract (not detected)
 *   qt   [cols][rows] uint8 (output), st [ceil(rows/128)][cols] fp32 (output),
 *        laid out as puro_quant_transpose(PURO_T_ACT) writes them
 * Both rows and cols must be multiples of 16.  The result differs from
 * quantizing the bf16 original (two roundings instead of one); it is what a
 * pass that saved only q and s can compute.
 */
puro_status puro_requant_act_t(const uint8_t *q, const float *s, int64_t rows, int64_t cols,
                               uint8_t *qt, float *st, puro_stream_t stream);

/*
 * puro_swiglu_quant -- SwiGLU of the MLP's gate/up projection output fused
 * with the quantization of the result, the down projection's input.  The
 * pages train a Qwen3-shaped model with BF16 activations around FP8 GEMMs
 * (en.roboind.com article on Puro-2B, section "FP8 takes advantage of the RTX
 * 5090's low precision efficiency"); its MLP gates with SiLU.  Per element,
 *   h[r][c] = bf16(silu(g) * u),  g = gu[r][c], u = gu[r][inter + c],
 *   silu(g) = g / (1 + e^-g), the value being that of the expression
 *   evaluated in fp64, rounded once to bf16 (to nearest even),
 * and h is quantized exactly as puro_quant_act_1x128 (and, optionally, the
 * transposed 128x1 form of puro_quant_transpose(PURO_T_ACT)) would quantize
 * it, without h passing through memory.
 *   gu   [rows][2*inter] bf16 (input): gate in the first inter columns of a
 *        row, up in the last inter (the halves of a fused gate/up weight)
 *   q, s [rows][inter] codes, [ceil(inter/128)][rows] scales (outputs)
 *   qt, st (optional, both NULL or both set): [inter][rows] codes and
 *        [ceil(rows/128)][inter] scales of the 128x1 tiles of h (the down
 *        projection's wgrad operand)
 *   h    (optional, NULL to skip): [rows][inter] bf16, the SwiGLU values
 * inter must be a multiple of 16, and rows too when qt is requested.  Inputs
 * must be finite with every |silu(g) u| below 2^127.
 */
puro_status puro_swiglu_quant(const uint16_t *gu, int64_t rows, int64_t inter,
                              uint8_t *q, float *s, uint8_t *qt, float *st, uint16_t *h,
                              puro_stream_t stream);

/*
 * puro_gemm_workspace_bytes -- device workspace that puro_gemm_fp8_blockwise
 * needs for this mode and shape (0 when none).  Deterministic: the same
 * arguments always give the same size and the same split of the K loop.
 */
size_t puro_gemm_workspace_bytes(puro_gemm_mode mode, int64_t M, int64_t N, int64_t K);

/*
 * puro_gemm_fp8_blockwise -- blockwise-scaled FP8 GEMM.
 *   out[m][n] = sum_k (dec(a[m][k]) * sa[k/128][m]) * (dec(b[n][k]) * sb(n, k))
 *   a    [M][K] uint8 codes,  sa [ceil(K/128)][M] fp32
 *   b    [N][K] uint8 codes
 *   sb   FPROP/DGRAD: [ceil(N/128)][ceil(K/128)] fp32, sb(n, k) = sb[n/128][k/128]
 *        WGRAD:       [ceil(K/128)][N] fp32,            sb(n, k) = sb[k/128][n]
 *   out  [M][N] fp32 or bf16 (round to nearest even)
 * PURO_WGRAD_TM takes the operands token-major instead: a [K][M] and b [K][N]
 * with a[k][m] and b[k][n] in place of a[m][k] and b[n][k] above, scales as
 * for PURO_WGRAD; M and N must then be multiples of 16.  It gives exactly the
 * bits PURO_WGRAD gives for the transposed operands.
 *   workspace / workspace_bytes: at least puro_gemm_workspace_bytes(mode, M, N, K)
 *        bytes of device memory (may be NULL when that is 0); its contents on
 *        entry do not matter.
 * K must be a multiple of 16; M and N are free.  Each 128-deep slice of K is
 * accumulated by the matrix cores in fp32 and promoted into the fp32
 * accumulator with its scales, acc += P * fp32(sA * sB); the result is
 * deterministic for a given shape.  Domain: every product sA * sB that a slice
 * uses must be a normal fp32 value (2^-126 .. 2^128).  Outside it the product
 * underflows or overflows (not detected); scales from the quantizers leave it
 * only when the product of the two tiles' maxima is below ~2^-108 (both below
 * ~2^-54) or above ~2^145.
 */
puro_status puro_gemm_fp8_blockwise(puro_gemm_mode mode,
                                    const uint8_t *a, const float *sa,
                                    const uint8_t *b, const float *sb,
                                    void *out, puro_out_dtype out_dtype,
                                    int64_t M, int64_t N, int64_t K,
                                    void *workspace, size_t workspace_bytes,
                                    puro_stream_t stream);

/*
 * puro_gemm_fp8_blockwise_noalloc -- puro_gemm_fp8_blockwise without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  It allocates nothing: the split-K partials that a shape's plan
 * needs go to a device scratch array the library holds, PURO_SCRATCH_BYTES
 * (64 MiB) per GPU, from the first call on a device until the process ends.
 * Same arguments, results and errors as puro_gemm_fp8_blockwise with the same
 * shape (the same plan and kernels: the output is bit for bit the same), plus:
 *   PURO_ERR_SCRATCH  the shape's plan needs more than PURO_SCRATCH_BYTES of
 *                     partials (puro_gemm_workspace_bytes(mode, M, N, K) tells
 *                     how much); every GEMM of the layer at 16384 tokens fits.
 * Every call on one GPU uses that GPU's single scratch array: calls that can
 * run at the same time on one GPU (other streams, other host threads) race and
 * must be serialized by the caller.  The scratch needs no clearing: every
 * partial is written before it is read.
 */
puro_status puro_gemm_fp8_blockwise_noalloc(puro_gemm_mode mode,
                                            const uint8_t *a, const float *sa,
                                            const uint8_t *b, const float *sb,
                                            void *out, puro_out_dtype out_dtype,
                                            int64_t M, int64_t N, int64_t K,
                                            puro_stream_t stream);

/*
 * puro_gemm_fp8_blockwise_accumulate -- the same GEMM, added into an fp32
 * output: out[m][n] = fp32(out[m][n] + G[m][n]), where G is exactly the value
 * puro_gemm_fp8_blockwise computes with PURO_OUT_F32 (one fp32 addition per
 * element).  For micro-batched training, whose weight gradients are summed
 * over the micro-batches of a step into one fp32 buffer (the pages tune
 * micro-batch sizes per pipeline stage: en.roboind.com article on Puro-2B,
 * section "Unit cost, higher computing power").  Arguments as for
 * puro_gemm_fp8_blockwise; out [M][N] fp32 is read and written and must not
 * overlap any operand or the workspace.  K = 0 leaves out unchanged.
 */
puro_status puro_gemm_fp8_blockwise_accumulate(puro_gemm_mode mode,
                                               const uint8_t *a, const float *sa,
                                               const uint8_t *b, const float *sb,
                                               float *out, int64_t M, int64_t N, int64_t K,
                                               void *workspace, size_t workspace_bytes,
                                               puro_stream_t stream);

/*
 * puro_gemm_fp8_swiglu_quant -- the fprop of the MLP's fused gate/up
 * projection with puro_swiglu_quant as its epilogue: the down projection's
 * 1x128 FP8 input is written straight from the GEMM's accumulators (the
 * SwiGLU MLP and the FP8 main linears as in puro_swiglu_quant; the 1x128
 * rule of puro_quant_act_1x128).  hq and hs are bit for bit what
 *   puro_swiglu_quant(gu, M, inter, hq, hs, NULL, NULL, NULL)
 * makes of this call's own gu, without gu passing through memory on the way
 * to h; gu is bit for bit what
 *   puro_gemm_fp8_blockwise(PURO_FPROP, a, sa, b, sb, gu, PURO_OUT_BF16, M, 2*inter, K)
 * writes whenever that call needs no workspace (no split of its K loop, as
 * for every layer shape at 16384 tokens), and within the same tolerance of
 * the exact product otherwise (the split sums in another order).
 *   a    [M][K] uint8 codes, sa [ceil(K/128)][M] fp32 (1x128 activation codes)
 *   b    [2*inter][K] uint8 codes, sb [2*inter/128][ceil(K/128)] fp32 (128x128
 *        weight codes): gate rows first, then up rows
 *   gu   (optional, NULL to skip) [M][2*inter] bf16: the gate/up output that
 *        the fprop alone would write (the SwiGLU backward needs it)
 *   hq   [M][inter] uint8, hs [inter/128][M] fp32: 1x128 codes and scales of
 *        h = bf16(silu(g) u) (output)
 * inter must be a multiple of 128 and K of 16, with (inter + 16) * K < 2^32;
 * M is free.  K = 0 gives g = u = 0: h = 0, codes 0, scales 1.  No workspace
 * (no split of the K loop).  The result is deterministic for a given shape.
 */
puro_status puro_gemm_fp8_swiglu_quant(const uint8_t *a, const float *sa,
                                       const uint8_t *b, const float *sb,
                                       int64_t M, int64_t inter, int64_t K,
                                       uint16_t *gu, uint8_t *hq, float *hs,
                                       puro_stream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *puro_status_str(puro_status s);

/* PURO_ABI_VERSION of the built library. */
int puro_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PURO_H */
