/*
 * CPU oracle for blockwise FP8 quantization and the blockwise-scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source with the HIP library.
 *
 * What it computes.  The pages (en.roboind.com article on Puro-2B, section
 * "FP8 takes advantage of the RTX 5090's low precision efficiency") say that
 * the main linear layers run their matrix multiplications on an FP8 path that
 * follows DeepSeek-V3's fine-grained block quantization, while sensitive
 * operations and training state stay in BF16/FP32.  They give no formulas.
 * This library fixes the open points as follows (each a reading, listed in the
 * design notes):
 *   - format: OCP E4M3FN ("e4m3"): bias 7, largest finite 448, no infinities,
 *     S.1111.111 is NaN; subnormals are m * 2^-9 (OCP 8-bit floating point
 *     specification, E4M3 encoding table);
 *   - tiles: 1x128 along the contraction axis for activations, 128x128 for
 *     weights, 128x1 (a 1x128 tile of the transpose) for the wgrad operands;
 *   - scale: s = amax / 448 as an IEEE fp32 division; an all-zero tile gets
 *     s = 1;
 *   - codes: q = e4m3(fp32(x / s)), round to nearest even, saturating;
 *   - GEMM: out[m][n] = sum_k deq(a)[m][k] * deq(b)[n][k], where deq multiplies
 *     a decoded code by its tile scale.  Computed here in fp64.
 *   - a tile that runs past the end of a row (a ragged tail) covers only the
 *     elements that exist;
 *   - requantization of saved 1x128 codes (orc_requant_act_t): dequantize to
 *     fp32 with one rounding, then the 128x1 rule on the transpose;
 *   - SwiGLU of the MLP's gate/up output (orc_swiglu): bf16 of the fp64 value
 *     of silu(g) * u, gate in the first half of each row.
 *
 * Parity pins (independent checks of this file) live in the test-suite:
 * exhaustive agreement of the encoder with PyTorch's CPU float8_e4m3fn cast,
 * code round-trips, the tile invariants (|q| <= 448, all-zero tile -> scale 1,
 * exactly representable tiles round-trip, power-of-two equivariance), hand
 * derived golden tiles, integer-exact GEMMs against numpy int64, linearity of
 * the GEMM in power-of-two scales and a numpy fp64 cross-check; for the
 * requantizer a torch composition, reduction to the bf16 transposed
 * quantizer and closed forms; for SwiGLU 50-digit arithmetic.
 *
 * Plain C99 + OpenMP (loops over independent tiles / output rows only).
 * Build without fast-math and without FP contraction.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stddef.h>

#define TILE 128

uint16_t orc_f64_to_bf16(double v);

/* ------------------------------------------------------------------ */
/* bf16 and e4m3 scalars                                               */
/* ------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE fp32 word: widening is exact. */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Decode one OCP E4M3FN code (OCP OFP8 spec, E4M3 table).
 * exp field 0: subnormal m * 2^-9; exp field 1..15: (1 + m/8) * 2^(e-7);
 * 0x7F and 0xFF are NaN. */
double orc_e4m3_decode(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 7 - 3);
    return sign ? -v : v;
}

/* Encode an fp32 value as OCP E4M3FN, rounding to nearest with ties to even,
 * saturating every magnitude at or above the largest finite value (448) to
 * 448.  The sign of zero is kept (negative values that round to zero give
 * 0x80).  NaN gives 0x7F.
 *
 * The value set is the union of the subnormal lattice {m * 2^-9, m = 0..7}
 * and, for each exponent e in [-6, 8], the lattice {n * 2^(e-3), n = 8..15}.
 * Rounding is done on the integer n by nearbyint() in the default rounding
 * mode (round half to even).  All scalings are by powers of two in fp64, so
 * they are exact. */
uint8_t orc_e4m3_encode(float f)
{
    uint8_t sign;
    double a;
    if (isnan(f))
        return 0x7F;
    sign = signbit(f) ? 0x80 : 0x00;
    a = fabs((double)f);
    if (a >= 448.0)                     /* saturate */
        return (uint8_t)(sign | 0x7E);
    if (a < ldexp(1.0, -6)) {            /* subnormal range */
        double n = nearbyint(ldexp(a, 9));       /* 0..8; 8 is 2^-6 = code 0x08 */
        return (uint8_t)(sign | (uint8_t)n);
    } else {
        int ex;
        int e;
        double n;
        frexp(a, &ex);                   /* a = fr * 2^ex, fr in [0.5, 1) */
        e = ex - 1;                      /* floor(log2 a), in [-6, 8] */
        n = nearbyint(ldexp(a, 3 - e));  /* 8..16 */
        if (n == 16.0) {                 /* rounded up into the next binade */
            e += 1;
            n = 8.0;
        }
        if (e > 8 || (e == 8 && n > 14.0))   /* beyond 448: saturate (unreachable for a < 448) */
            return (uint8_t)(sign | 0x7E);
        return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | ((int)n - 8)));
    }
}

/* Tile scale from the tile's absolute maximum: s = amax / 448 in IEEE fp32,
 * or 1 for an all-zero tile. */
float orc_tile_scale(float amax)
{
    if (amax == 0.0f)
        return 1.0f;
    return amax / 448.0f;
}

/* One element's code given its tile scale: e4m3(fp32(x / s)). */
uint8_t orc_quantize_value(float x, float s)
{
    float v = x / s;
    return orc_e4m3_encode(v);
}

void orc_e4m3_encode_array(const float *x, int64_t n, uint8_t *q)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        q[i] = orc_e4m3_encode(x[i]);
}

/* ------------------------------------------------------------------ */
/* Quantizers                                                          */
/* ------------------------------------------------------------------ */

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* 1x128 activation tiles.
 * x: bf16 [R][C] row-major.  q: uint8 [R][C].  s: fp32 [ceil(C/128)][R]
 * (one scale per tile; tile (r, j) covers x[r][128j .. min(128j+128, C)-1]). */
void orc_quant_act_1x128(const uint16_t *x, int64_t R, int64_t C,
                         uint8_t *q, float *s)
{
    int64_t nj = ceil_div(C, TILE);
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < R; ++r) {
        int64_t j;
        for (j = 0; j < nj; ++j) {
            int64_t c0 = j * TILE, c1 = c0 + TILE < C ? c0 + TILE : C, c;
            float amax = 0.0f, sc;
            for (c = c0; c < c1; ++c) {
                float v = fabsf(orc_bf16_to_f32(x[r * C + c]));
                if (v > amax)
                    amax = v;
            }
            sc = orc_tile_scale(amax);
            s[j * R + r] = sc;
            for (c = c0; c < c1; ++c)
                q[r * C + c] = orc_quantize_value(orc_bf16_to_f32(x[r * C + c]), sc);
        }
    }
}

/* 128x128 weight blocks.
 * w: bf16 [R][C].  q: uint8 [R][C].  s: fp32 [ceil(R/128)][ceil(C/128)]. */
void orc_quant_w_128x128(const uint16_t *w, int64_t R, int64_t C,
                         uint8_t *q, float *s)
{
    int64_t ni = ceil_div(R, TILE), nj = ceil_div(C, TILE);
    int64_t blk;
#pragma omp parallel for schedule(static)
    for (blk = 0; blk < ni * nj; ++blk) {
        int64_t i = blk / nj, j = blk % nj;
        int64_t r0 = i * TILE, r1 = r0 + TILE < R ? r0 + TILE : R;
        int64_t c0 = j * TILE, c1 = c0 + TILE < C ? c0 + TILE : C;
        int64_t r, c;
        float amax = 0.0f, sc;
        for (r = r0; r < r1; ++r)
            for (c = c0; c < c1; ++c) {
                float v = fabsf(orc_bf16_to_f32(w[r * C + c]));
                if (v > amax)
                    amax = v;
            }
        sc = orc_tile_scale(amax);
        s[i * nj + j] = sc;
        for (r = r0; r < r1; ++r)
            for (c = c0; c < c1; ++c)
                q[r * C + c] = orc_quantize_value(orc_bf16_to_f32(w[r * C + c]), sc);
    }
}

/* 128x1 activation tiles (the transposed operand of wgrad).
 * x: bf16 [R][C].  Tile (i, c) covers x[128i .. min(128i+128, R)-1][c].
 * qt: uint8 [C][R] with qt[c][r] the code of x[r][c].
 * st: fp32 [ceil(R/128)][C] with st[i][c] the scale of tile (i, c). */
void orc_quant_act_128x1_t(const uint16_t *x, int64_t R, int64_t C,
                           uint8_t *qt, float *st)
{
    int64_t ni = ceil_div(R, TILE);
    int64_t c;
#pragma omp parallel for schedule(static)
    for (c = 0; c < C; ++c) {
        int64_t i;
        for (i = 0; i < ni; ++i) {
            int64_t r0 = i * TILE, r1 = r0 + TILE < R ? r0 + TILE : R, r;
            float amax = 0.0f, sc;
            for (r = r0; r < r1; ++r) {
                float v = fabsf(orc_bf16_to_f32(x[r * C + c]));
                if (v > amax)
                    amax = v;
            }
            sc = orc_tile_scale(amax);
            st[i * C + c] = sc;
            for (r = r0; r < r1; ++r)
                qt[c * R + r] = orc_quantize_value(orc_bf16_to_f32(x[r * C + c]), sc);
        }
    }
}

/* Transposed 128x128 weight blocks: the weight blocks of w, with codes and
 * block scales stored transposed.
 * w: bf16 [R][C].  qt: uint8 [C][R], qt[c][r] = code of w[r][c].
 * st: fp32 [ceil(C/128)][ceil(R/128)], st[j][i] = scale of block (i, j). */
void orc_quant_w_128x128_t(const uint16_t *w, int64_t R, int64_t C,
                           uint8_t *qt, float *st)
{
    int64_t ni = ceil_div(R, TILE), nj = ceil_div(C, TILE);
    int64_t blk;
#pragma omp parallel for schedule(static)
    for (blk = 0; blk < ni * nj; ++blk) {
        int64_t i = blk / nj, j = blk % nj;
        int64_t r0 = i * TILE, r1 = r0 + TILE < R ? r0 + TILE : R;
        int64_t c0 = j * TILE, c1 = c0 + TILE < C ? c0 + TILE : C;
        int64_t r, c;
        float amax = 0.0f, sc;
        for (r = r0; r < r1; ++r)
            for (c = c0; c < c1; ++c) {
                float v = fabsf(orc_bf16_to_f32(w[r * C + c]));
                if (v > amax)
                    amax = v;
            }
        sc = orc_tile_scale(amax);
        st[j * ni + i] = sc;
        for (r = r0; r < r1; ++r)
            for (c = c0; c < c1; ++c)
                qt[c * R + r] = orc_quantize_value(orc_bf16_to_f32(w[r * C + c]), sc);
    }
}

/* Requantize saved 1x128 activation codes into transposed 128x1 tiles (the
 * other reading of the backward's "transpose-requantize": the forward pass
 * keeps only the FP8 codes of an activation, and the wgrad operand is rebuilt
 * from them).  Two steps, applied literally:
 *   1. dequantize to fp32: d[r][c] = fp32(dec(q[r][c]) * s[c/128][r]) (the
 *      product is formed exactly and rounded once to fp32);
 *   2. quantize d with the 128x1 rule of orc_quant_act_128x1_t: per tile of
 *      128 rows of one column, st = amax/448 (1 if the tile is all zero) and
 *      qt = e4m3(fp32(d / st)).
 * q: uint8 [R][C] with scales s: fp32 [ceil(C/128)][R] (the output layout of
 * orc_quant_act_1x128).  qt: uint8 [C][R], qt[c][r] the new code of element
 * (r, c); st: fp32 [ceil(R/128)][C].  NaN codes (0x7F, 0xFF) are outside the
 * contract; the quantizers never emit them. */
static float deq_act_f32(uint8_t c, float s)
{
    return (float)(orc_e4m3_decode(c) * (double)s);
}

void orc_requant_act_t(const uint8_t *q, const float *s, int64_t R, int64_t C,
                       uint8_t *qt, float *st)
{
    int64_t ni = ceil_div(R, TILE);
    int64_t c;
#pragma omp parallel for schedule(static)
    for (c = 0; c < C; ++c) {
        int64_t i, j = c / TILE;
        for (i = 0; i < ni; ++i) {
            int64_t r0 = i * TILE, r1 = r0 + TILE < R ? r0 + TILE : R, r;
            float amax = 0.0f, sc;
            for (r = r0; r < r1; ++r) {
                float v = fabsf(deq_act_f32(q[r * C + c], s[j * R + r]));
                if (v > amax)
                    amax = v;
            }
            sc = orc_tile_scale(amax);
            st[i * C + c] = sc;
            for (r = r0; r < r1; ++r)
                qt[c * R + r] = orc_quantize_value(deq_act_f32(q[r * C + c], s[j * R + r]), sc);
        }
    }
}

/* SwiGLU of the gate/up projection output, rounded to bf16: the input of the
 * MLP down projection.  The pages (roboind) keep activations in BF16 around
 * the FP8 GEMMs; the model is Qwen3-shaped, whose MLP gates with SiLU.  With
 * gate g and up u (both bf16),
 *   h = bf16(silu(g) * u),  silu(g) = g / (1 + exp(-g)),
 * evaluated in fp64 in that order (libm exp) and rounded once, to nearest
 * even, to bf16.  That is the correctly rounded bf16 of the exact value
 * except where the exact value lies within ~2^-50 (relative) of a bf16
 * rounding midpoint; there the fp64 value decides.  Two systematic such
 * classes: |g| < 2^-52, where fp64 gives silu(g) = g/2 exactly although the
 * exact value is larger by about g^2/4, and g > 37, where fp64 gives
 * silu(g) = g exactly although the exact value is smaller by about g e^-g;
 * a g*u/2 (or g*u) on a midpoint then rounds to even instead of to the side
 * the exact value lies on.
 * gu: bf16 [R][2*I]; gate = gu[r][c], up = gu[r][I + c] for c < I (the
 * first half of each row is the gate, the second the up projection).
 * h: bf16 [R][I].  The 1x128 / 128x1 codes of h are those of
 * orc_quant_act_1x128 / orc_quant_act_128x1_t applied to h. */
uint16_t orc_swiglu_value(uint16_t g, uint16_t u)
{
    double gd = (double)orc_bf16_to_f32(g);
    double ud = (double)orc_bf16_to_f32(u);
    double silu = gd / (1.0 + exp(-gd));
    return orc_f64_to_bf16(silu * ud);
}

void orc_swiglu(const uint16_t *gu, int64_t R, int64_t I, uint16_t *h)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < R; ++r) {
        int64_t c;
        for (c = 0; c < I; ++c)
            h[r * I + c] = orc_swiglu_value(gu[r * 2 * I + c], gu[r * 2 * I + I + c]);
    }
}

/* ------------------------------------------------------------------ */
/* GEMM                                                                */
/* ------------------------------------------------------------------ */

/* Modes.  In every mode out[m][n] = sum_k A[m][k] * B[n][k] with
 *   A[m][k] = dec(a[m][k]) * sa[k/128][m]                   (a: [M][K], sa: [ceil(K/128)][M])
 * and for B (b: [N][K]):
 *   BLOCK_SCALED_B (fprop, dgrad): B[n][k] = dec(b[n][k]) * sb[n/128][k/128],  sb: [ceil(N/128)][ceil(K/128)]
 *   ROW_SCALED_B   (wgrad):        B[n][k] = dec(b[n][k]) * sb[k/128][n],      sb: [ceil(K/128)][N]     */
enum { ORC_FPROP = 0, ORC_DGRAD = 1, ORC_WGRAD = 2 };

static double deq_a(const uint8_t *a, const float *sa, int64_t M, int64_t K,
                    int64_t m, int64_t k)
{
    return orc_e4m3_decode(a[m * K + k]) * (double)sa[(k / TILE) * M + m];
}

static double deq_b(int mode, const uint8_t *b, const float *sb, int64_t N,
                    int64_t K, int64_t n, int64_t k)
{
    double sc;
    if (mode == ORC_WGRAD)
        sc = (double)sb[(k / TILE) * N + n];
    else
        sc = (double)sb[(n / TILE) * ceil_div(K, TILE) + k / TILE];
    return orc_e4m3_decode(b[n * K + k]) * sc;
}

/* One output element: the fp64 dot product of the dequantized row m of A and
 * row n of B, summed in increasing k. */
double orc_gemm_element(int mode, const uint8_t *a, const float *sa,
                        const uint8_t *b, const float *sb,
                        int64_t M, int64_t N, int64_t K, int64_t m, int64_t n)
{
    double acc = 0.0;
    int64_t k;
    for (k = 0; k < K; ++k)
        acc += deq_a(a, sa, M, K, m, k) * deq_b(mode, b, sb, N, K, n, k);
    return acc;
}

/* Full reference output out[M][N] in fp64. */
void orc_gemm(int mode, const uint8_t *a, const float *sa,
              const uint8_t *b, const float *sb,
              int64_t M, int64_t N, int64_t K, double *out)
{
    int64_t m;
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        int64_t n;
        for (n = 0; n < N; ++n)
            out[m * N + n] = orc_gemm_element(mode, a, sa, b, sb, M, N, K, m, n);
    }
}

/* Reference values at a list of (m, n) positions. */
void orc_gemm_at(int mode, const uint8_t *a, const float *sa,
                 const uint8_t *b, const float *sb,
                 int64_t M, int64_t N, int64_t K,
                 const int64_t *ms, const int64_t *ns, int64_t count, double *out)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i)
        out[i] = orc_gemm_element(mode, a, sa, b, sb, M, N, K, ms[i], ns[i]);
}

/* L2 norms of the dequantized rows: na[m] = ||A[m][:]||, nb[n] = ||B[n][:]||.
 * The GEMM tolerance is stated relative to na[m] * nb[n]. */
void orc_deq_row_norms(int mode, const uint8_t *a, const float *sa,
                       const uint8_t *b, const float *sb,
                       int64_t M, int64_t N, int64_t K, double *na, double *nb)
{
    int64_t m, n;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        double acc = 0.0;
        int64_t k;
        for (k = 0; k < K; ++k) {
            double v = deq_a(a, sa, M, K, m, k);
            acc += v * v;
        }
        na[m] = sqrt(acc);
    }
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        double acc = 0.0;
        int64_t k;
        for (k = 0; k < K; ++k) {
            double v = deq_b(mode, b, sb, N, K, n, k);
            acc += v * v;
        }
        nb[n] = sqrt(acc);
    }
}

/* Dequantize a whole operand to fp64 (used by the cross-checks that hand the
 * dequantized matrices to a library matmul). */
void orc_dequant_a(const uint8_t *a, const float *sa, int64_t M, int64_t K, double *out)
{
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        int64_t k;
        for (k = 0; k < K; ++k)
            out[m * K + k] = deq_a(a, sa, M, K, m, k);
    }
}

void orc_dequant_b(int mode, const uint8_t *b, const float *sb, int64_t N, int64_t K,
                   double *out)
{
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        int64_t k;
        for (k = 0; k < K; ++k)
            out[n * K + k] = deq_b(mode, b, sb, N, K, n, k);
    }
}

/* Round an fp64 value to bf16 (round to nearest, ties to even) directly,
 * without passing through fp32 (which would round twice).  Returns the bf16
 * bit pattern.  bf16 has 8 significant bits and fp32's exponent range,
 * subnormals included; finite values above the largest bf16 round to
 * infinity as IEEE rounding does. */
uint16_t orc_f64_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    int ex, e;
    double n;
    if (isnan(v))
        return 0x7FC0;
    if (a == 0.0)
        return sign;
    if (a < ldexp(1.0, -126)) {               /* subnormal: multiples of 2^-133 */
        n = nearbyint(ldexp(a, 133));         /* 0..128; 128 = 2^-126 = min normal */
        return (uint16_t)(sign | (uint16_t)n);
    }
    frexp(a, &ex);
    e = ex - 1;                               /* floor(log2 a) */
    n = nearbyint(ldexp(a, 7 - e));           /* 128..256 */
    if (n == 256.0) {
        e += 1;
        n = 128.0;
    }
    if (e > 127)
        return (uint16_t)(sign | 0x7F80);     /* overflow to infinity */
    return (uint16_t)(sign | (uint16_t)(((e + 127) << 7) | ((int)n - 128)));
}

void orc_f64_to_bf16_array(const double *v, int64_t n, uint16_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = orc_f64_to_bf16(v[i]);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
