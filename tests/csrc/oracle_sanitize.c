/*
 * Drives every function of the oracle (oracle/oracle.c) on ragged shapes, with
 * each buffer allocated at exactly the size its layout needs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests only).  An access past
 * a buffer or undefined arithmetic stops the program with a sanitizer report.
 * It also checks two identities that need no second implementation: the 128x1
 * transposed quantizer equals the 1x128 quantizer of the materialized
 * transpose, and the transposed weight quantizer equals the transpose of the
 * plain one.  Exit status 0 when every shape passes.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint8_t orc_e4m3_encode(float f);
void orc_e4m3_encode_array(const float *x, int64_t n, uint8_t *q);
void orc_quant_act_1x128(const uint16_t *x, int64_t R, int64_t C, uint8_t *q, float *s);
void orc_quant_w_128x128(const uint16_t *w, int64_t R, int64_t C, uint8_t *q, float *s);
void orc_quant_act_128x1_t(const uint16_t *x, int64_t R, int64_t C, uint8_t *qt, float *st);
void orc_quant_w_128x128_t(const uint16_t *w, int64_t R, int64_t C, uint8_t *qt, float *st);
void orc_requant_act_t(const uint8_t *q, const float *s, int64_t R, int64_t C, uint8_t *qt, float *st);
void orc_swiglu(const uint16_t *gu, int64_t R, int64_t I, uint16_t *h);
void orc_gemm(int mode, const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
              int64_t M, int64_t N, int64_t K, double *out);
void orc_gemm_at(int mode, const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                 int64_t M, int64_t N, int64_t K, const int64_t *ms, const int64_t *ns, int64_t count, double *out);
void orc_deq_row_norms(int mode, const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                       int64_t M, int64_t N, int64_t K, double *na, double *nb);
void orc_dequant_a(const uint8_t *a, const float *sa, int64_t M, int64_t K, double *out);
void orc_dequant_b(int mode, const uint8_t *b, const float *sb, int64_t N, int64_t K, double *out);
void orc_f64_to_bf16_array(const double *v, int64_t n, uint16_t *out);

static uint64_t st = 88172645463325252ull;
static uint32_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (uint32_t)st; }
static int64_t cd(int64_t a, int64_t b) { return (a + b - 1) / b; }
static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); if (!p) { perror("malloc"); exit(2); } return p; }

/* finite bf16 bit patterns, a few tiles zero */
static uint16_t *bf16_input(int64_t n)
{
    uint16_t *x = xmalloc((size_t)n * 2);
    for (int64_t i = 0; i < n; ++i) {
        uint16_t h = (uint16_t)rnd();
        if ((h & 0x7f80) == 0x7f80) h &= 0xbfff;     /* no Inf / NaN */
        x[i] = (i % 977) < 130 ? (uint16_t)(h & 0x8000) : h;
    }
    return x;
}

static uint8_t *code_input(int64_t n)
{
    uint8_t *c = xmalloc((size_t)n);
    for (int64_t i = 0; i < n; ++i) { uint8_t v = (uint8_t)rnd(); c[i] = (v & 0x7f) == 0x7f ? (uint8_t)(v & 0xf0) : v; }
    return c;
}

static float *scale_input(int64_t n)
{
    float *s = xmalloc((size_t)n * 4);
    for (int64_t i = 0; i < n; ++i) s[i] = (float)(1 + rnd() % 1000) * 1e-3f;
    return s;
}

static int fail(const char *what, int64_t R, int64_t C)
{
    fprintf(stderr, "%s differs at %lld x %lld\n", what, (long long)R, (long long)C);
    return 1;
}

static int quantizers(int64_t R, int64_t C)
{
    int bad = 0;
    uint16_t *x = bf16_input(R * C), *xt = xmalloc((size_t)(R * C) * 2);
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) xt[c * R + r] = x[r * C + c];
    uint8_t *q = xmalloc((size_t)(R * C)), *qt = xmalloc((size_t)(R * C)), *q2 = xmalloc((size_t)(R * C));
    float *s = xmalloc((size_t)(cd(C, 128) * R) * 4), *stt = xmalloc((size_t)(cd(R, 128) * C) * 4);
    float *s2 = xmalloc((size_t)(cd(R, 128) * C) * 4);
    orc_quant_act_1x128(x, R, C, q, s);
    orc_quant_act_128x1_t(x, R, C, qt, stt);
    orc_quant_act_1x128(xt, C, R, q2, s2);          /* the same tiles, on the transpose */
    if (memcmp(qt, q2, (size_t)(R * C)) || memcmp(stt, s2, (size_t)(cd(R, 128) * C) * 4)) bad |= fail("128x1 tiles", R, C);
    if (C % 16 == 0 && R % 16 == 0) {
        uint8_t *rq = xmalloc((size_t)(R * C));
        float *rs = xmalloc((size_t)(cd(R, 128) * C) * 4);
        orc_requant_act_t(q, s, R, C, rq, rs);
        free(rq); free(rs);
    }
    free(s); free(stt); free(s2);
    float *w = xmalloc((size_t)(cd(R, 128) * cd(C, 128)) * 4), *wt = xmalloc((size_t)(cd(R, 128) * cd(C, 128)) * 4);
    orc_quant_w_128x128(x, R, C, q, w);
    orc_quant_w_128x128_t(x, R, C, qt, wt);
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c)
            if (qt[c * R + r] != q[r * C + c]) { bad |= fail("transposed weight codes", R, C); r = R; break; }
    for (int64_t i = 0; i < cd(R, 128); ++i)
        for (int64_t j = 0; j < cd(C, 128); ++j)
            if (memcmp(&wt[j * cd(R, 128) + i], &w[i * cd(C, 128) + j], 4)) bad |= fail("transposed weight scales", R, C);
    free(w); free(wt);
    if (C % 2 == 0) {
        uint16_t *h = xmalloc((size_t)(R * (C / 2)) * 2);
        orc_swiglu(x, R, C / 2, h);
        free(h);
    }
    free(x); free(xt); free(q); free(qt); free(q2);
    return bad;
}

static void gemms(int mode, int64_t M, int64_t N, int64_t K)
{
    int64_t nk = cd(K, 128);
    uint8_t *a = code_input(M * K), *b = code_input(N * K);
    float *sa = scale_input(nk * M);
    float *sb = scale_input(mode == 2 ? nk * N : cd(N, 128) * nk);
    double *out = xmalloc((size_t)(M * N) * 8), *na = xmalloc((size_t)M * 8), *nb = xmalloc((size_t)N * 8);
    double *da = xmalloc((size_t)(M * K) * 8), *db = xmalloc((size_t)(N * K) * 8), at[3];
    uint16_t *o16 = xmalloc((size_t)(M * N) * 2);
    int64_t ms[3] = {0, M - 1, M / 2}, ns[3] = {N - 1, 0, N / 2};
    orc_gemm(mode, a, sa, b, sb, M, N, K, out);
    orc_gemm_at(mode, a, sa, b, sb, M, N, K, ms, ns, 3, at);
    orc_deq_row_norms(mode, a, sa, b, sb, M, N, K, na, nb);
    orc_dequant_a(a, sa, M, K, da);
    orc_dequant_b(mode, b, sb, N, K, db);
    orc_f64_to_bf16_array(out, M * N, o16);
    free(a); free(b); free(sa); free(sb); free(out); free(na); free(nb); free(da); free(db); free(o16);
}

int main(void)
{
    static const int64_t rows[] = {1, 3, 16, 127, 129, 260};
    static const int64_t cols[] = {16, 112, 128, 144, 272};
    int bad = 0;
    for (size_t i = 0; i < sizeof rows / sizeof rows[0]; ++i)
        for (size_t j = 0; j < sizeof cols / sizeof cols[0]; ++j) bad |= quantizers(rows[i], cols[j]);
    static const int64_t shapes[][3] = {{1, 1, 16}, {17, 5, 144}, {130, 129, 272}, {256, 300, 400}};
    for (int mode = 0; mode < 3; ++mode)
        for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) gemms(mode, shapes[i][0], shapes[i][1], shapes[i][2]);
    float f[5] = {0.0f, -0.0f, 447.9f, -1e-5f, 3.0f};
    uint8_t q[5];
    orc_e4m3_encode_array(f, 5, q);
    if (q[1] != 0x80 || q[2] != 0x7e || orc_e4m3_encode(-1e-5f) != 0x80) bad |= fail("codec", 1, 5);
    printf("oracle under sanitizers: %s\n", bad ? "FAILED" : "ok");
    return bad;
}
