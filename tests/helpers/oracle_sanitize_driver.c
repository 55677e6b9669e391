/* oracle_sanitize_driver.c -- test helper (CPU only): calls every entry point of
 * oracle/nvfp4_oracle.c over the kinds of input the pins use -- every mode and layout, with
 * and without the rotation and margins, ragged and empty shapes, sub-sets of vectors, strip-
 * local scales, the decoder, the EDEN internals, and the scalar roundings at their edges (0,
 * subnormals, 448, infinities, NaN) -- so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer can report any out-of-bounds access, leak or undefined
 * operation.  It also checks that each call returns the documented status and that two calls
 * on the same input give the same bytes.  Exit status 0 means every call behaved. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t h);
void oracle_philox4x32_10(uint64_t key, const uint32_t ctr[4], uint32_t out[4]);
void oracle_signs(uint64_t rht_seed, float sigma[128]);
void oracle_fwht128(float a[128]);
float oracle_e4m3_value(uint8_t code);
uint8_t oracle_e4m3_rne_sat(float t);
uint8_t oracle_e4m3_up(float t);
float oracle_e2m1_value(uint8_t code);
int oracle_e2m1_rtn_mag(float a);
float oracle_tensor_scale(int mode, float amax);
float oracle_amax(const uint16_t *x, int64_t rows, int64_t cols, int axis, int rht,
                  uint64_t rht_seed);
int oracle_quantize_vectors(int mode, const uint16_t *x, int64_t rows, int64_t cols, int axis,
                            int rht, uint64_t seed, uint64_t rht_seed, float g,
                            const int64_t *vec_ids, int64_t nvec, uint8_t *codes,
                            uint8_t *scales, uint32_t *elem_margin, uint32_t *scale_margin);
int oracle_quantize(int mode, const uint16_t *x, int64_t rows, int64_t cols, int axis, int rht,
                    uint64_t seed, uint64_t rht_seed, uint8_t *codes, uint8_t *scales,
                    float *g_out, uint32_t *elem_margin, uint32_t *scale_margin);
int oracle_quantize_strips(int mode, const uint16_t *x, int64_t rows, int64_t cols, int axis,
                           int rht, uint64_t seed, uint64_t rht_seed, int64_t strip,
                           uint8_t *codes, uint8_t *scales, float *g_out,
                           uint32_t *elem_margin, uint32_t *scale_margin);
int oracle_dequantize(const uint8_t *codes, const uint8_t *scales, float g, int64_t nvec,
                      int64_t n, int rht, uint64_t rht_seed, float *out);
int oracle_eden_internals(const uint16_t *x, int64_t rows, int64_t cols, int axis,
                          uint64_t rht_seed, float g, int64_t vec, float *r_out, float *q_out,
                          float *S_out, float *c_out);
uint8_t oracle_scale_sr(float c, uint32_t w);
int oracle_elem_sr_mag(float a, uint32_t w);
void oracle_margin_n(int kind, const float *v, const uint32_t *aux, uint32_t *out, int64_t n);
void oracle_e4m3_rne_sat_n(const float *t, uint8_t *out, int64_t n);
void oracle_e4m3_up_n(const float *t, uint8_t *out, int64_t n);
void oracle_e2m1_rtn_mag_n(const float *a, uint8_t *out, int64_t n);
void oracle_scale_sr_n(float c, const uint32_t *w, uint8_t *out, int64_t n);
void oracle_elem_sr_mag_n(float a, const uint32_t *w, uint8_t *out, int64_t n);
void oracle_scale_sr_pairs_n(const float *c, const uint32_t *w, uint8_t *out, int64_t n);
void oracle_elem_sr_pairs_n(const float *a, const uint32_t *w, uint8_t *out, int64_t n);
void oracle_philox_n(const uint64_t *key, const uint32_t *ctr, uint32_t *out, int64_t n);
int oracle_mx_scale_exp(float m);
int oracle_mx_quantize(int sr, const uint16_t *x, int64_t rows, int64_t cols, int axis,
                       int rht, uint64_t seed, uint64_t rht_seed, uint8_t *codes,
                       uint8_t *scales);
int oracle_mx_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t nvec, int64_t n,
                         int rht, uint64_t rht_seed, float *out);

static int failures = 0;
#define CHECK(cond, ...) do { if (!(cond)) { fprintf(stderr, __VA_ARGS__); \
    fputc('\n', stderr); ++failures; } } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    rng_state ^= rng_state << 13; rng_state ^= rng_state >> 7; rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 16);
}

/* BF16 bits of a value with a random sign, exponent in [-20, 20) and mantissa; a few zeros,
 * signed zeros and extreme values mixed in. */
static uint16_t random_bf16(void)
{
    uint32_t r = next_u32();
    switch (r % 61) {
    case 0: return 0x0000;
    case 1: return 0x8000;
    case 2: return 0x0001;                      /* smallest subnormal */
    case 3: return 0x5B80;                      /* about 2^56 - within the contract's edge */
    default: break;
    }
    uint32_t e = 127 - 20 + (next_u32() % 40);
    return (uint16_t)(((r & 1u) << 15) | (e << 7) | ((r >> 1) & 0x7Fu));
}

static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); if (!p) abort(); return p; }

static void run_shape(int64_t rows, int64_t cols)
{
    size_t ne = (size_t)(rows * cols);
    uint16_t *x = xmalloc(ne * 2);
    for (size_t i = 0; i < ne; ++i) x[i] = random_bf16();
    for (int mode = 0; mode < 4; ++mode)
        for (int axis = 0; axis < 2; ++axis)
            for (int rht = 0; rht < 2; ++rht) {
                int64_t n = axis == 0 ? cols : rows, vecs = axis == 0 ? rows : cols;
                int rot = rht || mode == 2;
                int valid = n % 16 == 0 && (!rot || n % 128 == 0);
                size_t nc = (size_t)(vecs * (n / 2)), ns = (size_t)(vecs * (n / 16));
                uint8_t *c1 = xmalloc(nc), *s1 = xmalloc(ns), *c2 = xmalloc(nc), *s2 = xmalloc(ns);
                uint32_t *em = xmalloc((size_t)(vecs * n) * 4), *sm = xmalloc(ns * 4);
                float g1 = -1, g2 = -2;
                int rc1 = oracle_quantize(mode, x, rows, cols, axis, rht, 7, 9, c1, s1, &g1, em, sm);
                int rc2 = oracle_quantize(mode, x, rows, cols, axis, rht, 7, 9, c2, s2, &g2, NULL,
                                          NULL);
                CHECK(rc1 == (valid ? 0 : -2) && rc2 == rc1, "quantize %dx%d mode %d axis %d rht %d: rc %d",
                      (int)rows, (int)cols, mode, axis, rht, rc1);
                if (valid && rc1 == 0) {
                    CHECK(g1 == g2 && !memcmp(c1, c2, nc) && !memcmp(s1, s2, ns),
                          "quantize %dx%d mode %d: margins changed the result", (int)rows,
                          (int)cols, mode);
                    /* a sub-set of vectors, in a shuffled order */
                    int64_t k = vecs < 5 ? vecs : 5;
                    int64_t ids[5];
                    for (int64_t i = 0; i < k; ++i) ids[i] = (int64_t)(next_u32() % (uint32_t)vecs);
                    uint8_t *cv = xmalloc((size_t)(k * (n / 2))), *sv = xmalloc((size_t)(k * (n / 16)));
                    int rc = oracle_quantize_vectors(mode, x, rows, cols, axis, rht, 7, 9, g1, ids, k,
                                                     cv, sv, NULL, NULL);
                    CHECK(rc == 0, "quantize_vectors rc %d", rc);
                    for (int64_t i = 0; i < k && rc == 0; ++i)
                        CHECK(!memcmp(cv + i * (n / 2), c1 + ids[i] * (n / 2), (size_t)(n / 2)),
                              "quantize_vectors differs from quantize");
                    free(cv); free(sv);
                    /* decode */
                    float *out = xmalloc((size_t)(vecs * n) * 4);
                    CHECK(oracle_dequantize(c1, s1, g1, vecs, n, rot, 9, out) == 0, "dequantize");
                    free(out);
                    /* strip-local scales, two strip sizes */
                    for (int64_t strip = 1; strip <= 128; strip *= 128) {
                        float *gs = xmalloc((size_t)((vecs + strip - 1) / strip + 1) * 4);
                        CHECK(oracle_quantize_strips(mode, x, rows, cols, axis, rht, 7, 9, strip,
                                                     c2, s2, gs, em, sm) == 0, "strips");
                        free(gs);
                    }
                    if (mode == 2 && vecs > 0) {
                        float *r = xmalloc((size_t)n * 4), *q = xmalloc((size_t)n * 4);
                        float *S = xmalloc((size_t)(n / 128 + 1) * 4), *c = xmalloc((size_t)(n / 16 + 1) * 4);
                        CHECK(oracle_eden_internals(x, rows, cols, axis, 9, g1, vecs - 1, r, q, S, c) == 0,
                              "internals");
                        free(r); free(q); free(S); free(c);
                    }
                }
                free(c1); free(s1); free(c2); free(s2); free(em); free(sm);
            }
    /* the MXFP4 contract: blocks of 32 */
    for (int sr = 0; sr < 2; ++sr)
        for (int axis = 0; axis < 2; ++axis)
            for (int rht = 0; rht < 2; ++rht) {
                int64_t n = axis == 0 ? cols : rows, vecs = axis == 0 ? rows : cols;
                int valid = n % 32 == 0 && (!rht || n % 128 == 0);
                size_t nc = (size_t)(vecs * (n / 2)), ns = (size_t)(vecs * (n / 32));
                uint8_t *c = xmalloc(nc), *sc = xmalloc(ns);
                int rc = oracle_mx_quantize(sr, x, rows, cols, axis, rht, 3, 4, c, sc);
                CHECK(rc == (valid ? 0 : -2), "mx quantize %dx%d rc %d", (int)rows, (int)cols, rc);
                if (valid && rc == 0) {
                    float *out = xmalloc((size_t)(vecs * n) * 4);
                    CHECK(oracle_mx_dequantize(c, sc, vecs, n, rht, 4, out) == 0, "mx dequantize");
                    free(out);
                }
                free(c); free(sc);
            }
    float amax = oracle_amax(x, rows, cols, 0, 1, 3);
    CHECK(amax >= 0 || cols % 128, "amax");
    free(x);
}

static void run_scalars(void)
{
    enum { N = 4096 };
    float *v = xmalloc(N * 4);
    uint32_t *w = xmalloc(N * 4), *m = xmalloc(N * 4);
    uint8_t *b = xmalloc(N);
    const float edges[] = {0.0f, -0.0f, 1e-45f, 0.001953125f, 0.015625f, 0.25f, 0.75f, 5.0f,
                           6.0f, 7.99f, 432.0f, 448.0f, 449.0f, 3.4e38f, INFINITY, NAN};
    for (int i = 0; i < N; ++i) {
        v[i] = i < 16 ? edges[i] : ldexpf((float)(next_u32() % 10000) / 1000.0f,
                                          (int)(next_u32() % 24) - 12);
        w[i] = next_u32();
    }
    oracle_e4m3_rne_sat_n(v, b, N);
    oracle_e4m3_up_n(v, b, N);
    oracle_e2m1_rtn_mag_n(v, b, N);
    oracle_scale_sr_n(0.5f, w, b, N);
    oracle_elem_sr_mag_n(2.5f, w, b, N);
    /* the SR steps and margins are defined on their documented ranges */
    float *c = xmalloc(N * 4), *a = xmalloc(N * 4);
    uint32_t *u = xmalloc(N * 4);
    for (int i = 0; i < N; ++i) {
        c[i] = 0.015625f + (447.0f - 0.015625f) * (float)(next_u32() % 65536) / 65536.0f;
        a[i] = 6.0f * (float)(next_u32() % 65537) / 65536.0f;
        u[i] = w[i] ^ 0x5A5A5A5Au;
    }
    oracle_scale_sr_pairs_n(c, w, b, N);
    oracle_elem_sr_pairs_n(a, u, b, N);
    for (int kind = 0; kind < 6; ++kind) {
        const float *src = kind == 3 ? c : kind == 4 ? a : v;
        const uint32_t *aux = kind == 4 ? u : w;
        float *pos = xmalloc(N * 4);
        for (int i = 0; i < N; ++i) pos[i] = (kind == 0 || isnan(src[i])) ? src[i] : fabsf(src[i]);
        if (kind == 5) for (int i = 0; i < N; ++i) if (!isfinite(pos[i])) pos[i] = 1.0f;
        uint32_t *aux2 = xmalloc(N * 4);
        for (int i = 0; i < N; ++i) {
            float f = 1.0f + (float)(aux[i] % 1000);
            memcpy(&aux2[i], &f, 4);
        }
        if (kind == 1 || kind == 2) for (int i = 0; i < N; ++i) if (isnan(pos[i])) pos[i] = 1.0f;
        oracle_margin_n(kind, pos, kind == 5 ? aux2 : aux, m, N);
        free(pos); free(aux2);
    }
    uint64_t keys[64];
    uint32_t ctr[256], out[256];
    for (int i = 0; i < 64; ++i) keys[i] = ((uint64_t)next_u32() << 32) | next_u32();
    for (int i = 0; i < 256; ++i) ctr[i] = next_u32();
    oracle_philox_n(keys, ctr, out, 64);
    float sigma[128], h[128];
    oracle_signs(5, sigma);
    for (int i = 0; i < 128; ++i) h[i] = sigma[i] * (float)i;
    oracle_fwht128(h);
    for (int code = 0; code < 128; ++code) (void)oracle_e4m3_value((uint8_t)code);
    for (int code = 0; code < 16; ++code) (void)oracle_e2m1_value((uint8_t)code);
    CHECK(oracle_scale_sr(1.0f, 0) == 0x38, "scale SR of 1");
    CHECK(oracle_elem_sr_mag(6.0f, 0) == 7, "element SR at 6");
    CHECK(oracle_e2m1_rtn_mag(0.25f) == 0, "E2M1 tie");
    CHECK(oracle_tensor_scale(3, 1792.0f) == 1.0f, "4/6 tensor scale");
    for (int i = 0; i < N; ++i) (void)oracle_mx_scale_exp(fabsf(v[i]));
    CHECK(oracle_mx_scale_exp(6.0f) == 0 && oracle_mx_scale_exp(0.0f) == -127, "MX scale");
    free(v); free(w); free(m); free(b); free(c); free(a); free(u);
}

int main(void)
{
    const int64_t shapes[][2] = {{256, 1024}, {130, 144}, {48, 40}, {144, 48}, {200, 256},
                                 {256, 200}, {384, 640}, {128, 128}, {0, 256}, {256, 0},
                                 {16, 16}, {8, 8}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) run_shape(shapes[i][0], shapes[i][1]);
    run_scalars();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: all calls behaved\n");
    return 0;
}
