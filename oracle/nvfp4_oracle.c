/*
 * nvfp4_oracle.c -- CPU oracle for the MS-EDEN / SR / RTN / 4-over-6 NVFP4 quantizers.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this file's library.  The GPU product path never calls
 * it and shares no code, header or table with it.
 *
 * Sources (cited by page title and section):
 *  [Q2-TH]  "Quartet II: Accurate LLM Pre-Training in NVFP4 by Improved Unbiased Gradient
 *           Estimation" summary (itsolotime.com, Thai): abstract; Q1 "theory vs hardware
 *           compromises" (fixed 128-dim rotation groups, one rotation per tensor, no SR for
 *           scales below about 1/32000 of the max); Fig. 9 (unbiasedness test).
 *  [Q2-RU]  Quartet II blog paraphrase (denisavetisyan.com): "NVFP4 and micro-scaling",
 *           "MS-EDEN and randomized methods" (RHT + stochastic rounding).
 *  [FUSE]   "Format-Aware Fusion for Fast FP4 Pretraining" note (rit.work): global NVFP4
 *           max as a synchronisation point; one producer emitting both layouts; the
 *           CTA-local variant (maxima inside a block of work, separate row and column
 *           corrections applied after the GEMM's sum).
 *  [TG]     quant_prune_distill post 640 (Telegram digest), section "Method": SR definition,
 *           EDEN = random Hadamard rotation + multiplication by the ratio of the vector's
 *           scalar product with itself to the scalar product of the quantized rotated and
 *           the unquantized rotated vector; scales stochastically rounded to FP8; the
 *           forward 4/6 choice between the full (-6,6) grid and the clipped (-4,4) grid;
 *           1x16 linear groups rather than 16x16 squares.
 *
 * The pages give no formula, order of operations or constant beyond 128, 16, +-6/+-4 and
 * roughly 1/32000.  Every step below is the plainest reading; each reading is listed in
 * the design notes.  All arithmetic is IEEE binary32 with round-to-nearest-even, one
 * rounding per operation, no fused multiply-add (the build disables contraction with
 * -ffp-contract=off) and no flushing of subnormals: every floating-point value here decides
 * an integer (a code, a scale byte, an SR branch), and the GPU takes those decisions in
 * binary32 too.  A scalar product or a sum of squares is its definition written out: each
 * term rounded once, then a balanced pairwise sum in natural order.
 *
 * Pins (tests marked "not gpu"): Philox against rocRAND's engine and the Random123
 * known-answer vectors; the Hadamard transform against the Sylvester matrix (exact on
 * integers) and H*H = 128 I; E4M3 rounding against torch's float8_e4m3fn cast and brute
 * force; E2M1 rounding against brute-force nearest; SR probabilities by enumeration of every
 * random word; the EDEN ratio against fp64 within the pairwise-sum bound; the 4/6 choice
 * against an fp64 brute force; every margin (distance to a rounding boundary) against the
 * number of one-ulp steps that changes the rounding; scaling / sign / layout invariants; MSE
 * ordering and unbiasedness statistics; strip-local scales against the global method on one
 * strip and per-strip power-of-two equivariance.  Nothing here is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <float.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MODE_RTN 0
#define MODE_SR 1
#define MODE_EDEN 2
#define MODE_FP46 3

#define STREAM_SIGN 1u
#define STREAM_SCALE_SR 2u
#define STREAM_ELEM_SR 3u

#define GROUP 128
#define BLOCK 16

/* ------------------------------------------------------------------ bit helpers */
static float f32_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

float oracle_bf16_to_f32(uint16_t h) { return f32_of((uint32_t)h << 16); }

/* ------------------------------------------------------------------ Philox4x32-10
 * Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11):
 * each round multiplies counter words 0 and 2 by the two round multipliers, forms the
 * new counter from the high halves xor-ed with the other words and the key, and the
 * low halves; the key advances by the two Weyl constants between rounds. */
void oracle_philox4x32_10(uint64_t key, const uint32_t ctr[4], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = (uint32_t)key, k1 = (uint32_t)(key >> 32);
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* One 32-bit random word for item `index` of stream `stream` on layout `axis`.
 * Four consecutive items share one Philox call: counter = (index/4 lo, index/4 hi,
 * stream, axis), word = index mod 4. */
static uint32_t rand_word(uint64_t seed, uint64_t index, uint32_t stream, uint32_t axis)
{
    uint64_t j = index >> 2;
    uint32_t ctr[4] = {(uint32_t)j, (uint32_t)(j >> 32), stream, axis};
    uint32_t w[4];
    oracle_philox4x32_10(seed, ctr, w);
    return w[index & 3];
}

/* ------------------------------------------------------------------ rotation signs
 * One sign vector per call, shared by every group of the tensor and by both layouts
 * ([Q2-TH] Q1: one rotation seed per tensor).  sigma_j = -1 iff bit (j mod 32) of word
 * j/32 of Philox(rht_seed, (0, 0, STREAM_SIGN, 0)) is set. */
void oracle_signs(uint64_t rht_seed, float sigma[GROUP])
{
    uint32_t ctr[4] = {0u, 0u, STREAM_SIGN, 0u};
    uint32_t w[4];
    oracle_philox4x32_10(rht_seed, ctr, w);
    for (int j = 0; j < GROUP; ++j)
        sigma[j] = ((w[j >> 5] >> (j & 31)) & 1u) ? -1.0f : 1.0f;
}

/* ------------------------------------------------------------------ Hadamard transform
 * Unnormalised Walsh-Hadamard transform of 128 values in Sylvester (natural) order,
 * butterfly spans h = 1, 2, 4, ..., 64 in ascending order; each butterfly replaces
 * (a_i, a_{i+h}) by (a_i + a_{i+h}, a_i - a_{i+h}), rounded once each ([TG] Method,
 * [Q2-RU] RHT).  The 1/sqrt(128) normalisation is left out: every quantity except the
 * tensor scale is invariant to it, and the inverse uses the exact factor 2^-7. */
void oracle_fwht128(float a[GROUP])
{
    for (int h = 1; h < GROUP; h <<= 1)
        for (int i = 0; i < GROUP; ++i)
            if ((i & h) == 0) {
                float u = a[i], v = a[i + h];
                a[i] = u + v;
                a[i + h] = u - v;
            }
}

/* ------------------------------------------------------------------ E4M3 (OCP E4M3FN)
 * Bias 7, no infinities, 0x7F is NaN, largest finite 448 = 0x7E, smallest normal 2^-6,
 * subnormals k * 2^-9.  Scales are non-negative, so only codes 0x00..0x7E occur. */
float oracle_e4m3_value(uint8_t code)
{
    int e = (code >> 3) & 15, m = code & 7;
    if (e == 0) return ldexpf((float)m, -9);
    return ldexpf(1.0f + (float)m / 8.0f, e - 7);
}

/* Quantum (spacing of E4M3 values) around t >= 0, as a power-of-two exponent. */
static int e4m3_quantum_exp(float t)
{
    if (t < 0.015625f) return -9;      /* subnormal range: spacing 2^-9 */
    int e;
    frexpf(t, &e);                     /* t = f * 2^e, f in [0.5, 1) */
    return (e - 1) - 3;                /* 3 mantissa bits */
}

/* Encode n quanta of 2^q (n integer, the value an exact E4M3 value). */
static uint8_t e4m3_encode(double n, int q)
{
    if (q == -9) return (uint8_t)n;                 /* subnormal; n = 8 is 2^-6 = 0x08 */
    int ebias = q + 3 + 7;                          /* exponent field of [2^(q+3), 2^(q+4)) */
    return (uint8_t)((ebias << 3) + ((int)n - 8));  /* n = 16 carries into the exponent */
}

/* Nearest E4M3 value to t >= 0, ties to the even code, saturating at 448. */
uint8_t oracle_e4m3_rne_sat(float t)
{
    if (!(t < 448.0f)) return 0x7E;
    int q = e4m3_quantum_exp(t);
    double n = nearbyint(ldexp((double)t, -q));     /* exact scaling, round half to even */
    return e4m3_encode(n, q);
}

/* Smallest E4M3 value >= t >= 0, capped at 448. */
uint8_t oracle_e4m3_up(float t)
{
    if (!(t < 448.0f)) return 0x7E;
    int q = e4m3_quantum_exp(t);
    double n = ceil(ldexp((double)t, -q));
    return e4m3_encode(n, q);
}

/* ------------------------------------------------------------------ E2M1
 * Magnitudes V = {0, 0.5, 1, 1.5, 2, 3, 4, 6} ([TG] Method: grid spans (-6, 6)).
 * Round to nearest, ties to the even magnitude code, saturating at 6. */
static const float E2M1_V[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* The two stochastic-rounding steps (defined below, pinned by enumeration of every random
 * word); the quantizers call them for every decision they make. */
uint8_t oracle_scale_sr(float c, uint32_t w);
int oracle_elem_sr_mag(float a, uint32_t w);
static const float E2M1_THRESH[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};

float oracle_e2m1_value(uint8_t code)
{
    float v = E2M1_V[code & 7];
    return (code & 8) ? -v : v;
}

int oracle_e2m1_rtn_mag(float a)
{
    if (a <= 0.25f) return 0;
    if (a < 0.75f) return 1;
    if (a <= 1.25f) return 2;
    if (a < 1.75f) return 3;
    if (a <= 2.5f) return 4;
    if (a < 3.5f) return 5;
    if (a <= 5.0f) return 6;
    return 7;
}

/* ------------------------------------------------------------------ margins
 * Distance, in units in the last place, between a pre-rounding value and the boundary
 * of the rounding it feeds.  A GPU/oracle mismatch is excusable only within 2 ulp. */
#define MARGIN_NONE 0xFFFFFFFFu

static uint32_t ulp_dist(float a, float b)   /* a, b >= 0 and finite */
{
    uint32_t x = bits_of(fabsf(a)), y = bits_of(fabsf(b));
    return x > y ? x - y : y - x;
}

static uint32_t e2m1_margin(float a)
{
    uint32_t best = MARGIN_NONE;
    for (int i = 0; i < 7; ++i) {
        uint32_t d = ulp_dist(a, E2M1_THRESH[i]);
        if (d < best) best = d;
    }
    return best;
}

static uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

/* t against the midpoints next to its RNE result (and against the saturation point). */
static uint32_t e4m3_rne_margin(float t)
{
    uint8_t c = oracle_e4m3_rne_sat(t);
    uint32_t best = MARGIN_NONE;
    if (c > 0) {
        float mid = (oracle_e4m3_value(c - 1) + oracle_e4m3_value(c)) * 0.5f;
        best = umin(best, ulp_dist(t, mid));
    }
    if (c < 0x7E) {
        float mid = (oracle_e4m3_value(c) + oracle_e4m3_value(c + 1)) * 0.5f;
        best = umin(best, ulp_dist(t, mid));
    }
    return best;
}

/* t against the grid points next to its round-up result: the result moves up once t passes
 * its own value (except at the top, where every larger t saturates to the same code) and
 * down once t reaches the value below. */
static uint32_t e4m3_up_margin(float t)
{
    uint8_t c = oracle_e4m3_up(t);
    uint32_t best = MARGIN_NONE;
    if (c < 0x7E) best = ulp_dist(t, oracle_e4m3_value(c));
    if (c > 0) best = umin(best, ulp_dist(t, oracle_e4m3_value(c - 1)));
    return best;
}

/* Scale SR of c with word w rounds up exactly when the 20 dropped mantissa bits plus the
 * draw's top 20 bits carry out (reach 2^20): the margin is their sum's distance from 2^20. */
static uint32_t scale_sr_margin(float c, uint32_t w)
{
    uint32_t sum = (bits_of(c) & 0xFFFFFu) + (w >> 12);
    return sum > 0x100000u ? sum - 0x100000u : 0x100000u - sum;
}

/* Element SR of a in [0, 6) with word w (draw v = w >> 10) rounds up exactly when a reaches
 * the point lo + (1 - v * 2^-22) * (hi - lo) between its grid neighbours lo < hi: the margin
 * is a's distance from that point (exact in fp64, and exact again as a binary32: it needs at
 * most 24 significant bits). */
static uint32_t elem_sr_margin(float a, uint32_t w)
{
    int lo = 0;
    while (E2M1_V[lo + 1] <= a) ++lo;
    double ab = E2M1_V[lo] + (1.0 - (double)(w >> 10) / 4194304.0) * (E2M1_V[lo + 1] - E2M1_V[lo]);
    return ulp_dist(a, (float)ab);
}

/* ------------------------------------------------------------------ pairwise sums
 * Balanced pairwise sum in natural order: v_i <- v_{2i} + v_{2i+1}, level by level. */
static float tree_sum(const float *v, int n)   /* n a power of two, n <= 128 */
{
    float t[GROUP];
    memcpy(t, v, sizeof(float) * (size_t)n);
    for (int len = n; len > 1; len >>= 1)
        for (int i = 0; i < len / 2; ++i)
            t[i] = t[2 * i] + t[2 * i + 1];
    return t[0];
}

/* ------------------------------------------------------------------ tensor scale
 * The NVFP4 tensor scale maps the tensor's largest rotated magnitude to the top of the
 * FP8 scale range times the top of the element grid ([FUSE]: the global max is the one
 * tensor-wide quantity): g = amax / (6 * 448) for RTN, SR and MS-EDEN, and
 * g = amax / (4 * 448) for 4/6, so that the clipped option's scale amax/4 still fits. */
float oracle_tensor_scale(int mode, float amax)
{
    float d = (mode == MODE_FP46) ? 1792.0f : 2688.0f;
    return amax / d;
}

/* Reciprocal used for "divide by a scale": rounded once, and clamped to FLT_MAX so that
 * a zero or subnormal divisor yields finite quotients (0 * FLT_MAX = 0). */
static float clamped_rcp(float d)
{
    float r = 1.0f / d;
    return (r > FLT_MAX) ? FLT_MAX : r;
}

/* ------------------------------------------------------------------ vector access
 * Layout `axis` 0 quantizes the rows of X (vectors of length cols); axis 1 quantizes the
 * columns (vectors of length rows): the column layout is the row layout of X^T. */
static void load_vector(const uint16_t *x, int64_t rows, int64_t cols, int axis,
                        int64_t vec, float *out)
{
    if (axis == 0) {
        for (int64_t j = 0; j < cols; ++j) out[j] = oracle_bf16_to_f32(x[vec * cols + j]);
    } else {
        for (int64_t i = 0; i < rows; ++i) out[i] = oracle_bf16_to_f32(x[i * cols + vec]);
    }
}

/* r = H (sigma * x) per group of 128, or r = x when the rotation is off. */
static void rotate_vector(float *v, int64_t n, int rht, const float sigma[GROUP])
{
    if (!rht) return;
    for (int64_t g0 = 0; g0 < n; g0 += GROUP) {
        float a[GROUP];
        for (int j = 0; j < GROUP; ++j) a[j] = sigma[j] * v[g0 + j];
        oracle_fwht128(a);
        memcpy(v + g0, a, sizeof a);
    }
}

/* ------------------------------------------------------------------ amax (the sync point)
 * Largest |r| over vectors [v0, v1) of layout `axis`.  Exact; the order of the max does
 * not matter. */
static float range_amax(const uint16_t *x, int64_t rows, int64_t cols, int axis, int rht,
                        const float sigma[GROUP], int64_t v0, int64_t v1)
{
    int64_t n = axis == 0 ? cols : rows;
    float amax = 0.0f;
#pragma omp parallel for schedule(static) reduction(max : amax)
    for (int64_t v = v0; v < v1; ++v) {
        float buf_stack[4096];
        float *buf = buf_stack;
        float local = 0.0f;
        /* vectors longer than 4096 are processed group by group */
        for (int64_t g0 = 0; g0 < n; g0 += 4096) {
            int64_t len = (n - g0) < 4096 ? (n - g0) : 4096;
            if (axis == 0)
                for (int64_t j = 0; j < len; ++j)
                    buf[j] = oracle_bf16_to_f32(x[v * cols + g0 + j]);
            else
                for (int64_t j = 0; j < len; ++j)
                    buf[j] = oracle_bf16_to_f32(x[(g0 + j) * cols + v]);
            rotate_vector(buf, len, rht, sigma);
            for (int64_t j = 0; j < len; ++j) {
                float a = fabsf(buf[j]);
                if (a > local) local = a;
            }
        }
        if (local > amax) amax = local;
    }
    return amax;
}

/* Largest |r| over the whole layout ([FUSE]: packing waits until the partial maxima of
 * the whole tensor are collected). */
float oracle_amax(const uint16_t *x, int64_t rows, int64_t cols, int axis, int rht,
                  uint64_t rht_seed)
{
    float sigma[GROUP];
    oracle_signs(rht_seed, sigma);
    return range_amax(x, rows, cols, axis, rht, sigma, 0, axis == 0 ? rows : cols);
}

/* ------------------------------------------------------------------ one block of 16
 * Quantize r[0..15] by round-to-nearest with E4M3 block scale code s (already chosen)
 * and tensor scale g.  Writes codes, the dequantized rotated values q, and margins. */
static void rtn_block(const float *r, uint8_t s, float g, int mag_cap, uint8_t *codes,
                      float *q, uint32_t *emargin)
{
    if (s == 0) {
        for (int i = 0; i < BLOCK; ++i) {
            codes[i] = 0;
            q[i] = 0.0f;
            if (emargin) emargin[i] = MARGIN_NONE;
        }
        return;
    }
    float den = oracle_e4m3_value(s) * g;
    float rcp = clamped_rcp(den);
    for (int i = 0; i < BLOCK; ++i) {
        float y = r[i] * rcp;
        int mag = oracle_e2m1_rtn_mag(fabsf(y));
        if (mag > mag_cap) mag = mag_cap;
        /* sign bit set iff r < 0: an exact zero, of either sign, encodes as +0 */
        int neg = r[i] < 0.0f;
        codes[i] = (uint8_t)(mag | (neg << 3));
        float qv = den * E2M1_V[mag];
        q[i] = neg ? -qv : qv;
        if (emargin) emargin[i] = e2m1_margin(fabsf(y));
    }
}

/* ------------------------------------------------------------------ EDEN scalar products
 * <r, r> and <r, q> of one 128-group ([TG] Method: the ratio of the vector's scalar product
 * with itself to the scalar product of the quantized rotated and the unquantized rotated
 * vector).  q_i is the RTN dequantization of element i (den_b * V_i, rounded once, signed),
 * as rtn_block leaves it.  A scalar product is written out as its definition: each term
 * rounded once, P_i = r_i * r_i and Q_i = r_i * q_i, then a balanced pairwise sum of the 128
 * terms in natural order. */
static void eden_dots(const float *r, const float *q, float *num, float *dot)
{
    float P[GROUP], Q[GROUP];
    for (int i = 0; i < GROUP; ++i) {
        P[i] = r[i] * r[i];
        Q[i] = r[i] * q[i];
    }
    *num = tree_sum(P, GROUP);
    *dot = tree_sum(Q, GROUP);
}

/* Squared error of one block's RTN option ([TG] Method: the 4/6 choice keeps the grid with
 * the lower error): d_i = q_i - r_i with q_i the option's dequantized value (rounded once),
 * each square rounded once, summed by a balanced pairwise sum of the 16 terms. */
static float block_sq_error(const float *r, const float *q)
{
    float d2[BLOCK];
    for (int i = 0; i < BLOCK; ++i) {
        float d = q[i] - r[i];
        d2[i] = d * d;
    }
    return tree_sum(d2, BLOCK);
}

/* ------------------------------------------------------------------ one vector
 * The quantizers of one vector r (already rotated), length n, given the tensor scale.
 * vec is the vector's index in its layout (for the random streams and scale indices). */
static void quantize_rotated_vector(int mode, const float *r, int64_t n, int64_t vec,
                                    int axis, uint64_t seed, float g, uint8_t *codes,
                                    uint8_t *scales, uint32_t *emargin, uint32_t *smargin)
{
    const int64_t nblk = n / BLOCK;
    const float six_g_rcp = clamped_rcp(6.0f * g);
    const float four_g_rcp = clamped_rcp(4.0f * g);
    uint8_t bcodes[GROUP];
    float q[GROUP];

    if (mode == MODE_RTN || mode == MODE_EDEN) {
        /* RTN with an RNE block scale; MS-EDEN then corrects the scales per group
         * ([TG] Method: EDEN ratio, FP8 stochastic rounding of the scales). */
        for (int64_t g0 = 0; g0 < n; g0 += GROUP) {
            int64_t glen = (n - g0) < GROUP ? (n - g0) : GROUP;
            uint8_t s[GROUP / BLOCK];
            uint32_t sm[GROUP / BLOCK];
            for (int64_t b = 0; b < glen / BLOCK; ++b) {
                const float *rb = r + g0 + b * BLOCK;
                float m = 0.0f;
                for (int i = 0; i < BLOCK; ++i)
                    if (fabsf(rb[i]) > m) m = fabsf(rb[i]);
                float t = m * six_g_rcp;
                s[b] = oracle_e4m3_rne_sat(t);
                sm[b] = (s[b] == 0 && t == 0.0f) ? MARGIN_NONE : e4m3_rne_margin(t);
                rtn_block(rb, s[b], g, 7, bcodes + b * BLOCK, q + b * BLOCK,
                          emargin ? emargin + g0 + b * BLOCK : NULL);
            }
            for (int64_t i = 0; i < glen; ++i) {
                int64_t e = g0 + i;
                if (e % 2 == 0) codes[e / 2] = bcodes[i];
                else codes[e / 2] |= (uint8_t)(bcodes[i] << 4);
            }
            if (mode == MODE_RTN) {
                for (int64_t b = 0; b < glen / BLOCK; ++b) {
                    scales[(g0 / BLOCK) + b] = s[b];
                    if (smargin) smargin[(g0 / BLOCK) + b] = sm[b];
                }
                continue;
            }
            /* EDEN ratio S = <r, r> / <r, q> over the group of 128. */
            float num, den;
            eden_dots(r + g0, q, &num, &den);
            float S = (den > 0.0f) ? num / den : 1.0f;
            for (int b = 0; b < GROUP / BLOCK; ++b) {
                int64_t k = vec * nblk + (g0 / BLOCK) + b;   /* index in the scale array */
                uint8_t out;
                uint32_t m2 = sm[b];
                if (s[b] == 0) {
                    out = 0;
                } else {
                    float c = S * oracle_e4m3_value(s[b]);
                    if (!(c < 448.0f)) {
                        out = 0x7E;
                        m2 = umin(m2, ulp_dist(c, 448.0f));
                    } else if (c < 0.015625f) {
                        /* below 2^-6 = 448 / 28672, roughly 1/32000 of the top scale: no SR */
                        out = oracle_e4m3_rne_sat(c);
                        m2 = umin(m2, umin(e4m3_rne_margin(c), ulp_dist(c, 0.015625f)));
                    } else {
                        uint32_t w = rand_word(seed, (uint64_t)k, STREAM_SCALE_SR,
                                               (uint32_t)axis);
                        out = oracle_scale_sr(c, w);
                        m2 = umin(m2, umin(scale_sr_margin(c, w),
                                           umin(ulp_dist(c, 0.015625f), ulp_dist(c, 448.0f))));
                    }
                }
                scales[(g0 / BLOCK) + b] = out;
                if (smargin) smargin[(g0 / BLOCK) + b] = m2;
            }
        }
        return;
    }

    if (mode == MODE_SR) {
        /* Plain stochastic rounding ([TG] Method; [Q2-TH] opening paragraph): block scale
         * rounded up so that no element clips, then each element rounds to one of its two
         * grid neighbours with probability given by its distance to them. */
        for (int64_t b = 0; b < nblk; ++b) {
            const float *rb = r + b * BLOCK;
            float m = 0.0f;
            for (int i = 0; i < BLOCK; ++i)
                if (fabsf(rb[i]) > m) m = fabsf(rb[i]);
            float t = m * six_g_rcp;
            uint8_t s = oracle_e4m3_up(t);
            scales[b] = s;
            if (smargin) smargin[b] = (t == 0.0f) ? MARGIN_NONE : e4m3_up_margin(t);
            float den = oracle_e4m3_value(s) * g;
            float rcp = clamped_rcp(den);
            for (int i = 0; i < BLOCK; ++i) {
                int64_t e = b * BLOCK + i;
                uint8_t code = 0;
                uint32_t em = MARGIN_NONE;
                if (s != 0) {
                    float y = rb[i] * rcp;
                    float a = fminf(fabsf(y), 6.0f);
                    int mag;
                    if (a >= 6.0f) {
                        mag = 7;
                    } else {
                        uint32_t w = rand_word(seed, (uint64_t)(vec * n + e), STREAM_ELEM_SR,
                                               (uint32_t)axis);
                        mag = oracle_elem_sr_mag(a, w);
                        em = elem_sr_margin(a, w);
                    }
                    code = (uint8_t)(mag | ((rb[i] < 0.0f) << 3));
                }
                if (e % 2 == 0) codes[e / 2] = code;
                else codes[e / 2] |= (uint8_t)(code << 4);
                if (emargin) emargin[e] = em;
            }
        }
        return;
    }

    /* MODE_FP46: per block, the full +-6 grid or the clipped +-4 grid, whichever has the
     * lower squared error ([TG] Method, forward pass); ties keep +-6. */
    for (int64_t b = 0; b < nblk; ++b) {
        const float *rb = r + b * BLOCK;
        float m = 0.0f;
        for (int i = 0; i < BLOCK; ++i)
            if (fabsf(rb[i]) > m) m = fabsf(rb[i]);
        float tA = m * six_g_rcp, tB = m * four_g_rcp;
        uint8_t sA = oracle_e4m3_rne_sat(tA), sB = oracle_e4m3_rne_sat(tB);
        uint8_t cA[BLOCK], cB[BLOCK];
        float qA[BLOCK], qB[BLOCK];
        uint32_t mA[BLOCK], mB[BLOCK];
        rtn_block(rb, sA, g, 7, cA, qA, mA);
        rtn_block(rb, sB, g, 6, cB, qB, mB);
        float errA = block_sq_error(rb, qA), errB = block_sq_error(rb, qB);
        int pickA = errA <= errB;
        scales[b] = pickA ? sA : sB;
        if (smargin) {
            uint32_t m2 = ulp_dist(errA, errB);
            if (tA != 0.0f) m2 = umin(m2, umin(e4m3_rne_margin(tA), e4m3_rne_margin(tB)));
            smargin[b] = m2;
        }
        for (int i = 0; i < BLOCK; ++i) {
            int64_t e = b * BLOCK + i;
            uint8_t code = pickA ? cA[i] : cB[i];
            if (e % 2 == 0) codes[e / 2] = code;
            else codes[e / 2] |= (uint8_t)(code << 4);
            if (emargin) emargin[e] = pickA ? mA[i] : mB[i];
        }
    }
}

/* ------------------------------------------------------------------ public entry points */

/* Quantize the vectors vec_ids[0..nvec) (all vectors when vec_ids is NULL) of layout
 * `axis`, given the tensor scale g.  Outputs are indexed by position in vec_ids:
 * codes [nvec][n/2] (byte j = code(2j) | code(2j+1) << 4), scales [nvec][n/16],
 * optional margins elem_margin [nvec][n] and scale_margin [nvec][n/16]. */
int oracle_quantize_vectors(int mode, const uint16_t *x, int64_t rows, int64_t cols,
                            int axis, int rht, uint64_t seed, uint64_t rht_seed, float g,
                            const int64_t *vec_ids, int64_t nvec, uint8_t *codes,
                            uint8_t *scales, uint32_t *elem_margin, uint32_t *scale_margin)
{
    int64_t n = axis == 0 ? cols : rows;
    int64_t total = axis == 0 ? rows : cols;
    if (n % BLOCK) return -2;
    if ((rht || mode == MODE_EDEN) && n % GROUP) return -2;
    if (!vec_ids) nvec = total;
    float sigma[GROUP];
    oracle_signs(rht_seed, sigma);
    int use_rht = rht || mode == MODE_EDEN;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < nvec; ++i) {
        int64_t vec = vec_ids ? vec_ids[i] : i;
        if (vec < 0 || vec >= total) { bad = 1; continue; }
        float *buf = (float *)malloc(sizeof(float) * (size_t)n);
        if (!buf) { bad = 1; continue; }
        load_vector(x, rows, cols, axis, vec, buf);
        rotate_vector(buf, n, use_rht, sigma);
        quantize_rotated_vector(mode, buf, n, vec, axis, seed, g, codes + i * (n / 2),
                                scales + i * (n / BLOCK),
                                elem_margin ? elem_margin + i * n : NULL,
                                scale_margin ? scale_margin + i * (n / BLOCK) : NULL);
        free(buf);
    }
    return bad ? -2 : 0;
}

/* Whole-layout quantization: amax, tensor scale, then every vector. */
int oracle_quantize(int mode, const uint16_t *x, int64_t rows, int64_t cols, int axis,
                    int rht, uint64_t seed, uint64_t rht_seed, uint8_t *codes,
                    uint8_t *scales, float *g_out, uint32_t *elem_margin,
                    uint32_t *scale_margin)
{
    int use_rht = rht || mode == MODE_EDEN;
    float amax = oracle_amax(x, rows, cols, axis, use_rht, rht_seed);
    float g = oracle_tensor_scale(mode, amax);
    *g_out = g;
    return oracle_quantize_vectors(mode, x, rows, cols, axis, use_rht, seed, rht_seed, g,
                                   NULL, 0, codes, scales, elem_margin, scale_margin);
}

/* ------------------------------------------------------------------ strip-local scales
 * The CTA-local variant of [FUSE]: the maximum behind the FP32 second-level scale is
 * taken inside one block of work rather than over the whole tensor, so no block waits for
 * the others, and the GEMM applies one correction per row block of its first operand and
 * one per column block of its second after the sum over K.  A correction that stays fixed
 * during that sum has to cover whole vectors, so the reading taken here: the vectors of a
 * layout form strips of `strip` consecutive vectors (128 on the GPU, one tile), strip s
 * takes g_s = tensor scale of max |r| over its own vectors, and each of its vectors is
 * quantized exactly as in the global method with g_s in place of g; every random stream
 * keeps the vector's index in the whole layout.  g_out receives ceil(vecs / strip) floats. */
int oracle_quantize_strips(int mode, const uint16_t *x, int64_t rows, int64_t cols, int axis,
                           int rht, uint64_t seed, uint64_t rht_seed, int64_t strip,
                           uint8_t *codes, uint8_t *scales, float *g_out,
                           uint32_t *elem_margin, uint32_t *scale_margin)
{
    int64_t n = axis == 0 ? cols : rows;
    int64_t total = axis == 0 ? rows : cols;
    int use_rht = rht || mode == MODE_EDEN;
    if (strip <= 0 || n % BLOCK) return -2;
    if (use_rht && n % GROUP) return -2;
    float sigma[GROUP];
    oracle_signs(rht_seed, sigma);
    for (int64_t v0 = 0; v0 < total; v0 += strip) {
        int64_t v1 = (total - v0) < strip ? total : v0 + strip;
        float g = oracle_tensor_scale(mode, range_amax(x, rows, cols, axis, use_rht, sigma,
                                                       v0, v1));
        g_out[v0 / strip] = g;
        if (n == 0) continue;
        int64_t *ids = (int64_t *)malloc(sizeof(int64_t) * (size_t)(v1 - v0));
        if (!ids) return -2;
        for (int64_t v = v0; v < v1; ++v) ids[v - v0] = v;
        int rc = oracle_quantize_vectors(mode, x, rows, cols, axis, use_rht, seed, rht_seed, g,
                                         ids, v1 - v0, codes + v0 * (n / 2),
                                         scales + v0 * (n / BLOCK),
                                         elem_margin ? elem_margin + v0 * n : NULL,
                                         scale_margin ? scale_margin + v0 * (n / BLOCK) : NULL);
        free(ids);
        if (rc) return rc;
    }
    return 0;
}

/* Dequantize nvec vectors of length n: value = sign * (s * g) * V[mag]; with the
 * rotation on, undo it: x_j = sigma_j * (H q)_j * 2^-7 (H H = 128 I). */
int oracle_dequantize(const uint8_t *codes, const uint8_t *scales, float g, int64_t nvec,
                      int64_t n, int rht, uint64_t rht_seed, float *out)
{
    if (n % BLOCK) return -2;
    if (rht && n % GROUP) return -2;
    float sigma[GROUP];
    oracle_signs(rht_seed, sigma);
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < nvec; ++v) {
        float *o = out + v * n;
        for (int64_t e = 0; e < n; ++e) {
            uint8_t byte = codes[v * (n / 2) + e / 2];
            uint8_t code = (e % 2 == 0) ? (byte & 15) : (byte >> 4);
            float den = oracle_e4m3_value(scales[v * (n / BLOCK) + e / BLOCK]) * g;
            float qv = den * E2M1_V[code & 7];
            o[e] = (code & 8) ? -qv : qv;
        }
        if (rht) {
            for (int64_t g0 = 0; g0 < n; g0 += GROUP) {
                float a[GROUP];
                memcpy(a, o + g0, sizeof a);
                oracle_fwht128(a);
                for (int j = 0; j < GROUP; ++j) o[g0 + j] = (sigma[j] * a[j]) * 0.0078125f;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ diagnostics for pins */

/* Per-group EDEN internals for vector `vec` of layout `axis` given g: the ratio S, the
 * two sums, and the pre-SR corrected scales c (n/16 values).  Used by the fp64 pin. */
int oracle_eden_internals(const uint16_t *x, int64_t rows, int64_t cols, int axis,
                          uint64_t rht_seed, float g, int64_t vec, float *r_out,
                          float *q_out, float *S_out, float *c_out)
{
    int64_t n = axis == 0 ? cols : rows;
    if (n % GROUP) return -2;
    float sigma[GROUP];
    float *buf = (float *)malloc(sizeof(float) * (size_t)n);
    if (!buf) return -2;
    oracle_signs(rht_seed, sigma);
    load_vector(x, rows, cols, axis, vec, buf);
    rotate_vector(buf, n, 1, sigma);
    const float six_g_rcp = clamped_rcp(6.0f * g);
    for (int64_t g0 = 0; g0 < n; g0 += GROUP) {
        uint8_t bcodes[GROUP], s[GROUP / BLOCK];
        float q[GROUP];
        for (int b = 0; b < GROUP / BLOCK; ++b) {
            const float *rb = buf + g0 + b * BLOCK;
            float m = 0.0f;
            for (int i = 0; i < BLOCK; ++i)
                if (fabsf(rb[i]) > m) m = fabsf(rb[i]);
            s[b] = oracle_e4m3_rne_sat(m * six_g_rcp);
            rtn_block(rb, s[b], g, 7, bcodes + b * BLOCK, q + b * BLOCK, NULL);
        }
        float num, den;
        eden_dots(buf + g0, q, &num, &den);
        for (int i = 0; i < GROUP; ++i) {
            r_out[g0 + i] = buf[g0 + i];
            q_out[g0 + i] = q[i];
        }
        float S = (den > 0.0f) ? num / den : 1.0f;
        S_out[g0 / GROUP] = S;
        for (int b = 0; b < GROUP / BLOCK; ++b)
            c_out[g0 / BLOCK + b] = s[b] ? S * oracle_e4m3_value(s[b]) : 0.0f;
    }
    free(buf);
    return 0;
}

/* The scale-SR step alone, for the enumeration pin: E4M3 result of corrected scale c
 * (2^-6 <= c < 448) with random word w. */
uint8_t oracle_scale_sr(float c, uint32_t w)
{
    uint32_t up_bits = (bits_of(c) + (w >> 12)) & 0xFFF00000u;
    return oracle_e4m3_rne_sat(f32_of(up_bits));
}

/* The element-SR step alone: magnitude code of a = min(|y|, 6) with the element's random
 * word w.  Its top 22 bits v, read as the fraction v * 2^-22 of a grid step, are added to a's
 * position between its neighbours lo < hi and the sum is rounded down onto the grid: the
 * magnitude is hi exactly when frac + v * 2^-22 >= 1, so over the 2^22 draws it moves up
 * floor(frac * 2^22) times.  frac and the threshold 1 - v * 2^-22 are both exact in binary32. */
int oracle_elem_sr_mag(float a, uint32_t w)
{
    if (a >= 6.0f) return 7;
    int lo = 0;
    while (E2M1_V[lo + 1] <= a) ++lo;
    float frac = (a - E2M1_V[lo]) / (E2M1_V[lo + 1] - E2M1_V[lo]);
    uint32_t v = w >> 10;
    return frac >= (float)(4194304u - v) / 4194304.0f ? lo + 1 : lo;
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ array forms (for pins) */
void oracle_e4m3_rne_sat_n(const float *t, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_rne_sat(t[i]);
}

void oracle_e4m3_up_n(const float *t, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_up(t[i]);
}

void oracle_e2m1_rtn_mag_n(const float *a, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e2m1_rtn_mag(a[i]);
}

void oracle_scale_sr_n(float c, const uint32_t *w, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_scale_sr(c, w[i]);
}

void oracle_elem_sr_mag_n(float a, const uint32_t *w, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_elem_sr_mag(a, w[i]);
}

/* Margins of single roundings, for the pins: kind 0 = E2M1 nearest of |v|, 1 = E4M3 nearest
 * of v >= 0, 2 = E4M3 round-up of v >= 0, 3 = scale SR of v with word aux[i], 4 = element SR
 * of v in [0, 6) with word aux[i], 5 = ulp distance between v and aux[i] read as a
 * float. */
void oracle_margin_n(int kind, const float *v, const uint32_t *aux, uint32_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        switch (kind) {
        case 0: out[i] = e2m1_margin(fabsf(v[i])); break;
        case 1: out[i] = e4m3_rne_margin(v[i]); break;
        case 2: out[i] = e4m3_up_margin(v[i]); break;
        case 3: out[i] = scale_sr_margin(v[i], aux[i]); break;
        case 4: out[i] = elem_sr_margin(v[i], aux[i]); break;
        default: out[i] = ulp_dist(v[i], f32_of(aux[i])); break;
        }
    }
}

/* Element-wise forms over paired arrays, for checking the GPU's own device functions. */
void oracle_scale_sr_pairs_n(const float *c, const uint32_t *w, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_scale_sr(c[i], w[i]);
}

void oracle_elem_sr_pairs_n(const float *a, const uint32_t *w, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_elem_sr_mag(a[i], w[i]);
}

void oracle_philox_n(const uint64_t *key, const uint32_t *ctr, uint32_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) oracle_philox4x32_10(key[i], ctr + 4 * i, out + 4 * i);
}

/* ------------------------------------------------------------------ MXFP4 block contract
 * The recipe of the native FP4 matrix-core consumer.  gfx950's scaled matrix instructions
 * multiply E2M1 elements that carry one power-of-two (E8M0) scale per 32 consecutive elements
 * along K, and nothing per 16: an NVFP4 operand's E4M3 block scales (3 mantissa bits) cannot
 * be carried by them.  This contract is the plainest one they can consume: the vectors and
 * layouts, rotation and random streams of the NVFP4 quantizers; blocks of 32; block scale
 * 2^e with e the smallest integer such that 6 * 2^e >= max |r| over the block (the grid's top,
 * 6, covers the block: nothing clips, so SR stays unbiased, as with the NVFP4 SR scale),
 * e clamped to [-127, 127] (E8M0 byte = e + 127; an all-zero block gets byte 0); elements
 * y = r * 2^-e (one rounding; the scaling is exact unless y is subnormal) rounded to the E2M1
 * grid by RTN ([TG] Method: round to nearest) or SR ([Q2-TH] opening paragraph). */

/* Smallest e with 6 * 2^e >= m, clamped; -127 for m = 0. */
int oracle_mx_scale_exp(float m)
{
    if (!(m > 0.0f)) return -127;
    int E;
    frexpf(m, &E);                          /* m = f 2^E, f in [0.5, 1) */
    int e = E - 4;                          /* 6 * 2^(E-4) = 0.375 * 2^E < m */
    while (ldexp(6.0, e) < (double)m) ++e;  /* exact in double */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

int oracle_mx_quantize(int sr, const uint16_t *x, int64_t rows, int64_t cols, int axis,
                       int rht, uint64_t seed, uint64_t rht_seed, uint8_t *codes,
                       uint8_t *scales)
{
    int64_t n = axis == 0 ? cols : rows;
    int64_t nvec = axis == 0 ? rows : cols;
    if (n % 32) return -2;
    if (rht && n % GROUP) return -2;
    float sigma[GROUP];
    oracle_signs(rht_seed, sigma);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t vec = 0; vec < nvec; ++vec) {
        float *r = (float *)malloc(sizeof(float) * (size_t)(n ? n : 1));
        if (!r) { bad = 1; continue; }
        load_vector(x, rows, cols, axis, vec, r);
        rotate_vector(r, n, rht, sigma);
        for (int64_t b = 0; b < n / 32; ++b) {
            const float *rb = r + 32 * b;
            float m = 0.0f;
            for (int i = 0; i < 32; ++i)
                if (fabsf(rb[i]) > m) m = fabsf(rb[i]);
            int e = oracle_mx_scale_exp(m);
            scales[vec * (n / 32) + b] = (uint8_t)(e + 127);
            float p = ldexpf(1.0f, -e);     /* exact: -e in [-127, 127] */
            for (int i = 0; i < 32; ++i) {
                int64_t pos = 32 * b + i;
                float y = rb[i] * p;
                int mag;
                if (sr) {
                    uint32_t w = rand_word(seed, (uint64_t)(vec * n + pos), STREAM_ELEM_SR,
                                           (uint32_t)axis);
                    mag = oracle_elem_sr_mag(fminf(fabsf(y), 6.0f), w);
                } else {
                    mag = oracle_e2m1_rtn_mag(fabsf(y));
                }
                uint8_t code = (uint8_t)(mag | ((rb[i] < 0.0f) << 3));
                uint8_t *dst = codes + vec * (n / 2) + pos / 2;
                if (pos % 2 == 0) *dst = code;
                else *dst |= (uint8_t)(code << 4);
            }
        }
        free(r);
    }
    return bad ? -2 : 0;
}

/* value = sign * V[mag] * 2^e; with the rotation, x_j = sigma_j * (H q)_j * 2^-7. */
int oracle_mx_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t nvec, int64_t n,
                         int rht, uint64_t rht_seed, float *out)
{
    if (n % 32) return -2;
    if (rht && n % GROUP) return -2;
    float sigma[GROUP];
    oracle_signs(rht_seed, sigma);
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < nvec; ++v) {
        float *o = out + v * n;
        for (int64_t pos = 0; pos < n; ++pos) {
            uint8_t byte = codes[v * (n / 2) + pos / 2];
            uint8_t code = (pos % 2 == 0) ? (byte & 15) : (byte >> 4);
            float s = ldexpf(1.0f, (int)scales[v * (n / 32) + pos / 32] - 127);
            float qv = E2M1_V[code & 7] * s;
            o[pos] = (code & 8) ? -qv : qv;
        }
        if (rht) {
            for (int64_t g0 = 0; g0 < n; g0 += GROUP) {
                float a[GROUP];
                memcpy(a, o + g0, sizeof a);
                oracle_fwht128(a);
                for (int j = 0; j < GROUP; ++j) o[g0 + j] = (sigma[j] * a[j]) * 0.0078125f;
            }
        }
    }
    return 0;
}

void oracle_mx_scale_exp_n(const float *m, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)(oracle_mx_scale_exp(m[i]) + 127);
}
