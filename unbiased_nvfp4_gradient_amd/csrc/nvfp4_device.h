// nvfp4_device.h -- scalar device functions of the gfx950 NVFP4 kernels: the Philox4x32-10
// generator and the roundings onto the E4M3 (scale) and E2M1 (element) grids.
//
// The kernels in nvfp4_kernels.hip and the conversion check under tests/helpers include this
// file, so the check exercises exactly the code the quantizers run.  Formats: OCP E4M3FN
// (bias 7, largest finite 448, subnormals k * 2^-9) for the 1x16 block scales and E2M1
// (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) for the elements, as NVFP4 uses them (Telegram
// digest quant_prune_distill post 640, "Method": FP8 scales, the +-6 element grid).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4k {

constexpr float FLT_BIG = 3.40282347e+38f;

// ------------------------------------------------------------------------------ Philox
// Philox4x32-10 (Salmon et al., SC'11): 10 rounds of two 32x32->64 multiplies, key bumped by
// the Weyl constants between rounds.
struct Word4 { uint32_t w[4]; };

__device__ __forceinline__ Word4 philox(uint64_t key, uint32_t c0, uint32_t c1, uint32_t c2,
                                        uint32_t c3)
{
    uint32_t k0 = (uint32_t)key, k1 = (uint32_t)(key >> 32);
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;   // one v_mad_u64_u32 each
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0, n2;
        if (round == 0) {
            // the first round's inputs are partly wave-uniform: plain XORs let the
            // compiler keep that part on the scalar unit
            n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
            n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        } else {
            // three-input XOR in one v_bitop3_b32 (truth table 0x96: odd parity)
            n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
            n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        }
        c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    Word4 r;
    r.w[0] = c0; r.w[1] = c1; r.w[2] = c2; r.w[3] = c3;
    return r;
}

// ------------------------------------------------------------------------------ formats
// Smallest E4M3FN value >= t >= 0, capped at 448.
__device__ __forceinline__ uint32_t e4m3_up(float t)
{
    if (!(t < 448.0f)) return 0x7Eu;
    if (t < 0.015625f) return (uint32_t)__builtin_ceilf(t * 512.0f);
    uint32_t u = (__float_as_uint(t) + 0xFFFFFu) & 0xFFF00000u;
    return (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);
}

// E4M3 byte of a normal c in [2^-6, 448) rounded stochastically: add the top 20 bits of
// the random word w to the 20 mantissa bits E4M3 drops, keep the 3 that remain.  The fp32
// bits >> 20 are exponent << 3 | mantissa, so the E4M3 byte is that minus the bias
// difference (127 - 7) << 3 = 960; a carry out of the mantissa bumps the exponent, and
// c < 448 cannot carry past 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_sr_normal(uint32_t bits, uint32_t w)
{
    return ((bits + (w >> 12)) >> 20) - 960u;
}

__device__ __forceinline__ float e4m3_val(uint32_t c)
{
    const uint32_t e = c >> 3, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

__device__ __forceinline__ float e2m1_val(uint32_t mag)
{
    const uint32_t e = mag >> 1, m = mag & 1u;
    const uint32_t b = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
    return __uint_as_float(b);
}

typedef float float2v __attribute__((ext_vector_type(2)));

// (m & a) | (~m & b): the bits of a where m is set, of b elsewhere.  m (uniform) passes through an
// empty asm so that the compiler keeps the select (one v_bfi_b32) rather than splitting a
// constant mask into separate AND and OR instructions.
__device__ __forceinline__ uint32_t bit_select(uint32_t m, uint32_t a, uint32_t b)
{
    asm("" : "+s"(m));
    return (m & a) | (~m & b);
}

// Stochastic rounding onto the signed E2M1 grid, eight elements into one dword of codes
// (element k in nibble k).  Element k with random word w[k]: with lo < hi the grid neighbours
// of a = min(|y|, 6) and frac = (a - lo) / (hi - lo), the top 22 bits v of w[k] are added to
// the fraction as v * 2^-22 and the sum rounds down, so the magnitude is hi iff
// frac + v * 2^-22 >= 1; the sign is y's (y is never -0 here: it comes from fma(r, rcp, +0)).
// gfx950's SR conversion does exactly this per element of its pair, with the draw taken from
// bits 31..10 of its random operand for the low element and bits 30..9 for the high one, and
// saturates |y| >= 6 to magnitude 7.  Each element needs its own draw, so every instruction
// converts the pair (y[2j], y[2j+1]) twice: once with w[2j] (its low nibble kept) and once
// with w[2j+1] >> 1 (its high nibble kept, which then sees bits 31..10 of w[2j+1]).
// The instruction writes byte j of its destination and leaves the other three bytes as they
// were, but the compiler does not carry the builtin's old-value operand into that register
// (it does for the round-to-nearest form), so only byte j of each result is defined here:
// the bytes are merged with bit selects.
__device__ __forceinline__ uint32_t e2m1_sr_pack8(const float *y, const uint32_t *w)
{
    uint32_t u[4];
#define NVFP4_SR_PAIR(j)                                                                       \
    {                                                                                          \
        const float2v p = {y[2 * (j)], y[2 * (j) + 1]};                                        \
        const uint32_t l = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, w[2 * (j)], 1.0f, (j)); \
        const uint32_t h =                                                                     \
            __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, w[2 * (j) + 1] >> 1, 1.0f, (j)); \
        u[j] = bit_select(0x0F0F0F0Fu, l, h);                                                  \
    }
    NVFP4_SR_PAIR(0) NVFP4_SR_PAIR(1) NVFP4_SR_PAIR(2) NVFP4_SR_PAIR(3)
#undef NVFP4_SR_PAIR
    return bit_select(0x0000FFFFu, bit_select(0x000000FFu, u[0], u[1]),
                      bit_select(0x00FF0000u, u[2], u[3]));
}

// Nearest-even E4M3 of t >= 0, saturating: the hardware conversion is exact below 448.
// Its result indexes the 128-entry scale table: the mask keeps even a NaN input (outside the
// contract) inside the table; a finite t >= 0 never sets bit 7.
__device__ __forceinline__ uint32_t e4m3_rne_hw(float t)
{
    // bytes 1..3 of the result are masked off, so the instruction's old-value operand (the
    // bits it leaves in place) can be any live register: t's own bits, rather than a zero
    // that would cost a move
    const float c = fminf(t, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, (int)__float_as_uint(c), false) &
           0x7Fu;
}

// Codes of y0, y1 (nearest-even E2M1, sign of the input) into byte `sel` of w.
#define CVT_FP4(w, y0, y1, sel) \
    __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((w), (y0), (y1), 1.0f, (sel))

// Signed grid values of the two codes in byte `sel` of w.
#define DEC_FP4(w, sel) __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((w), 1.0f, (sel))

// Reciprocal rounded once, clamped so a zero / subnormal divisor stays finite.
__device__ __forceinline__ float clamped_rcp(float d)
{
    const float r = 1.0f / d;
    return r > FLT_BIG ? FLT_BIG : r;
}

// Exponent of the MXFP4 block scale: the smallest e with 6 * 2^e >= m (m the block's max |r|,
// finite, >= 0), clamped to [-127, 127]; -127 for m = 0.
// frexp gives m = f * 2^E with f in [0.5, 1) (subnormal m too); 6 * 2^(E-3) = 0.75 * 2^E covers
// m exactly when f <= 0.75, else 6 * 2^(E-2) = 1.5 * 2^E is the smallest that does.
__device__ __forceinline__ int mx_scale_exp(float m)
{
    if (!(m > 0.0f)) return -127;
    const int E = __builtin_amdgcn_frexp_expf(m);
    const float f = __builtin_amdgcn_frexp_mantf(m);
    const int e = E - 3 + (f > 0.75f ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

}  // namespace nvfp4k
