// nvfp4_kernels.hip -- gfx950 kernels of the NVFP4 quantizers (MS-EDEN, SR, RTN, 4/6) and
// the dequantizer.
//
// Method sources (pages summarising "Quartet II: Accurate LLM Pre-Training in NVFP4 by
// Improved Unbiased Gradient Estimation"):
//   - Telegram digest quant_prune_distill post 640, "Method": SR; EDEN = random Hadamard
//     rotation + correction by <x,x>/<Q(Rx),Rx>; FP8 scales rounded stochastically; 4/6
//     choice between the +-6 and +-4 grids; 1x16 groups.
//   - itsolotime.com summary, Q1 "theory vs hardware compromises": 128-dim rotation groups,
//     one rotation per tensor, no SR for scales below about 1/32000 of the max.
//   - rit.work note on "Format-Aware Fusion for Fast FP4 Pretraining": the global max is a
//     synchronisation point; one producer writes both layouts.
//
// Arithmetic is binary32 with one rounding per operation: the library is built with
// -ffp-contract=off and no fast-math, so a multiply-add is fused only where __builtin_fmaf
// is written, and only where the fused form gives the same value as the separate operations
// (a product by +-1 or a sum with +0).  A scalar product or sum of squares is its definition:
// each term rounded once, then a balanced pairwise sum in natural order.
//
// Work decomposition.  The input is cut into 128 x 128 BF16 tiles (32 KiB).  Persistent
// workgroups stream tiles into two LDS buffers with direct global->LDS loads (the next
// tile lands while the current one is processed).  Each 128-element group is held by a pair
// of adjacent lanes, 64 values each: lanes 0..255 of a workgroup take the tile's 128 row
// segments (row layout), lanes 256..511 its 128 column segments (column layout).  Six of
// the seven butterfly stages of the Hadamard transform, the 1x16 block maxima and all but
// the last level of the EDEN pairwise sums stay in registers; the span-64 stage is one
// v_fmac_f32_dpp per value across the pair (the high half is read negated for it), and the
// last sum level one DPP swap.  MS-EDEN, RTN and 4/6 fit 128 registers (4 waves per SIMD).
// The LDS tile's 16-byte chunks are XOR-swizzled by row to spread both the row reads (one
// 16-byte chunk per lane) and the column reads (one 2-byte element per lane) over the banks.
//
// Conversions use gfx950's own instructions where they compute exactly the contract's
// rounding: v_cvt_scalef32_pk_fp4_f32 with scale 1.0 is round-to-nearest-even onto the E2M1
// grid with saturation and the sign of its input (two codes per instruction, packed in
// place), v_cvt_scalef32_pk_f32_fp4 decodes codes exactly, and v_cvt_pk_fp8_f32 is
// nearest-even E4M3 below 448 (the input is clamped at 448 first).  All other steps are
// plain binary32 arithmetic.  A scaled element is formed as fma(r, rcp, +0), which turns an
// exact zero of either sign into +0, so a code's sign bit is set exactly when r < 0.
//
// The global amax must be known before any scale can be rounded, so a quantization is two
// passes over X: k_amax (rotate, each workgroup's maxima stored in its own workspace slots,
// or one atomic max per workgroup and layout for the split phase-1 entry point) then k_quant
// (reduce those slots, rotate again, quantize, pack, store).  k_quant walks the tiles in the
// reverse order, so its first tiles are those k_amax touched last, which are the likeliest
// to still sit in the last-level cache.
//
// Strip-local scales (the CTA-local variant of the rit.work note on "Format-Aware Fusion for
// Fast FP4 Pretraining": maxima inside a block of work, row and column corrections applied
// after the GEMM's sum over K) take the same two passes with LOCAL = true and a small kernel
// between them: k_amax stores each wave's maximum over each tile (no atomics), k_strip_tables
// reduces them per strip (128 consecutive vectors: one tile row for the row layout, one tile
// column for the column layout) and writes each strip's g and scale table, and k_quant copies
// the table of each tile's strips into LDS along with the tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "nvfp4_device.h"

namespace nvfp4k {

enum Mode { MODE_RTN = 0, MODE_SR = 1, MODE_EDEN = 2, MODE_FP46 = 3,
            MODE_MX_RTN = 4, MODE_MX_SR = 5 };   // the last two: the MXFP4 block contract

constexpr bool is_mx(int mode) { return mode == MODE_MX_RTN || mode == MODE_MX_SR; }
enum Layouts { LAY_ROW = 1, LAY_COL = 2, LAY_BOTH = 3 };

constexpr uint32_t STREAM_SIGN = 1u, STREAM_SCALE_SR = 2u, STREAM_ELEM_SR = 3u;
constexpr int TILE = 128;            // tile edge == rotation group size
constexpr int CHUNKS = TILE / 8;     // 16-byte chunks per tile row

// ------------------------------------------------------------------------------ signs
struct Signs { uint32_t w[4]; };

__device__ __forceinline__ Signs make_signs(uint64_t rht_seed)
{
    const Word4 p = philox(rht_seed, 0u, 0u, STREAM_SIGN, 0u);
    Signs s;
#pragma unroll
    for (int i = 0; i < 4; ++i) s.w[i] = p.w[i];
    return s;
}

// sigma_p = -1 iff bit p of the 128-bit sign word; returned as an fp32 sign-bit mask.
__device__ __forceinline__ uint32_t sign_mask(const Signs &s, int p)
{
    return ((s.w[p >> 5] >> (p & 31)) & 1u) << 31;
}

// ------------------------------------------------------------------------------ tile
// 32 KiB.  Chunk c (8 BF16) of tile row i sits at slot i*16 + f(i, c), with
// f(i, c) = c ^ S(i) ^ (4 * bit 3 of c) and S(i) = (i & 15) ^ (4 * bit 6 of i).  The LDS
// serves 32 banks of 4 bytes, i.e. 8 slots, at a time, so what matters is f mod 8: the low
// bits of S spread consecutive rows over the banks; bit 3 of c (the row half a lane reads)
// and bit 6 of i (rows i and i + 64, read by the two lanes of a pair in one column read)
// each flip bit 2 of the slot, so the two lanes of a pair never share a bank in either
// reader.
struct Tile { uint4 chunk[TILE * CHUNKS]; };

__device__ __forceinline__ int swz_key(int i) { return (i & 15) ^ (((i >> 6) & 1) << 2); }
__device__ __forceinline__ int swz_slot(int i, int c) { return c ^ swz_key(i) ^ (((c >> 3) & 1) << 2); }
__device__ __forceinline__ int swz(int i, int c) { return i * CHUNKS + swz_slot(i, c); }
// The chunk held in slot s of row i (f(i, .) is its own kind of inverse: bit 3 survives it).
__device__ __forceinline__ int swz_chunk(int i, int s)
{
    const int u = s ^ swz_key(i);
    return u ^ (((u >> 3) & 1) << 2);
}

// Per-position fp32 sign-bit masks of the rotation (sigma_p = -1 -> 0x80000000), built
// once per workgroup in LDS and read as broadcasts right before use.  With the rotation,
// positions 64..127 (the high half of a group) carry the complement, so that half is read
// as -sigma*x; without it every mask is 0.
//   mr[h][k]  masks of positions 64h + 4k .. 64h + 4k + 3 (row order); the padding word
//             puts the two halves in different LDS banks.
//   mc[s][h]  masks of positions 64h + 16q + s for q = 0..3 (column reader order).
struct SignTable {
    uint4 mr[2][17];
    uint4 mc[16][2];
};

__device__ __forceinline__ void build_sign_table(SignTable &st, uint64_t rht_seed, bool rot)
{
    const int t = threadIdx.x;
    if (t < TILE) {
        uint32_t mask = 0u;
        if (rot) {
            const Signs s = make_signs(rht_seed);
            const int q = t >> 5;                        // sign word holding bit t
            const uint32_t word = q == 0 ? s.w[0] : q == 1 ? s.w[1] : q == 2 ? s.w[2] : s.w[3];
            mask = ((word >> (t & 31)) & 1u) << 31;
        }
        const int h = t >> 6, pl = t & 63;
        // with the rotation, the high half of every group is read negated (fwht_pair_blocks
        // undoes it in its last stage)
        if (rot && h) mask ^= 0x80000000u;
        reinterpret_cast<uint32_t *>(&st.mr[h][0])[pl] = mask;
        reinterpret_cast<uint32_t *>(&st.mc[pl & 15][h])[pl >> 4] = mask;
    }
}

// Synchronous load of tile (r0, c0) through registers; elements outside [0,R) x [0,C)
// read as zero.  Used for the ragged edge tiles only.
__device__ __forceinline__ void load_tile_sync(Tile &t, const uint16_t *__restrict__ x,
                                               int64_t R, int64_t C, int64_t r0, int64_t c0)
{
    for (int q = threadIdx.x; q < TILE * CHUNKS; q += blockDim.x) {
        const int i = q >> 4, c = q & 15;
        const int64_t row = r0 + i, col = c0 + 8 * c;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (row < R && col < C) v = *reinterpret_cast<const uint4 *>(x + row * C + col);
        t.chunk[swz(i, c)] = v;
    }
}

#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

// A 16-byte store marked non-temporal (streaming: `nt` on the instruction).
__device__ __forceinline__ void store_nt(float4 *p, float4 v)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(p));
}

// Byte offsets, from a full tile's first element, of the 16-byte chunks one lane moves in
// the direct global->LDS load (below).  With W waves, round k of wave w fills LDS slots
// (w + W k) * 64 + lane, i.e. tile row i = i0 + 4 W k with i0 = 4 w + lane / 16 < 32, and
// the chunk held in slot lane mod 16: the low bits of S(i) are those of i0 in every round,
// and bit 6 of i (the 4 in S) is set from row 64 on, which flips bit 2 of the chunk.  So a
// lane needs two offsets, one for the rounds above row 64 and one for the rest, plus 4 W
// rows per round.  They are 64-bit, so one load path serves every row length.
struct DmaLane { uint64_t a, b; };

template <int W>
__device__ __forceinline__ DmaLane dma_lane(int64_t C)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i0 = 4 * w + (lane >> 4);
    const int c = swz_chunk(i0, lane & 15);
    const uint64_t rowb = 2u * (uint64_t)i0 * (uint64_t)C;
    DmaLane d;
    d.a = rowb + 16u * (uint64_t)c;
    d.b = rowb + 16u * (uint64_t)(c ^ 4);
    return d;
}

// Start loading tile (r0, c0) into t (W waves take part).  A full tile goes straight from
// memory into LDS (global_load_lds_dwordx4: lane L of a wave instruction fills 16-byte slot
// base + L), so the load runs while the workgroup computes on its other buffer; each lane
// fetches the chunk whose swizzled slot it fills.  The data is visible after the next
// __syncthreads (which waits for this wave's outstanding memory operations).  Edge tiles
// load synchronously.
template <int W>
__device__ __forceinline__ void stage_tile(Tile &t, const uint16_t *__restrict__ x, int64_t R,
                                           int64_t C, int64_t r0, int64_t c0,
                                           const DmaLane &dl)
{
    if (r0 + TILE <= R && c0 + TILE <= C) {
        const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        const char *base = reinterpret_cast<const char *>(x + r0 * C + c0);
        const int64_t step = 8 * W * C;                 // bytes of 4 W rows
#pragma unroll
        for (int k = 0; k < 32 / W; ++k) {
            const char *p = base + k * step + (4 * W * k < 64 ? dl.a : dl.b);
            __builtin_amdgcn_global_load_lds(p, LDS_PTR(&t.chunk[(w + W * k) * 64]), 16, 0, 0);
        }
    } else {
        load_tile_sync(t, x, R, C, r0, c0);
    }
}

// Hide a value from loop-invariant code motion: the swizzled LDS addresses below are
// recomputed (one v_xor each) per tile instead of being hoisted into dozens of registers
// that stay live across the whole loop.
__device__ __forceinline__ uint32_t opaque(uint32_t v)
{
    __asm__ volatile("" : "+v"(v));
    return v;
}

// ------------------------------------------------------------------------------ half groups
// A 128-element group is held by a pair of adjacent lanes: lane half h = 0 holds positions
// 0..63, h = 1 holds 64..127, 64 registers each.

constexpr int HALF = TILE / 2;

// Row segment i, half h of the tile -> r[k] = sigma_p * x_p, p = 64h + k (exact BF16 decode,
// sign folded in).  Chunk cc + 8h of row i sits at byte i*256 + 16*(cc ^ 8h ^ 4h ^ S(i))
// = base ^ (cc << 4), with base = (i*256 + 16 S(i)) ^ (192 h).
__device__ __forceinline__ void read_row_half(const Tile &t, const SignTable &st, int i, int h,
                                              float r[HALF])
{
    const char *t8 = reinterpret_cast<const char *>(t.chunk);
    const uint32_t base = opaque((uint32_t)(i * 256 + 16 * swz_key(i)) ^ (uint32_t)(h ? 192 : 0));
    const uint4 *mrow = st.mr[h];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
        const uint4 v = *reinterpret_cast<const uint4 *>(t8 + (base ^ (uint32_t)(cc << 4)));
        const uint4 m0 = mrow[2 * cc], m1 = mrow[2 * cc + 1];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        const uint32_t m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // (w << 16) + mask flips bit 31 exactly when the mask is set
            r[8 * cc + 2 * k] = __uint_as_float((w[k] << 16) + m[2 * k]);
            r[8 * cc + 2 * k + 1] = __uint_as_float((w[k] & 0xFFFF0000u) ^ m[2 * k + 1]);
        }
    }
}

// Column segment j, half h -> r[k] = sigma_p * x_p, p = 64h + k.  Element (i, j) sits at
// byte i*256 + 16*f(i, J) + 2*(j&7), J = j>>3: for i = 64h + 16q + s, S(i) = s ^ 4h, so that
// is off(s) + 16384h + 4096q with the lane's J ^ (4 * bit 3 of J) ^ 4h as its column chunk.
__device__ __forceinline__ void read_col_half(const Tile &t, const SignTable &st, int j, int h,
                                              float r[HALF])
{
    // Every lane-dependent part of the address is in one offset, so that each load is a few
    // address steps from the tile itself: the compiler tags LDS accesses with the variable
    // they touch only up to a small depth of such steps, and an untagged read would also wait
    // for the next tile's loads into the other buffer.  The column chunk (bits 4..7) and the
    // half and element (bits 14 and 1..3) do not overlap, so the chunk's xor with s16 can be
    // applied to their sum.
    const char *t8 = reinterpret_cast<const char *>(t.chunk);
    const int J = j >> 3;
    const uint32_t lane = opaque((uint32_t)(16 * (J ^ (((J >> 3) & 1) << 2) ^ (h << 2))) +
                                 (uint32_t)(16384 * h) + 2 * (uint32_t)(j & 7));
#pragma unroll
    for (int s16 = 0; s16 < 16; ++s16) {
        const char *p = t8 + (lane ^ (uint32_t)(16 * s16)) + 256 * s16;
        const uint4 m = st.mc[s16][h];
        const uint32_t mm[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t v = *reinterpret_cast<const uint16_t *>(p + 4096 * q);
            r[16 * q + s16] = __uint_as_float((v << 16) + mm[q]);
        }
    }
}

// Value held by the other lane of the pair (DPP quad_perm [1,0,3,2]).
__device__ __forceinline__ float pair_swap(float v)
{
    // every lane reads a lane of its own quad, so no lane keeps its old value: mov_dpp
    // leaves the destination's old contents undefined and needs no copy to seed them
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// r <- H r over the pair, and the 1x16 block maxima of |r|.  Unnormalised Sylvester
// Walsh-Hadamard transform: butterfly spans 1, 2, ..., 32 inside each half, then span 64
// across the pair.  The readers fold the random signs in and read the high half negated,
// so before the last stage the low lane holds a (the transform of its half) and the high
// lane holds b' = -b.  The last stage is own + m * partner with m = -1 in the low lane
// (a - b' = a + b) and m = +1 in the high lane (b' + a = a - b): one v_fmac_f32_dpp, the
// DPP swap reading the partner's register.  Only the sign of an exact zero can differ from
// the direct a +- b (a zero's sign does not survive into any nonzero sum, and every
// consumer treats a zero of either sign alike: codes encode it as +0), so every value is
// the contract's.
//
// The compiler does not fold a DPP move into v_fmac_f32, so the last stage and the block
// maximum are written out, one 16-value block per statement.  The s_nop gives the two wait
// states a DPP read of a register written by the previous VALU instruction needs; inside
// the statement every DPP read is of a register no earlier instruction of it wrote.
__device__ __forceinline__ void fwht_pair_blocks(float r[HALF], int h, float bmax[4])
{
#pragma unroll
    for (int s = 1; s < HALF; s <<= 1) {
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            if ((i & s) == 0) {
                const float u = r[i], v = r[i + s];
                r[i] = u + v;
                r[i + s] = u - v;
            }
        }
    }
    const float m = h ? 1.0f : -1.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        float *q = r + 16 * b;
        float mx;
#define FMAC_DPP(k) "v_fmac_f32_dpp %" #k ", %" #k ", %17 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        __asm__("s_nop 1\n\t"
                FMAC_DPP(0) FMAC_DPP(1) FMAC_DPP(2) FMAC_DPP(3) FMAC_DPP(4) FMAC_DPP(5)
                FMAC_DPP(6) FMAC_DPP(7) FMAC_DPP(8) FMAC_DPP(9) FMAC_DPP(10) FMAC_DPP(11)
                FMAC_DPP(12) FMAC_DPP(13) FMAC_DPP(14) FMAC_DPP(15)
                "v_max3_f32 %16, |%0|, |%1|, |%2|\n\t"
                "v_max3_f32 %16, %16, |%3|, |%4|\n\t"
                "v_max3_f32 %16, %16, |%5|, |%6|\n\t"
                "v_max3_f32 %16, %16, |%7|, |%8|\n\t"
                "v_max3_f32 %16, %16, |%9|, |%10|\n\t"
                "v_max3_f32 %16, %16, |%11|, |%12|\n\t"
                "v_max3_f32 %16, %16, |%13|, |%14|\n\t"
                "v_max_f32 %16, %16, |%15|"
                : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]), "+v"(q[4]), "+v"(q[5]),
                  "+v"(q[6]), "+v"(q[7]), "+v"(q[8]), "+v"(q[9]), "+v"(q[10]), "+v"(q[11]),
                  "+v"(q[12]), "+v"(q[13]), "+v"(q[14]), "+v"(q[15]), "=&v"(mx)
                : "v"(m));
#undef FMAC_DPP
        bmax[b] = mx;
    }
}

// Phase 1 needs only max |r| over the group, and the signs of the last two stages' inputs
// do not matter for it.  After the in-lane spans 1..16 the low lane holds quarters q0, q1
// (positions 0..31, 32..63) and the high lane q2, q3.  Span 32 gives s = q0 + q1, d = q0 - q1
// in the low lane and s', d' in the high lane, and the group's outputs are s +- s' and
// d +- d'.  Since max(|u + v|, |u - v|) = |u| + |v| and binary32 rounding is monotone and
// symmetric in sign, the largest |output| is the largest of fl(|s_k| + |s'_k|) and
// fl(|d_k| + |d'_k|) over k: 64 sums, not 128 outputs.  The low lane stores (s, d) in
// registers (k, k + 32), the high lane (d', s') -- A + m*B and A - m*B with m = +-1, one
// exact FMA each -- so one DPP read of the partner's register k + 32 gives the low lane s'_k
// and the high lane d_k: each lane forms 32 sums |own k| + |partner k + 32| and their max.
__device__ __forceinline__ float fwht_pair_absmax(float r[HALF], int h)
{
#pragma unroll
    for (int s = 1; s < HALF / 2; s <<= 1) {
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            if ((i & s) == 0) {
                const float u = r[i], v = r[i + s];
                r[i] = u + v;
                r[i + s] = u - v;
            }
        }
    }
    const float m = h ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < HALF / 2; ++i) {
        const float u = r[i], v = r[i + HALF / 2];
        r[i] = __builtin_fmaf(v, m, u);
        r[i + HALF / 2] = __builtin_fmaf(v, -m, u);
    }
    float mx = 0.0f;
#pragma unroll
    for (int c = 0; c < HALF / 2; c += 8) {
        const float *lo = r + c, *hi = r + HALF / 2 + c;
        float t0, t1, t2, t3, t4, t5, t6, t7;
        // operands: 0 = running max, 1..8 = sums, 9..16 = own k, 17..24 = own k + 32 (read
        // from the partner by DPP).  The s_nop gives the DPP reads their two wait states.
#define ADD_DPP(t, a, b) "v_add_f32_dpp %" #t ", |%" #b "|, |%" #a "| quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        __asm__("s_nop 1\n\t"
                ADD_DPP(1, 9, 17) ADD_DPP(2, 10, 18) ADD_DPP(3, 11, 19) ADD_DPP(4, 12, 20)
                ADD_DPP(5, 13, 21) ADD_DPP(6, 14, 22) ADD_DPP(7, 15, 23) ADD_DPP(8, 16, 24)
                "v_max3_f32 %0, %0, %1, %2\n\t"
                "v_max3_f32 %0, %0, %3, %4\n\t"
                "v_max3_f32 %0, %0, %5, %6\n\t"
                "v_max3_f32 %0, %0, %7, %8"
                : "+v"(mx), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5),
                  "=&v"(t6), "=&v"(t7)
                : "v"(lo[0]), "v"(lo[1]), "v"(lo[2]), "v"(lo[3]), "v"(lo[4]), "v"(lo[5]),
                  "v"(lo[6]), "v"(lo[7]), "v"(hi[0]), "v"(hi[1]), "v"(hi[2]), "v"(hi[3]),
                  "v"(hi[4]), "v"(hi[5]), "v"(hi[6]), "v"(hi[7]));
#undef ADD_DPP
    }
    return mx;
}

// Balanced pairwise sum of 2^k values in natural order, in place.
template <int N>
__device__ __forceinline__ float tree(float *v)
{
#pragma unroll
    for (int len = N; len > 1; len >>= 1) {
#pragma unroll
        for (int i = 0; i < len / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
    }
    return v[0];
}

__device__ __forceinline__ float block_max(const float *r)
{
    float m = fmaxf(fabsf(r[0]), fabsf(r[1]));     // pairs of fmaxf fold into v_max3_f32
#pragma unroll
    for (int i = 2; i < 16; i += 2) m = fmaxf(m, fmaxf(fabsf(r[i]), fabsf(r[i + 1])));
    return m;
}

// Table over the 127 E4M3 codes a scale can take (0x00..0x7E): (scale value s, den = s*g,
// rcp(den)).  Code 0 gets rcp = 0: a block with scale 0 then scales every element to +0 and
// rounds it to code 0x0, which is what the contract prescribes for it, without a select.
// Entry 127 (0x7F is NaN in E4M3, never a scale) holds (g, rcp(6g), rcp(4g)).
struct ScaleTable { float4 e[128]; };

constexpr int TAB_G = 127;

__device__ __forceinline__ float4 scale_entry(int j, float g)
{
    if (j == TAB_G) return make_float4(g, clamped_rcp(6.0f * g), clamped_rcp(4.0f * g), 0.0f);
    const float sv = e4m3_val((uint32_t)j);
    const float den = sv * g;
    return make_float4(sv, den, j ? clamped_rcp(den) : 0.0f, 0.0f);
}

__device__ __forceinline__ void build_scale_table(ScaleTable &tb, float g, int tid)
{
    if (tid < 128) tb.e[tid] = scale_entry(tid, g);
}

// ------------------------------------------------------------------------------ arguments
struct LayoutOut {
    uint8_t *codes;    // [vecs][n/2]
    uint8_t *scales;   // [vecs][n/16] (MXFP4: [vecs][n/32])
    float *g;          // [1], or [ceil(vecs/128)] with strip-local scales
    int tiled;         // MXFP4 only: codes [n/128][vecs][64], scales [n/128][vecs][4]
};

struct QuantArgs {
    const uint16_t *x;
    int64_t R, C;
    LayoutOut out[2];          // [0] row layout, [1] column layout
    // fp32 bits of max |r| (phase 1 output): [0] row, [1] column when nparts == 0; else
    // [nparts][2] the maxima of each phase-1 workgroup, reduced by every phase-2 workgroup;
    // with strip-local scales, [tile][layout][wave] the maximum of each of the 4 waves of a
    // layout over each tile
    uint32_t *amax_bits;
    int64_t nparts;
    // strip-local scales: [tiles_r row strips, then tiles_c column strips][128] scale tables
    float4 *tables;
    uint64_t seed, rht_seed;
    int64_t tiles_r, tiles_c, tiles;   // tile rows, tiles per tile row, total tiles
    int64_t blk_c;             // blocks of blk x blk tiles per block row (tiles_c / blk)
    int blk;                   // block edge of the visiting order, 4 or 1
};

// Waves per workgroup: 4 per layout (128 groups x 2 halves = 256 lanes per layout).
constexpr int waves_for(int lay) { return lay == LAY_BOTH ? 8 : 4; }

// Lane roles: each layout takes 256 lanes (128 groups x 2 halves) of a workgroup.
struct Role {
    int lay;   // 0 row layout, 1 column layout (wave-uniform)
    int g;     // group (row or column) within the tile, 0..127
    int h;     // half of the group held by this lane
};

template <int LAY>
__device__ __forceinline__ Role lane_role()
{
    const int t = threadIdx.x;
    Role ro;
    // wave-uniform, so the two layouts take scalar branches instead of masked execution
    ro.lay = __builtin_amdgcn_readfirstlane((LAY == LAY_BOTH) ? (t >> 8)
                                                               : (LAY == LAY_ROW ? 0 : 1));
    ro.g = (t & 255) >> 1;
    ro.h = t & 1;
    return ro;
}

// ------------------------------------------------------------------------------ kernels
__global__ void k_zero_u32(uint32_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// Tensor scales of an empty input: g = amax / D for each requested layout.
__global__ void k_write_g(const uint32_t *amax_bits, float D, float *g0, float *g1)
{
    if (threadIdx.x == 0) {
        if (g0) *g0 = __uint_as_float(amax_bits[0]) / D;
        if (g1) *g1 = __uint_as_float(amax_bits[1]) / D;
    }
}

// The order in which the tiles are visited.  Order index o names a tile: when both tile
// counts are multiples of 4 (a.blk = 4) the tiles are taken in 4 x 4 blocks, block by block
// in row-major order and row-major inside a block; otherwise (a.blk = 1) plainly row-major.
// A workgroup visits o = j, j + s, j + 2s, ... (s = gridDim.x, a multiple of 16 when
// blocked), or the same indices counted back from the last, so it keeps one place inside
// every block it visits and moves a fixed number of blocks per step: a step is a few
// wave-uniform additions instead of a 64-bit division per tile.
//
// j is the workgroup's place in a step.  Workgroups are dispatched to the 8 XCDs round robin
// (workgroup w on XCD w mod 8), so when a step holds whole groups of 8 x 16 workgroups
// the 16 tiles of each block go to 16 workgroups of one XCD, which process them at the same
// time: the four 8-byte scale pieces of a 32-byte sector (a vector's scales from 4 tiles in
// a row of a block for the row layout, in a column for the column layout) then meet in that
// XCD's L2 and leave it as one sector.
struct TileWalk {
    int64_t br, bc;      // current block row and column
    int64_t dq, dr;      // blocks per step: (s / blk^2) / blk_c, (s / blk^2) % blk_c
    int ir, ic;          // the tile's place inside its block
};

__device__ __forceinline__ int64_t first_order_index(const QuantArgs &a)
{
    const int64_t w = blockIdx.x, s = gridDim.x;
    if (a.blk == 1 || (s & 127)) return w;
    const int64_t xcd = w & 7, slot = w >> 3;
    return 16 * ((slot >> 4) * 8 + xcd) + (slot & 15);
}

__device__ __forceinline__ TileWalk tile_walk(const QuantArgs &a, int64_t o)
{
    const int bb = a.blk * a.blk;
    const int64_t blk_idx = o / bb, sb = (int64_t)gridDim.x / bb;
    const int i = (int)(o - blk_idx * bb);
    return TileWalk{blk_idx / a.blk_c, blk_idx % a.blk_c, sb / a.blk_c, sb % a.blk_c,
                    i / a.blk, i % a.blk};
}

__device__ __forceinline__ int64_t walk_r0(const QuantArgs &a, const TileWalk &w)
{
    return (w.br * a.blk + w.ir) * TILE;
}

__device__ __forceinline__ int64_t walk_c0(const QuantArgs &a, const TileWalk &w)
{
    return (w.bc * a.blk + w.ic) * TILE;
}

__device__ __forceinline__ void walk_forward(const QuantArgs &a, TileWalk &w)
{
    w.br += w.dq;
    w.bc += w.dr;
    if (w.bc >= a.blk_c) { w.bc -= a.blk_c; ++w.br; }
}

__device__ __forceinline__ void walk_back(const QuantArgs &a, TileWalk &w)
{
    w.br -= w.dq;
    w.bc -= w.dr;
    if (w.bc < 0) { w.bc += a.blk_c; --w.br; }
}

// Max |r| over this lane's half group of tile (r0, c0).
template <bool ROT>
__device__ __forceinline__ float tile_amax(const Tile &tile, const SignTable &st,
                                           const QuantArgs &a, const Role &ro, int64_t r0,
                                           int64_t c0)
{
    const bool valid = (ro.lay == 0) ? (r0 + ro.g < a.R) : (c0 + ro.g < a.C);
    if (!valid) return 0.0f;
    float r[HALF];
    if (ro.lay == 0) read_row_half(tile, st, ro.g, ro.h, r);
    else read_col_half(tile, st, ro.g, ro.h, r);
    if (ROT) return fwht_pair_absmax(r, ro.h);
    float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
    for (int p = 0; p < HALF; p += 4) {
        m0 = fmaxf(m0, fmaxf(fabsf(r[p]), fabsf(r[p + 1])));
        m1 = fmaxf(m1, fmaxf(fabsf(r[p + 2]), fabsf(r[p + 3])));
    }
    return fmaxf(m0, m1);
}

// Strip of tile (r0, c0) for layout lay: its table index among the row strips, then the
// column strips.
__device__ __forceinline__ int64_t strip_slot(const QuantArgs &a, int lay, int64_t r0,
                                              int64_t c0)
{
    return lay == 0 ? r0 / TILE : a.tiles_r + c0 / TILE;
}

// Maximum over the wave: rotations within each row of 16 lanes (DPP row_ror 1, 2, 4, 8), then
// the four rows' results read out.  No LDS round trips.
__device__ __forceinline__ float wave_max(float m)
{
#define ROR_MAX(n) { const int v = __builtin_bit_cast(int, m); \
        m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(v, v, 0x120 + (n), \
                                                                          0xF, 0xF, false))); }
    ROR_MAX(1);
    ROR_MAX(2);
    ROR_MAX(4);
    ROR_MAX(8);
#undef ROR_MAX
    const int b = __builtin_bit_cast(int, m);
    return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
}

// Strip-local scales: each wave stores its maximum over tile (r0, c0) (4 waves per layout).
__device__ __forceinline__ void store_wave_max(const QuantArgs &a, const Role &ro, int64_t r0,
                                               int64_t c0, float m)
{
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) {
        const int64_t tile = (r0 / TILE) * a.tiles_c + c0 / TILE;
        a.amax_bits[tile * 8 + 4 * ro.lay + ((threadIdx.x >> 6) & 3)] = __float_as_uint(m);
    }
}

// Pass 1: amax of |r| per layout.  Persistent workgroups walk the tiles with two LDS
// buffers (the next tile streams in while the current one is processed).  At the end each
// workgroup stores its two maxima in its own slots (nparts > 0), or takes one atomicMax per
// layout into amax_bits[0..1] (nparts == 0: the caller cleared them); with LOCAL, one store
// per wave and tile instead.
template <bool ROT, int LAY, bool LOCAL>
__global__ void __launch_bounds__(512, 4) k_amax(QuantArgs a)
{
    __shared__ Tile tile0;
    __shared__ Tile tile1;
    __shared__ SignTable st;
    __shared__ uint32_t wmax[2];
    const int t = threadIdx.x;
    const Role ro = lane_role<LAY>();
    constexpr int WAVES = waves_for(LAY);
    const DmaLane dl = dma_lane<WAVES>(a.C);
    build_sign_table(st, a.rht_seed, ROT);
    if (t < 2) wmax[t] = 0u;
    float local = 0.0f;
    int64_t k = first_order_index(a), r0 = 0, c0 = 0;
    TileWalk tw{0, 0, 0, 0, 0, 0};
    if (k < a.tiles) {
        tw = tile_walk(a, k);
        r0 = walk_r0(a, tw);
        c0 = walk_c0(a, tw);
        stage_tile<WAVES>(tile0, a.x, a.R, a.C, r0, c0, dl);
    }
    while (k < a.tiles) {
        const int64_t k1 = k + gridDim.x;
        __syncthreads();                                   // tile0 landed; tile1 is free
        int64_t r1 = 0, c1 = 0;
        walk_forward(a, tw);                               // tile k1
        if (k1 < a.tiles) {
            r1 = walk_r0(a, tw);
            c1 = walk_c0(a, tw);
            stage_tile<WAVES>(tile1, a.x, a.R, a.C, r1, c1, dl);
        }
        {
            const float m = tile_amax<ROT>(tile0, st, a, ro, r0, c0);
            if constexpr (LOCAL) store_wave_max(a, ro, r0, c0, m);
            else local = fmaxf(local, m);
        }
        if (k1 >= a.tiles) break;
        const int64_t k2 = k1 + gridDim.x;
        __syncthreads();                                   // tile1 landed; tile0 is free
        walk_forward(a, tw);                               // tile k2
        if (k2 < a.tiles) {
            r0 = walk_r0(a, tw);
            c0 = walk_c0(a, tw);
            stage_tile<WAVES>(tile0, a.x, a.R, a.C, r0, c0, dl);
        }
        {
            const float m = tile_amax<ROT>(tile1, st, a, ro, r1, c1);
            if constexpr (LOCAL) store_wave_max(a, ro, r1, c1, m);
            else local = fmaxf(local, m);
        }
        k = k2;
    }
    if constexpr (LOCAL) return;
    // wave max, then one atomic per wave into LDS, one per workgroup and layout into memory
    for (int off = 32; off > 0; off >>= 1) local = fmaxf(local, __shfl_xor(local, off));
    __syncthreads();
    if ((t & 63) == 0) atomicMax(&wmax[ro.lay], __float_as_uint(local));
    __syncthreads();
    if (a.nparts > 0) {
        if (t < 2) a.amax_bits[2 * blockIdx.x + t] = wmax[t];    // 0 for a layout not run
    } else if (t == 0) {
        if (LAY & LAY_ROW) atomicMax(&a.amax_bits[0], wmax[0]);
        if (LAY & LAY_COL) atomicMax(&a.amax_bits[1], wmax[1]);
    }
}

// fp32 bits of the maximum |r| of layout lay (wave-uniform): the phase-1 result, or the
// largest of the per-workgroup maxima.  Compared as unsigned integers, as the atomics do.
__device__ __forceinline__ uint32_t layout_amax_bits(const QuantArgs &a, int lay)
{
    if (a.nparts == 0) return a.amax_bits[lay];
    const int lane = threadIdx.x & 63;
    uint32_t m0 = 0u, m1 = 0u;
    int64_t i = lane;
    for (; i + 64 < a.nparts; i += 128) {
        m0 = max(m0, a.amax_bits[2 * i + lay]);
        m1 = max(m1, a.amax_bits[2 * (i + 64) + lay]);
    }
    if (i < a.nparts) m0 = max(m0, a.amax_bits[2 * i + lay]);
    uint32_t m = max(m0, m1);
#define ROR_UMAX(n) m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x120 + (n), \
                                                                    0xF, 0xF, false));
    ROR_UMAX(1);
    ROR_UMAX(2);
    ROR_UMAX(4);
    ROR_UMAX(8);
#undef ROR_UMAX
    return max(max((uint32_t)__builtin_amdgcn_readlane((int)m, 0),
                   (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
               max((uint32_t)__builtin_amdgcn_readlane((int)m, 32),
                   (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
}

// Round-to-nearest of one 1x16 block rb[0..15] with scale code s (table entry e):
// packed codes into w0 (elements 0..7) and w1 (8..15); a zero scale gives all-zero codes
// (its table rcp is 0).
// y = fma(r, rcp, +0) is r * rcp rounded once, except that an exact zero becomes +0, so
// the code's sign bit is set iff r < 0.
__device__ __forceinline__ float scaled(float r, float rcp) { return __builtin_fmaf(r, rcp, 0.0f); }

__device__ __forceinline__ void rtn_block(const float *rb, uint32_t s, const float4 e,
                                          uint32_t &w0, uint32_t &w1)
{
    const float rcp = e.z;
    // the four conversions into a word write its four bytes, so the bits the first one
    // leaves in place never survive: it is seeded with its own first input instead of a
    // zero that would cost a move
    const float y0 = scaled(rb[0], rcp), y8 = scaled(rb[8], rcp);
    uint32_t a = __float_as_uint(y0), b = __float_as_uint(y8);
    a = CVT_FP4(a, y0, scaled(rb[1], rcp), 0);
    a = CVT_FP4(a, scaled(rb[2], rcp), scaled(rb[3], rcp), 1);
    a = CVT_FP4(a, scaled(rb[4], rcp), scaled(rb[5], rcp), 2);
    a = CVT_FP4(a, scaled(rb[6], rcp), scaled(rb[7], rcp), 3);
    b = CVT_FP4(b, y8, scaled(rb[9], rcp), 0);
    b = CVT_FP4(b, scaled(rb[10], rcp), scaled(rb[11], rcp), 1);
    b = CVT_FP4(b, scaled(rb[12], rcp), scaled(rb[13], rcp), 2);
    b = CVT_FP4(b, scaled(rb[14], rcp), scaled(rb[15], rcp), 3);
    w0 = a;      // s = 0: rcp = 0, so every code is 0x0 already
    w1 = b;
}

// Signed grid values of a block's 16 codes.
template <int K>
__device__ __forceinline__ void decode_pair(uint32_t w0, uint32_t w1, float V[16])
{
    const float2v v0 = DEC_FP4(w0, K), v1 = DEC_FP4(w1, K);
    V[2 * K] = v0.x;
    V[2 * K + 1] = v0.y;
    V[8 + 2 * K] = v1.x;
    V[8 + 2 * K + 1] = v1.y;
}

__device__ __forceinline__ void decode_block(uint32_t w0, uint32_t w1, float V[16])
{
    decode_pair<0>(w0, w1, V);
    decode_pair<1>(w0, w1, V);
    decode_pair<2>(w0, w1, V);
    decode_pair<3>(w0, w1, V);
}

// Squared error of one block's RTN option: d_i = q_i - r_i with q_i = den * V_i (the option's
// dequantized value, rounded once), each d_i^2 rounded once, summed pairwise over the 16.
__device__ __forceinline__ float block_sq_error(const float *r, uint32_t w0, uint32_t w1,
                                                float den)
{
    float V[16], d2[16];
    decode_block(w0, w1, V);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float d = den * V[i] - r[i];
        d2[i] = d * d;
    }
    return tree<16>(d2);
}

// Saturate magnitude 7 (value 6) to 6 (value 4) in every nibble of a packed word.
__device__ __forceinline__ uint32_t cap_mag6(uint32_t w)
{
    const uint32_t seven = w & (w >> 1) & (w >> 2) & 0x11111111u;
    return w ^ seven;
}

// Quantize this lane's half group: blocks 4h..4h+3 of the group in r[0..63] (rotated when
// the mode rotates), their maxima of |r| in bmax; nbl = number of those blocks inside the
// vector.  vec = vector index in
// its layout, n = vector length, gi = group index within the vector.  Writes this half's
// 32 code bytes and 4 scale bytes (codes/scales point at the group's first byte).
template <int MODE>
__device__ __forceinline__ void quantize_half(float r[HALF], const float bmax[4], int h,
                                              int nbl, float g,
                                              const ScaleTable &tb, float rcp6g, float rcp4g,
                                              uint64_t seed, uint32_t axis, int64_t vec,
                                              int64_t n, int64_t gi,
                                              uint8_t *__restrict__ codes,
                                              uint8_t *__restrict__ scales)
{
    uint32_t cw[8];
    uint32_t sc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) { sc[b] = 0u; cw[2 * b] = 0u; cw[2 * b + 1] = 0u; }

    if constexpr (MODE == MODE_RTN || MODE == MODE_EDEN) {
        float bp[4], bq[4], sv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            bp[b] = 0.0f; bq[b] = 0.0f; sv[b] = 0.0f;
            if (MODE == MODE_EDEN || b < nbl) {
                const float *rb = r + 16 * b;
                const uint32_t s = e4m3_rne_hw(bmax[b] * rcp6g);
                const float4 e = tb.e[s];
                rtn_block(rb, s, e, cw[2 * b], cw[2 * b + 1]);
                sc[b] = s;
                sv[b] = e.x;
                if constexpr (MODE == MODE_EDEN) {
                    // the block's terms of <r,r> and <r,q>, each rounded once: r_i * r_i and
                    // r_i * q_i with q_i = den * V_i (the RTN dequantization, rounded once),
                    // summed pairwise; the block is an aligned subtree of the group's tree
                    float V[16], P[16], Q[16];
                    decode_block(cw[2 * b], cw[2 * b + 1], V);
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        P[i] = rb[i] * rb[i];
                        Q[i] = rb[i] * (e.y * V[i]);
                    }
                    bp[b] = tree<16>(P);
                    bq[b] = tree<16>(Q);
                }
            }
        }
        if constexpr (MODE == MODE_EDEN) {
            // the group's 128-term pairwise sums: the blocks' sums (levels 1..4), two more
            // levels inside the half, the last across the pair (low half + high half in
            // both lanes)
            const float pn = tree<4>(bp), qn = tree<4>(bq);
            const float po = pair_swap(pn), qo = pair_swap(qn);
            const float num = h ? po + pn : pn + po;
            const float den = h ? qo + qn : qn + qo;
            const float S = den > 0.0f ? num / den : 1.0f;
            // scale index of this half's first block is a multiple of 4: one Philox block
            const uint64_t j = ((uint64_t)(vec * (n >> 4) + gi * 8) >> 2) + (uint64_t)h;
            const Word4 w = philox(seed, (uint32_t)j, (uint32_t)(j >> 32), STREAM_SCALE_SR, axis);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float c = S * sv[b];
                uint32_t out;
                if (!(c < 448.0f)) out = 0x7Eu;
                else if (c < 0.015625f) out = e4m3_rne_hw(c);      // no SR below 2^-6
                else out = e4m3_sr_normal(__float_as_uint(c), w.w[b]);
                // a zero scale stays zero even where S is not finite (inputs beyond 2^56)
                sc[b] = sc[b] ? out : 0u;
            }
        }
    } else if constexpr (MODE == MODE_SR) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (b < nbl) {
                const float *rb = r + 16 * b;
                const uint32_t s = e4m3_up(bmax[b] * rcp6g);
                const float rcp = tb.e[s].z;
                sc[b] = s;
                if (s) {
                    // element index of the block's first element, a multiple of 4
                    const int64_t e0 = vec * n + gi * TILE + HALF * h + 16 * b;
#pragma unroll
                    for (int d = 0; d < 2; ++d) {   // 8 elements, two Philox calls
                        uint32_t ws[8];
                        float y[8];
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            const uint64_t j = ((uint64_t)e0 >> 2) + 2 * d + c;
                            const Word4 w = philox(seed, (uint32_t)j, (uint32_t)(j >> 32),
                                                   STREAM_ELEM_SR, axis);
#pragma unroll
                            for (int k = 0; k < 4; ++k) ws[4 * c + k] = w.w[k];
                        }
#pragma unroll
                        for (int k = 0; k < 8; ++k) y[k] = scaled(rb[8 * d + k], rcp);
                        cw[2 * b + d] = e2m1_sr_pack8(y, ws);
                    }
                }
            }
        }
    } else {   // MODE_FP46
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (b < nbl) {
                const float *rb = r + 16 * b;
                const float m = bmax[b];
                const uint32_t sA = e4m3_rne_hw(m * rcp6g), sB = e4m3_rne_hw(m * rcp4g);
                const float4 eA = tb.e[sA], eB = tb.e[sB];
                uint32_t a0, a1, b0, b1;
                rtn_block(rb, sA, eA, a0, a1);
                rtn_block(rb, sB, eB, b0, b1);
                b0 = cap_mag6(b0);
                b1 = cap_mag6(b1);
                const float errA = block_sq_error(rb, a0, a1, eA.y);
                const float errB = block_sq_error(rb, b0, b1, eB.y);
                const bool pickA = errA <= errB;
                sc[b] = pickA ? sA : sB;
                cw[2 * b] = pickA ? a0 : b0;
                cw[2 * b + 1] = pickA ? a1 : b1;
            }
        }
    }

    // ---- stores: this half's 32 code bytes and 4 scale bytes
    if (nbl == 4 && (n & (TILE - 1)) == 0) {
        uint4 *cp = reinterpret_cast<uint4 *>(codes + 32 * h);
        cp[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
        cp[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
        *reinterpret_cast<uint32_t *>(scales + 4 * h) =
            sc[0] | (sc[1] << 8) | (sc[2] << 16) | (sc[3] << 24);
    } else {
        uint2 *cp = reinterpret_cast<uint2 *>(codes + 32 * h);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (b < nbl) {
                cp[b] = make_uint2(cw[2 * b], cw[2 * b + 1]);
                scales[4 * h + b] = (uint8_t)sc[b];
            }
        }
    }
}

// ------------------------------------------------------------------------------ MXFP4
// The MXFP4 block contract, the operand format of gfx950's scaled matrix instructions: blocks
// of 32 with one power-of-two (E8M0) scale 2^e, e the smallest integer with 6 * 2^e >= max |r|
// over the block (clamped to [-127, 127]; an all-zero block gets -127), elements
// y = r * 2^-e rounded onto the E2M1 grid by RTN or SR.
//
// This lane's two 32-blocks of a group (positions 64h .. 64h + 63 of r, their 16-block maxima
// in bmax); nbl = 16-blocks inside the vector (even).  Writes 32 code bytes and 2 scale bytes.
template <bool SR>
__device__ __forceinline__ void quantize_half_mx(const float r[HALF], const float bmax[4],
                                                 int h, int nbl, uint64_t seed, uint32_t axis,
                                                 int64_t vec, int64_t n, int64_t gi,
                                                 uint8_t *__restrict__ codes,
                                                 uint8_t *__restrict__ scales, bool aligned)
{
    uint32_t cw[8];
    uint32_t sc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        sc[b] = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) cw[4 * b + k] = 0u;
        if (2 * b < nbl) {
            const float *rb = r + 32 * b;
            const int e = mx_scale_exp(fmaxf(bmax[2 * b], bmax[2 * b + 1]));
            sc[b] = (uint32_t)(e + 127);
            const float p = __builtin_amdgcn_ldexpf(1.0f, -e);     // exact, normal
            if constexpr (!SR) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float *q = rb + 8 * k;
                    const float y0 = scaled(q[0], p);
                    uint32_t w = __float_as_uint(y0);
                    w = CVT_FP4(w, y0, scaled(q[1], p), 0);
                    w = CVT_FP4(w, scaled(q[2], p), scaled(q[3], p), 1);
                    w = CVT_FP4(w, scaled(q[4], p), scaled(q[5], p), 2);
                    w = CVT_FP4(w, scaled(q[6], p), scaled(q[7], p), 3);
                    cw[4 * b + k] = w;
                }
            } else {
                // element index of the block's first element, a multiple of 4
                const int64_t e0 = vec * n + gi * TILE + HALF * h + 32 * b;
#pragma unroll
                for (int d = 0; d < 4; ++d) {   // 8 elements, two Philox calls
                    uint32_t ws[8];
                    float y[8];
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const uint64_t j = ((uint64_t)e0 >> 2) + 2 * d + c;
                        const Word4 w = philox(seed, (uint32_t)j, (uint32_t)(j >> 32),
                                               STREAM_ELEM_SR, axis);
#pragma unroll
                        for (int k = 0; k < 4; ++k) ws[4 * c + k] = w.w[k];
                    }
#pragma unroll
                    for (int k = 0; k < 8; ++k) y[k] = scaled(rb[8 * d + k], p);
                    cw[4 * b + d] = e2m1_sr_pack8(y, ws);
                }
            }
        }
    }
    if (nbl == 4 && aligned) {
        uint4 *cp = reinterpret_cast<uint4 *>(codes + 32 * h);
        cp[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
        cp[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
        *reinterpret_cast<uint16_t *>(scales + 2 * h) = (uint16_t)(sc[0] | (sc[1] << 8));
    } else {
        uint2 *cp = reinterpret_cast<uint2 *>(codes + 32 * h);
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (b < nbl) cp[b] = make_uint2(cw[2 * b], cw[2 * b + 1]);
#pragma unroll
        for (int b = 0; b < 2; ++b)
            if (2 * b < nbl) scales[2 * h + b] = (uint8_t)sc[b];
    }
}

// Quantize this lane's half group of tile (r0, c0); tb holds the tile's scale table and
// its (g, rcp(6g), rcp(4g)).
//
// next() runs once the tile's LDS reads are issued (every lane reads, those past the edge
// too): the two-buffer loop starts the following tile's loads there.  Issued after the reads,
// those loads into the other buffer can never hold the reads back, whereas issued before them
// the compiler may not be able to tell which buffer they fill and wait for them first.
template <int MODE, bool ROT, typename Next>
__device__ __forceinline__ void tile_quant(const Tile &tile, const SignTable &st,
                                           const ScaleTable &tb, const QuantArgs &a,
                                           const LayoutOut &o, const Role &ro, int64_t r0,
                                           int64_t c0, Next next)
{
    const int64_t n = ro.lay == 0 ? a.C : a.R;
    const int64_t vec = ro.lay == 0 ? r0 + ro.g : c0 + ro.g;
    const int64_t start = ro.lay == 0 ? c0 : r0;       // first position of this group
    float r[HALF];
    if (ro.lay == 0) read_row_half(tile, st, ro.g, ro.h, r);
    else read_col_half(tile, st, ro.g, ro.h, r);
    __asm__ volatile("" ::: "memory");
    next();
    __asm__ volatile("" ::: "memory");                 // the loads stay before the stores
    if (vec >= (ro.lay == 0 ? a.R : a.C)) return;
    float bm[4];
    if (ROT) {
        fwht_pair_blocks(r, ro.h, bm);
    } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) bm[b] = block_max(r + 16 * b);
    }
    const int64_t left = n - start;
    const int nb = left >= TILE ? 8 : (int)(left >> 4);
    const int nbl = nb - 4 * ro.h < 0 ? 0 : (nb - 4 * ro.h > 4 ? 4 : nb - 4 * ro.h);
    if constexpr (is_mx(MODE)) {
        // this group's 64 code bytes and 4 scale bytes: in the vector's row, or (K-tiled, n a
        // multiple of 128) in the vector's slot of the group's K tile
        const int64_t vecs = ro.lay == 0 ? a.R : a.C;
        uint8_t *cg = o.tiled ? o.codes + (start >> 7) * vecs * 64 + vec * 64
                              : o.codes + vec * (n >> 1) + (start >> 1);
        uint8_t *sg = o.tiled ? o.scales + (start >> 7) * vecs * 4 + vec * 4
                              : o.scales + vec * (n >> 5) + (start >> 5);
        quantize_half_mx<MODE == MODE_MX_SR>(r, bm, ro.h, nbl, a.seed, (uint32_t)ro.lay, vec, n,
                                             start / TILE, cg, sg, (n & (TILE - 1)) == 0);
    } else {
        const float4 gs = tb.e[TAB_G];
        quantize_half<MODE>(r, bm, ro.h, nbl, gs.x, tb, gs.y, gs.z, a.seed, (uint32_t)ro.lay, vec,
                            n, start / TILE, o.codes + vec * (n >> 1) + (start >> 1),
                            o.scales + vec * (n >> 4) + (start >> 4));
    }
}

// Workgroup barrier between tiles of pass 2 that does not wait for the tile's code and scale
// stores.  __syncthreads would wait for every outstanding memory operation of the wave,
// stores included, so each tile would pay the write latency.  The vector memory counter
// retires in issue order, so waiting until at most `stores` operations are outstanding, where
// the last `stores` the wave issued are its stores of the tile just computed, waits for the
// wave's loads into LDS (issued before them) and nothing younger; lgkmcnt(0) waits for its
// LDS reads and writes.  The empty asm statements keep the compiler from moving memory
// operations across the barrier.
template <int STORES>
__device__ __forceinline__ void tile_barrier()
{
    // s_waitcnt fields (gfx9): vmcnt bits 3:0 and 15:14, expcnt 6:4 (7 = no wait), lgkmcnt 11:8
    constexpr int IMM = (STORES & 15) | (7 << 4) | (0 << 8) | (((STORES >> 4) & 3) << 14);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(IMM);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// The barrier before reading a tile whose loads were issued before the wave's last tile
// computation: that computation issued exactly 3 stores (two 16-byte code stores and one
// 4-byte scale store, the full-tile path of quantize_half) when the tile was full and the
// vectors a multiple of 128 long; otherwise wait for everything.
__device__ __forceinline__ void tile_barrier_after(bool three_stores)
{
    if (three_stores) tile_barrier<3>();
    else tile_barrier<0>();
}

// Pass 2: quantize and pack every group of the requested layouts.  Tiles are walked in
// the reverse order of pass 1 (its last tiles are the likeliest to still be cached), with
// the same two-buffer streaming for one layout and for both.
// Waves per SIMD each variant is compiled for: with both layouts (8 waves per workgroup) the
// most that fit without spilling, 4 (128 registers) for MS-EDEN, RTN, 4/6 and the unrotated
// SR, 3 (168) for SR with the rotation.  With one layout (4 waves) the two 32 KiB tile
// buffers leave room for two workgroups per CU, i.e. 2 waves per SIMD, so those variants may
// use up to 256 registers.
constexpr int quant_waves_per_simd(int mode, bool rot, int lay)
{
    if (lay != LAY_BOTH) return 2;
    if ((mode == MODE_SR || mode == MODE_MX_SR) && rot) return 3;
    return 4;
}

// Between the passes with strip-local scales: workgroup `slot` reduces the wave maxima of its
// strip (row strip s: the tiles of tile row s; column strip s: of tile column s), stores the
// strip's g into its layout's output and writes the strip's scale table.
__global__ void __launch_bounds__(256) k_strip_tables(QuantArgs a, int layouts, float D)
{
    __shared__ float wm[4];
    const int64_t slot = blockIdx.x;
    const bool row = slot < a.tiles_r;
    if (!(layouts & (row ? LAY_ROW : LAY_COL))) return;
    const int64_t s = row ? slot : slot - a.tiles_r;
    const int64_t count = 4 * (row ? a.tiles_c : a.tiles_r);
    float m = 0.0f;
    for (int64_t i = threadIdx.x; i < count; i += 256) {
        const int64_t other = i >> 2;
        const int64_t tile = row ? s * a.tiles_c + other : other * a.tiles_c + s;
        m = fmaxf(m, __uint_as_float(a.amax_bits[tile * 8 + (row ? 0 : 4) + (i & 3)]));
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
    __syncthreads();
    const float g = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3])) / D;
    const LayoutOut o = row ? a.out[0] : a.out[1];
    if (threadIdx.x == 0) o.g[s] = g;
    if (threadIdx.x < 128) a.tables[slot * 128 + threadIdx.x] = scale_entry(threadIdx.x, g);
}

// Strip-local scales: start copying the scale table of tile (r0, c0)'s strip for this lane's
// layout into tb: two wave instructions of 64 16-byte chunks, issued by the layout's first two
// waves.  Visible after the next __syncthreads, like the tile.
__device__ __forceinline__ void stage_table(ScaleTable &tb, const QuantArgs &a, const Role &ro,
                                            int64_t r0, int64_t c0)
{
    const int w = __builtin_amdgcn_readfirstlane((int)((threadIdx.x >> 6) & 3));
    if (w < 2) {
        const float4 *src = a.tables + strip_slot(a, ro.lay, r0, c0) * 128 + 64 * w +
                            (threadIdx.x & 63);
        __builtin_amdgcn_global_load_lds(src, LDS_PTR(&tb.e[64 * w]), 16, 0, 0);
    }
}

template <int MODE, bool ROT, int LAY, bool LOCAL>
__global__ void __launch_bounds__(512, quant_waves_per_simd(MODE, ROT, LAY))
k_quant(QuantArgs a)
{
    constexpr int NLAY = (LAY == LAY_BOTH) ? 2 : 1;
    __shared__ Tile tile0;
    __shared__ Tile tile1;
    __shared__ SignTable st;
    // one table per layout, and per tile buffer when every tile has its own scale
    __shared__ ScaleTable tabs[LOCAL ? 2 : 1][NLAY];
    const int t = threadIdx.x;
    const Role ro = lane_role<LAY>();
    constexpr int WAVES = waves_for(LAY);
    const DmaLane dl = dma_lane<WAVES>(a.C);
    const int li = (LAY == LAY_BOTH) ? ro.lay : 0;
    ScaleTable &tb0 = tabs[0][li];
    ScaleTable &tb1 = tabs[LOCAL ? 1 : 0][li];
    // select this lane's layout without indexing the argument struct at run time
    const LayoutOut o = (ro.lay == 0) ? a.out[0] : a.out[1];
    build_sign_table(st, a.rht_seed, ROT);
    int64_t k = first_order_index(a), r0 = 0, c0 = 0;
    // tiles in the reverse order of pass 1: order index tiles - 1 - k, walking back
    TileWalk tw{0, 0, 0, 0, 0, 0};
    if (k < a.tiles) tw = tile_walk(a, a.tiles - 1 - k);
    // the first tile streams in while the tensor scale is reduced and its table built
    if (k < a.tiles) {
        r0 = walk_r0(a, tw);
        c0 = walk_c0(a, tw);
        stage_tile<WAVES>(tile0, a.x, a.R, a.C, r0, c0, dl);
        if constexpr (LOCAL) stage_table(tb0, a, ro, r0, c0);
    }
    if constexpr (!LOCAL && !is_mx(MODE)) {
        const float D = (MODE == MODE_FP46) ? 1792.0f : 2688.0f;
        const float g = __uint_as_float(layout_amax_bits(a, ro.lay)) / D;
        build_scale_table(tb0, g, t & 255);
        if (blockIdx.x == 0 && (t & 255) == 0) *o.g = g;
    }
    // vectors of this wave's layout a multiple of 128 long: full tiles take the 3-store path
    const bool n128 = (((ro.lay == 0) ? a.C : a.R) & (TILE - 1)) == 0;
    bool three = false;               // the wave's last computation issued exactly 3 stores
    while (k < a.tiles) {
        const int64_t k1 = k + gridDim.x;
        tile_barrier_after(three);                         // tile0 landed; tile1 is free
        int64_t r1 = 0, c1 = 0;
        walk_back(a, tw);                                  // tile tiles - 1 - k1
        const bool more1 = k1 < a.tiles;
        if (more1) {
            r1 = walk_r0(a, tw);
            c1 = walk_c0(a, tw);
        }
        tile_quant<MODE, ROT>(tile0, st, tb0, a, o, ro, r0, c0, [&] {
            if (more1) {
                stage_tile<WAVES>(tile1, a.x, a.R, a.C, r1, c1, dl);
                if constexpr (LOCAL) stage_table(tb1, a, ro, r1, c1);
            }
        });
        three = n128 && r0 + TILE <= a.R && c0 + TILE <= a.C;
        if (!more1) break;
        const int64_t k2 = k1 + gridDim.x;
        tile_barrier_after(three);                         // tile1 landed; tile0 is free
        walk_back(a, tw);                                  // tile tiles - 1 - k2
        const bool more2 = k2 < a.tiles;
        if (more2) {
            r0 = walk_r0(a, tw);
            c0 = walk_c0(a, tw);
        }
        tile_quant<MODE, ROT>(tile1, st, tb1, a, o, ro, r1, c1, [&] {
            if (more2) {
                stage_tile<WAVES>(tile0, a.x, a.R, a.C, r0, c0, dl);
                if constexpr (LOCAL) stage_table(tb0, a, ro, r0, c0);
            }
        });
        three = n128 && r1 + TILE <= a.R && c1 + TILE <= a.C;
        k = k2;
    }
}

// Lane q ^ m of v within rows of 16 lanes (m = 1, 2, 4, 8): DPP for 1, 2 and 8, a
// swizzle for 4.
template <int M>
__device__ __forceinline__ float xor16(float v)
{
    const int b = __builtin_bit_cast(int, v);
    int r;
    if constexpr (M == 1) r = __builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false);
    else if constexpr (M == 2) r = __builtin_amdgcn_update_dpp(b, b, 0x4E, 0xF, 0xF, false);
    else if constexpr (M == 8) r = __builtin_amdgcn_update_dpp(b, b, 0x128, 0xF, 0xF, false);
    else r = __builtin_amdgcn_ds_swizzle(b, (M << 10) | 0x1F);
    return __builtin_bit_cast(float, r);
}

// One butterfly stage of span 8 M across lanes: the lower position takes a + b, the upper
// a - b (lower - upper), as fma(+-1, mine, partner) with one rounding.
template <int M>
__device__ __forceinline__ void cross_stage(float v[8], int q)
{
    const float sg = (q & M) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(sg, v[i], xor16<M>(v[i]));
}

// The same stage in one v_fmac_f32_dpp per value, for the spans whose partner lane a DPP
// pattern reaches (M = 1, 2: quad_perm; M = 8: row_ror 8), on values held up to a per-lane
// sign c (true value = c * w).  The partner holds the same c before the stage (the lanes
// differ only in bit M, and c depends on the lower bits), so sg * t_own + t_partner =
// (sg * c) * (w_own + sg * w_partner): w += sg * partner's w, rounded once, and c picks up sg.
// The s_nop gives the DPP reads their two wait states after the last write of v.
template <int M>
__device__ __forceinline__ void dpp_stage(float v[8], float sg)
{
#define DQ_DPP(k, ctl) "v_fmac_f32_dpp %" #k ", %" #k ", %8 " ctl " row_mask:0xf bank_mask:0xf\n\t"
#define DQ_STAGE(ctl)                                                                          \
    __asm__("s_nop 1\n\t" DQ_DPP(0, ctl) DQ_DPP(1, ctl) DQ_DPP(2, ctl) DQ_DPP(3, ctl)          \
            DQ_DPP(4, ctl) DQ_DPP(5, ctl) DQ_DPP(6, ctl) DQ_DPP(7, ctl)                         \
            : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),         \
              "+v"(v[6]), "+v"(v[7])                                                          \
            : "v"(sg))
    if constexpr (M == 1) DQ_STAGE("quad_perm:[1,0,3,2]");
    else if constexpr (M == 2) DQ_STAGE("quad_perm:[2,3,0,1]");
    else DQ_STAGE("row_ror:8");
#undef DQ_STAGE
#undef DQ_DPP
}

// Dequantize: 16 lanes per (vector, group), lane q holding positions 4q .. 4q + 3 and
// 64 + 4q .. 64 + 4q + 3, so that the codes (2 + 2 bytes) and the two 16-byte output pieces
// of neighbouring lanes are contiguous.  out[vec][pos] fp32.  g of vector v is gp[v >> g_shift] (one tensor scale: a
// shift that maps every vector to 0).  sgn: the rotation's 128 sign bits, drawn by the
// launcher (each wave here is too short to draw them itself: the scalar unit, shared by a
// CU's waves, would spend more on them than the wave spends on its 512 elements).  With
// the rotation, the butterfly runs spans 1, 2 and
// 64 inside the lane and spans 4 .. 32 across lanes q ^ 1 .. q ^ 8, in ascending order,
// each output a + b or a - b rounded once.  One group per row of 16 lanes and no loop: the waves
// end right after their stores, so no wave waits on its own writes (a persistent loop over
// groups measured 20% slower without the rotation).
template <bool ROT>
__global__ void __launch_bounds__(256) k_dequant(const uint8_t *__restrict__ codes,
                                                 const uint8_t *__restrict__ scales,
                                                 const float *__restrict__ gp, int g_shift,
                                                 int64_t vecs, int64_t n, Signs sgn,
                                                 float *__restrict__ out)
{
    const int64_t groups_per_vec = (n + TILE - 1) / TILE;
    const int64_t id = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
    const int q = threadIdx.x & 15;
    // the 16 lanes of a row share id: they leave together
    const int64_t groups = vecs * groups_per_vec;
    if (id >= groups) return;
    int64_t vec, gi;
    if (groups <= 0xFFFFFFFFll) {       // the usual case: a 32-bit division (uniform branch)
        const uint32_t id32 = (uint32_t)id, gpv32 = (uint32_t)groups_per_vec;
        vec = id32 / gpv32;
        gi = id32 - (uint32_t)vec * gpv32;
    } else {
        vec = id / groups_per_vec;
        gi = id % groups_per_vec;
    }
    const int64_t start = gi * TILE;
    const int len = (n - start) >= TILE ? TILE : (int)(n - start);
    // Lane q holds positions 4q + (i & 3) + 64 (i >> 2), i = 0..7: each of its two store
    // instructions then writes 256 contiguous bytes per row of 16 lanes (whole 32-byte
    // sectors).  len is a multiple of 16, so each quadruple is wholly inside or outside.
    const float gv = gp[vec >> g_shift];
    const uint8_t *cb = codes + vec * (n >> 1) + (start >> 1) + 2 * q;
    const uint8_t *sb = scales + vec * (n >> 4) + (start >> 4) + (q >> 2);
    float *ob = out + vec * n + start + 4 * q;
    if constexpr (!ROT) {
        // decode and store each quadruple in turn (decoding both first, then storing, took
        // 112 us instead of 101 us on c4's row layout)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (64 * half + 4 * q < len) {
                const uint32_t cw = *reinterpret_cast<const uint16_t *>(cb + 32 * half);
                const float den = e4m3_val(sb[4 * half]) * gv;
                const float2v V0 = DEC_FP4(cw, 0), V1 = DEC_FP4(cw, 1);
                *reinterpret_cast<float4 *>(ob + 64 * half) =
                    make_float4(den * V0.x, den * V0.y, den * V1.x, den * V1.y);
            }
        }
        return;
    }
    // With the rotation every group is whole (len = 128).
    float v[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint32_t cw = *reinterpret_cast<const uint16_t *>(cb + 32 * half);
        const float den = e4m3_val(sb[4 * half]) * gv;
        // signed grid values of the 4 codes (exact), times den: one rounding each
        const float2v V0 = DEC_FP4(cw, 0), V1 = DEC_FP4(cw, 1);
        v[4 * half] = den * V0.x;
        v[4 * half + 1] = den * V0.y;
        v[4 * half + 2] = den * V1.x;
        v[4 * half + 3] = den * V1.y;
    }
    // The butterfly in ascending spans, each output a + b or a - b rounded once: spans 1 and 2
    // inside each quadruple, spans 4 .. 32 across lanes q ^ 1 .. q ^ 8, span 64 between the
    // lane's two quadruples.
#pragma unroll
    for (int h = 1; h < 4; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if ((i & h) == 0) {
                const float u = v[i], w = v[i + h];
                v[i] = u + w;
                v[i + h] = u - w;
            }
        }
    }
    // spans 4, 8 and 32 leave the lane's values times c = sg1 * sg2 * sg8, which the sign
    // masks take back out (span 64, inside the lane, keeps the common factor)
    dpp_stage<1>(v, (q & 1) ? -1.0f : 1.0f);                  // span 4
    dpp_stage<2>(v, (q & 2) ? -1.0f : 1.0f);                  // span 8
    cross_stage<4>(v, q);                                      // span 16
    dpp_stage<8>(v, (q & 8) ? -1.0f : 1.0f);                  // span 32
#pragma unroll
    for (int i = 0; i < 4; ++i) {                              // span 64
        const float u = v[i], w = v[i + 4];
        v[i] = u + w;
        v[i + 4] = u - w;
    }
    const uint32_t c = (uint32_t)((q ^ (q >> 1) ^ (q >> 3)) & 1) << 31;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = __uint_as_float(__float_as_uint(v[i]) ^
                               sign_mask(sgn, 4 * q + (i & 3) + 64 * (i >> 2)) ^ c) *
               0.0078125f;
    // Streaming (non-temporal) stores: 100 us on c4's row layout (with lane q writing
    // positions 8q .. 8q + 7 instead: 114 us with them, 164 us without; the quantizer's code
    // stores got slower with them and keep ordinary stores).
    store_nt(reinterpret_cast<float4 *>(ob), make_float4(v[0], v[1], v[2], v[3]));
    store_nt(reinterpret_cast<float4 *>(ob + 64), make_float4(v[4], v[5], v[6], v[7]));
}

}  // namespace nvfp4k

// ------------------------------------------------------------------------------ launchers
// Called by the C ABI layer (nvfp4_api.cpp) after argument validation.
namespace nvfp4k {

// Compute units of the current device, looked up once per device.  The cache is a constant
// of the device: threads that race on a first lookup store the same value.
constexpr int MAX_DEVICES = 64;

static int cu_count()
{
    static std::atomic<int> cached[MAX_DEVICES];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return 256;
    int cus = cached[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

// Persistent grid: as many workgroups as can be resident at once (occupancy of this kernel
// at this block size), never more than there are tiles.
template <typename K>
static int grid_for(K kernel, int threads, int64_t tiles)
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    const int64_t cap = (int64_t)cu_count() * per_cu;
    return (int)(tiles < cap ? tiles : cap);
}

// Phase-1 workgroups at most (their maxima fill the quantizers' workspace).
constexpr int64_t MAX_PARTS = 2048;

// A grid for the blocked visiting order must be a multiple of 16 workgroups (each keeps
// one place inside the blocks it visits): round it down, or visit row-major if it would
// vanish.
static void fit_grid(QuantArgs &a, int64_t &grid)
{
    if (a.blk == 1) return;
    if (grid >= 16) {
        grid -= grid % 16;
    } else {
        a.blk = 1;
        a.blk_c = a.tiles_c;
    }
}

// Returns the number of workgroups launched.
template <bool ROT, int LAY, bool LOCAL>
static int64_t launch_amax(const QuantArgs &args, hipStream_t st)
{
    QuantArgs a = args;
    const int threads = 64 * waves_for(LAY);
    int64_t grid = grid_for(k_amax<ROT, LAY, LOCAL>, threads, a.tiles);
    if (grid > MAX_PARTS) grid = MAX_PARTS;
    fit_grid(a, grid);
    k_amax<ROT, LAY, LOCAL><<<(unsigned)grid, threads, 0, st>>>(a);
    return grid;
}

template <bool ROT, bool LOCAL>
static int64_t amax_lay(const QuantArgs &a, int lay, hipStream_t st)
{
    if (lay == LAY_ROW) return launch_amax<ROT, LAY_ROW, LOCAL>(a, st);
    if (lay == LAY_COL) return launch_amax<ROT, LAY_COL, LOCAL>(a, st);
    return launch_amax<ROT, LAY_BOTH, LOCAL>(a, st);
}

template <int MODE, bool ROT, int LAY, bool LOCAL>
static void launch_quant(const QuantArgs &args, hipStream_t st)
{
    QuantArgs a = args;
    const int threads = 64 * waves_for(LAY);
    int64_t grid = grid_for(k_quant<MODE, ROT, LAY, LOCAL>, threads, a.tiles);
    fit_grid(a, grid);
    k_quant<MODE, ROT, LAY, LOCAL><<<(unsigned)grid, threads, 0, st>>>(a);
}

template <int MODE, bool ROT, bool LOCAL>
static void quant_lay(const QuantArgs &a, int lay, hipStream_t st)
{
    if (lay == LAY_ROW) launch_quant<MODE, ROT, LAY_ROW, LOCAL>(a, st);
    else if (lay == LAY_COL) launch_quant<MODE, ROT, LAY_COL, LOCAL>(a, st);
    else launch_quant<MODE, ROT, LAY_BOTH, LOCAL>(a, st);
}

template <bool LOCAL>
static void quant_mode(const QuantArgs &a, int mode, int rht, int lay, hipStream_t st)
{
    switch (mode) {
    case MODE_RTN: rht ? quant_lay<MODE_RTN, true, LOCAL>(a, lay, st)
                       : quant_lay<MODE_RTN, false, LOCAL>(a, lay, st); break;
    case MODE_SR: rht ? quant_lay<MODE_SR, true, LOCAL>(a, lay, st)
                      : quant_lay<MODE_SR, false, LOCAL>(a, lay, st); break;
    case MODE_EDEN: quant_lay<MODE_EDEN, true, LOCAL>(a, lay, st); break;
    default: rht ? quant_lay<MODE_FP46, true, LOCAL>(a, lay, st)
                 : quant_lay<MODE_FP46, false, LOCAL>(a, lay, st); break;
    }
}

static QuantArgs make_args(const void *x, int64_t R, int64_t C, uint32_t *amax_bits,
                           uint64_t seed, uint64_t rht_seed)
{
    QuantArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.R = R;
    a.C = C;
    a.out[0] = {nullptr, nullptr, nullptr};
    a.out[1] = {nullptr, nullptr, nullptr};
    a.amax_bits = amax_bits;
    a.nparts = 0;
    a.tables = nullptr;
    a.seed = seed;
    a.rht_seed = rht_seed;
    a.tiles_r = (R + TILE - 1) / TILE;
    a.tiles_c = (C + TILE - 1) / TILE;
    a.tiles = a.tiles_c * a.tiles_r;
    a.blk = (a.tiles_r % 4 == 0 && a.tiles_c % 4 == 0) ? 4 : 1;
    a.blk_c = a.tiles_c / a.blk;
    return a;
}

}  // namespace nvfp4k

// Phase 1: amax[0..1] <- max |r| of the requested layouts (0 for the others).
extern "C" hipError_t nvfp4k_amax(int rht, int layouts, const void *x, int64_t R, int64_t C,
                                  float *amax, uint64_t rht_seed, hipStream_t st)
{
    using namespace nvfp4k;
    QuantArgs a = make_args(x, R, C, reinterpret_cast<uint32_t *>(amax), 0, rht_seed);
    k_zero_u32<<<1, 64, 0, st>>>(a.amax_bits, 2);
    if (a.tiles > 0) rht ? amax_lay<true, false>(a, layouts, st) : amax_lay<false, false>(a, layouts, st);
    return hipGetLastError();
}

// Phase 2: quantize given the phase-1 maxima.
extern "C" hipError_t nvfp4k_quant(int mode, int rht, int layouts, const void *x, int64_t R,
                                   int64_t C, uint8_t *codes0, uint8_t *scales0, float *g0,
                                   uint8_t *codes1, uint8_t *scales1, float *g1,
                                   const float *amax, uint64_t seed, uint64_t rht_seed,
                                   hipStream_t st)
{
    using namespace nvfp4k;
    if (mode < MODE_RTN || mode > MODE_FP46) return hipErrorInvalidValue;
    QuantArgs a = make_args(x, R, C, reinterpret_cast<uint32_t *>(const_cast<float *>(amax)),
                            seed, rht_seed);
    a.out[0] = {codes0, scales0, g0};
    a.out[1] = {codes1, scales1, g1};
    if (a.tiles == 0) {
        k_write_g<<<1, 64, 0, st>>>(a.amax_bits, mode == MODE_FP46 ? 1792.0f : 2688.0f,
                                    (layouts & LAY_ROW) ? g0 : nullptr,
                                    (layouts & LAY_COL) ? g1 : nullptr);
        return hipGetLastError();
    }
    quant_mode<false>(a, mode, rht, layouts, st);
    return hipGetLastError();
}

// MXFP4 quantization, one pass (the E8M0 scales need no tensor-wide maximum).
extern "C" hipError_t nvfp4k_quant_mx(int sr, int rht, int layouts, const void *x, int64_t R,
                                      int64_t C, uint8_t *codes0, uint8_t *scales0, int tiled0,
                                      uint8_t *codes1, uint8_t *scales1, int tiled1,
                                      uint64_t seed, uint64_t rht_seed, hipStream_t st)
{
    using namespace nvfp4k;
    QuantArgs a = make_args(x, R, C, nullptr, seed, rht_seed);
    a.out[0] = {codes0, scales0, nullptr, tiled0};
    a.out[1] = {codes1, scales1, nullptr, tiled1};
    if (a.tiles == 0) return hipSuccess;
    if (sr) rht ? quant_lay<MODE_MX_SR, true, false>(a, layouts, st)
                : quant_lay<MODE_MX_SR, false, false>(a, layouts, st);
    else rht ? quant_lay<MODE_MX_RTN, true, false>(a, layouts, st)
             : quant_lay<MODE_MX_RTN, false, false>(a, layouts, st);
    return hipGetLastError();
}

// Bytes of workspace the one-call quantizers need: two maxima per phase-1 workgroup.
extern "C" size_t nvfp4k_workspace(void) { return 8 * (size_t)nvfp4k::MAX_PARTS; }

// ------------------------------------------------------------------------------ scratch
// Workspace in device memory the library owns, for callers that cannot allocate: the phase-1
// maxima of one call of eden_quantize_noalloc.  Every GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: its address on a device comes from hipGetSymbolAddress with that device
// current, looked up once per device and kept.  Every call on one GPU shares its copy, so
// calls that overlap on one GPU race.  No slot needs clearing: each call's phase 2 reads only
// slots its own phase 1 wrote.
namespace nvfp4k {
constexpr size_t SCRATCH_BYTES = 16384;
static_assert(8 * MAX_PARTS <= SCRATCH_BYTES, "the scratch must hold every phase-1 maximum");
}  // namespace nvfp4k

static __device__ __align__(256) uint8_t scratch[nvfp4k::SCRATCH_BYTES];

// The current device's copy of the scratch array and its size.
extern "C" hipError_t nvfp4k_scratch(void **ptr, size_t *bytes)
{
    using namespace nvfp4k;
    static std::mutex lock;
    static void *addr[MAX_DEVICES] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(lock);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = SCRATCH_BYTES;
    return hipSuccess;
}

// One-call quantization with one tensor scale per layout: phase 1 leaves each workgroup's
// maxima in the workspace (no clearing needed: every slot read is written), and each
// phase-2 workgroup reduces them before it rounds any scale.
extern "C" hipError_t nvfp4k_quantize(int mode, int rht, int layouts, const void *x, int64_t R,
                                      int64_t C, uint8_t *codes0, uint8_t *scales0, float *g0,
                                      uint8_t *codes1, uint8_t *scales1, float *g1,
                                      void *workspace, uint64_t seed, uint64_t rht_seed,
                                      hipStream_t st)
{
    using namespace nvfp4k;
    if (mode < MODE_RTN || mode > MODE_FP46) return hipErrorInvalidValue;
    uint32_t *parts = static_cast<uint32_t *>(workspace);
    if (R * C == 0) {
        // nothing to reduce: amax = 0, so g = 0 for each requested layout
        k_zero_u32<<<1, 64, 0, st>>>(parts, 2);
        k_write_g<<<1, 64, 0, st>>>(parts, 1.0f, (layouts & LAY_ROW) ? g0 : nullptr,
                                    (layouts & LAY_COL) ? g1 : nullptr);
        return hipGetLastError();
    }
    QuantArgs a = make_args(x, R, C, parts, seed, rht_seed);
    a.out[0] = {codes0, scales0, g0};
    a.out[1] = {codes1, scales1, g1};
    a.nparts = 1;                                   // phase 1: store per-workgroup maxima
    a.nparts = rht ? amax_lay<true, false>(a, layouts, st) : amax_lay<false, false>(a, layouts, st);
    quant_mode<false>(a, mode, rht, layouts, st);
    return hipGetLastError();
}

// Workspace of the strip-local quantizer: a 2 KiB scale table per row strip and per column
// strip, then 32 bytes of wave maxima per tile.
extern "C" size_t nvfp4k_strip_workspace(int64_t R, int64_t C)
{
    const int64_t tr = (R + nvfp4k::TILE - 1) / nvfp4k::TILE;
    const int64_t tc = (C + nvfp4k::TILE - 1) / nvfp4k::TILE;
    return 2048 * (size_t)(tr + tc) + 32 * (size_t)(tr * tc);
}

// Strip-local quantization: wave maxima per tile, strip tables, then the quantize pass.
extern "C" hipError_t nvfp4k_quant_strips(int mode, int rht, int layouts, const void *x,
                                          int64_t R, int64_t C, uint8_t *codes0,
                                          uint8_t *scales0, float *g0, uint8_t *codes1,
                                          uint8_t *scales1, float *g1, void *workspace,
                                          uint64_t seed, uint64_t rht_seed, hipStream_t st)
{
    using namespace nvfp4k;
    if (mode < MODE_RTN || mode > MODE_FP46) return hipErrorInvalidValue;
    QuantArgs a = make_args(x, R, C, nullptr, seed, rht_seed);
    a.out[0] = {codes0, scales0, g0};
    a.out[1] = {codes1, scales1, g1};
    a.tables = static_cast<float4 *>(workspace);
    a.amax_bits = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) +
                                               2048 * (a.tiles_r + a.tiles_c));
    if (a.tiles > 0) rht ? amax_lay<true, true>(a, layouts, st) : amax_lay<false, true>(a, layouts, st);
    // strips with no elements (rows or cols == 0) reduce nothing and get g = 0
    if (a.tiles_r + a.tiles_c > 0)
        k_strip_tables<<<(unsigned)(a.tiles_r + a.tiles_c), 256, 0, st>>>(
            a, layouts, mode == MODE_FP46 ? 1792.0f : 2688.0f);
    if (a.tiles > 0) quant_mode<true>(a, mode, rht, layouts, st);
    return hipGetLastError();
}

// The rotation's sign words, Philox4x32-10 of key rht_seed at counter (0, 0, STREAM_SIGN, 0)
// -- the words make_signs draws on the device -- computed on the host.
static nvfp4k::Signs host_signs(uint64_t key)
{
    uint32_t c0 = 0u, c1 = 0u, c2 = nvfp4k::STREAM_SIGN, c3 = 0u;
    uint32_t k0 = (uint32_t)key, k1 = (uint32_t)(key >> 32);
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return nvfp4k::Signs{{c0, c1, c2, c3}};
}

extern "C" hipError_t nvfp4k_dequantize(int local, const uint8_t *codes, const uint8_t *scales,
                                        const float *g, int64_t vecs, int64_t n, int rht,
                                        uint64_t rht_seed, float *out, hipStream_t st)
{
    using namespace nvfp4k;
    const int64_t groups = vecs * ((n + TILE - 1) / TILE);
    if (groups == 0) return hipSuccess;
    const int64_t blocks = (groups + 15) / 16;        // 16 groups of 16 lanes per block
    const int shift = local ? 7 : 62;      // vector -> index of its g (all vectors < 2^31)
    if (rht)
        k_dequant<true><<<(unsigned)blocks, 256, 0, st>>>(codes, scales, g, shift, vecs, n,
                                                          host_signs(rht_seed), out);
    else
        k_dequant<false><<<(unsigned)blocks, 256, 0, st>>>(codes, scales, g, shift, vecs, n,
                                                           Signs{{0u, 0u, 0u, 0u}}, out);
    return hipGetLastError();
}
