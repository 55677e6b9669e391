// nvfp4_gemm.hip -- the GEMM check consumer: C = A * B^T of two NVFP4 operands on gfx950
// matrix cores.
//
// Quartet II runs every linear layer's products on NVFP4 operands (itsolotime.com summary,
// abstract: NVFP4 GEMM kernels up to 4.2x over BF16 on Blackwell).  gfx950's scaled MFMA
// takes power-of-two (E8M0) scales per 32 elements, not E4M3 scales per 16, so this consumer
// dequantizes into LDS instead: a code's value V (<= 2 significant bits) times its block's
// E4M3 scale (<= 4 significant bits) has at most 6 significant bits and lies in
// [2^-10, 2688], so the FP16 operand is exact.  v_mfma_f32_32x32x16_f16 multiplies exactly
// and accumulates in FP32; the two FP32 tensor scales (and 2^-7 when both operands carry
// the same random-sign Hadamard rotation along K, since H H = 128 I) are applied in the
// epilogue.  With strip-local scales (the CTA-local variant of the rit.work note on
// "Format-Aware Fusion for Fast FP4 Pretraining": separate row and column corrections applied
// after the sum over K) an operand has one g per 128 rows, and the epilogue takes the g of
// the output row's strip of A and of the output column's strip of B.
//
// Tiling: a C tile of 256 x 256 per workgroup of 8 waves, each wave a 64 x 128 sub-tile
// (2 x 4 MFMA 32x32 tiles, 128 FP32 accumulators per lane); K in steps of 64 (four 1x16
// blocks) through two LDS stages.  Lane layout of the 32x32x16 MFMA (checked on the
// device): lane l supplies A row l%32 and B column l%32, elements k = 8*(l/32) .. +7;
// accumulator r of lane l is C[8*(r/4) + 4*(l/32) + r%4][l%32].
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4g {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
// VALU instructions the scheduler places after each MFMA in the K loop (on the 16384 x 8192
// x 8192 check, 2 was measured slower; 3 to 8 alike within noise).
constexpr int VALU_PER_MFMA = 4;
constexpr int LDS_ROW = BK + 8;          // halfs per LDS row (16-byte pad against bank conflicts)
constexpr int STAGE = (BM + BN) * LDS_ROW;   // halfs of one A + B stage

struct Operand {
    const uint8_t *codes;    // [rows][K/2]
    const uint8_t *scales;   // [rows][K/16]
    const float *g;          // g of row r: g[r >> g_shift]
    int g_shift;             // 7 (one g per 128 rows) or 62 (one g)
};

// One thread's share of a 256 x 64 operand slice: row t/2, elements 32*(t%2) .. +31,
// as stored (16 code bytes, 2 scale bytes).
struct Raw {
    uint4 codes;
    uint32_t scales;
};

__device__ __forceinline__ Raw load_raw(const Operand &op, int64_t rows, int64_t K, int64_t row0,
                                        int64_t k0)
{
    const int t = threadIdx.x, r = t >> 1, half = t & 1;
    // rows past the operand re-read its last row: they only feed entries of C that are not
    // stored, and the K loop keeps no branch
    const int64_t row = row0 + r < rows ? row0 + r : rows - 1;
    Raw raw;
    raw.codes = *reinterpret_cast<const uint4 *>(op.codes + row * (K >> 1) + (k0 >> 1) +
                                                 16 * half);
    raw.scales = *reinterpret_cast<const uint16_t *>(op.scales + row * (K >> 4) + (k0 >> 4) +
                                                     2 * half);
    return raw;
}

__device__ __forceinline__ float e4m3_val(uint32_t c)
{
    const uint32_t e = c >> 3, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Codes 2 SEL and 2 SEL + 1 of a 32-bit word times scale s as a packed FP16 pair.  The grid
// values decode exactly to FP16 (the conversion's scale operand applies only a power of two,
// so it stays 1 and the E4M3 scale is a separate multiply), and the product of a value
// (<= 2 significant bits) and an E4M3 scale (<= 4) has at most 6 significant bits, between
// 2^-10 and 2688: exact in FP16.
template <int SEL>
__device__ __forceinline__ uint32_t dq_pair(uint32_t w, half2v s)
{
    const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(
                                                    w, 1.0f, SEL)) * s;
    return __builtin_bit_cast(uint32_t, h);
}

// Dequantize one thread's 32 elements and write them to its row of an LDS operand tile.
__device__ __forceinline__ void store_dequant(const Raw &raw, _Float16 *lds)
{
    const int t = threadIdx.x, r = t >> 1, half = t & 1;
    const _Float16 f0 = (_Float16)e4m3_val(raw.scales & 0xFFu);
    const _Float16 f1 = (_Float16)e4m3_val(raw.scales >> 8);
    const half2v s0 = {f0, f0}, s1 = {f1, f1};
    const uint32_t w[4] = {raw.codes.x, raw.codes.y, raw.codes.z, raw.codes.w};
    uint32_t o[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const half2v s = k < 2 ? s0 : s1;
        o[4 * k + 0] = dq_pair<0>(w[k], s);
        o[4 * k + 1] = dq_pair<1>(w[k], s);
        o[4 * k + 2] = dq_pair<2>(w[k], s);
        o[4 * k + 3] = dq_pair<3>(w[k], s);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(lds + r * LDS_ROW + 32 * half);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
}

__device__ __forceinline__ half8 frag(const _Float16 *lds, int row, int k)
{
    return *reinterpret_cast<const half8 *>(lds + row * LDS_ROW + k);
}

struct Frame {
    Operand A, B;
    int64_t M, N, K, m0, n0, nk;
    int wm, wn, lane;
};

// Eight codes (word k of a thread's 32 elements) times its block scale, as 16 bytes of FP16.
__device__ __forceinline__ uint4 dq_word(uint32_t w, half2v s)
{
    return make_uint4(dq_pair<0>(w, s), dq_pair<1>(w, s), dq_pair<2>(w, s), dq_pair<3>(w, s));
}

// Scale byte SEL of a thread's two block scales as an FP16 pair.  gfx950's FP8 conversion
// decodes OCP E4M3 exactly.
template <int SEL>
__device__ __forceinline__ half2v scale_pair(uint32_t scales)
{
    const _Float16 v = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)scales, SEL);
    return half2v{v, v};
}

// One step of the K loop: the MFMAs of slice kt from stage rd, while slice kt + 1 (held in
// ra, rb as raw codes) is dequantized into stage wr and slice kt + 2 is loaded.  rd and wr are
// distinct LDS arrays, so the two streams of work are independent.  Each of the four 16-wide
// k sub-steps reads its fragments, dequantizes one of the four code words of ra and rb, and
// runs its 8 MFMAs; the scheduling hints alternate one MFMA with a few VALU instructions, so
// the dequantization issues while the matrix core is busy.  Loads past the last slice
// re-read the last slice, and the stage written on the last step is never read.
__device__ __forceinline__ void kstep(const Frame &fr, const _Float16 *__restrict__ rd,
                                      _Float16 *__restrict__ wr, Raw &ra, Raw &rb, int64_t kt,
                                      f32x16 (&acc)[2][4])
{
    __syncthreads();       // rd written; wr no longer read
    const Raw qa = ra, qb = rb;
    const int64_t kn = (kt + 2 < fr.nk ? kt + 2 : fr.nk - 1) * BK;
    ra = load_raw(fr.A, fr.M, fr.K, fr.m0, kn);
    rb = load_raw(fr.B, fr.N, fr.K, fr.n0, kn);
    const int t = threadIdx.x, r = t >> 1, half = t & 1;
    uint4 *dstA = reinterpret_cast<uint4 *>(wr + r * LDS_ROW + 32 * half);
    uint4 *dstB = reinterpret_cast<uint4 *>(wr + BM * LDS_ROW + r * LDS_ROW + 32 * half);
    const uint32_t wa[4] = {qa.codes.x, qa.codes.y, qa.codes.z, qa.codes.w};
    const uint32_t wb[4] = {qb.codes.x, qb.codes.y, qb.codes.z, qb.codes.w};
    const half2v sa[2] = {scale_pair<0>(qa.scales), scale_pair<1>(qa.scales)};
    const half2v sb[2] = {scale_pair<0>(qb.scales), scale_pair<1>(qb.scales)};
    const _Float16 *As = rd, *Bs = rd + BM * LDS_ROW;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int kl = 16 * q + 8 * (fr.lane >> 5);
        half8 a[2], b[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = frag(As, fr.wm + 32 * i + (fr.lane & 31), kl);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = frag(Bs, fr.wn + 32 * j + (fr.lane & 31), kl);
        dstA[q] = dq_word(wa[q], sa[q >> 1]);       // words 0, 1: first block; 2, 3: second
        dstB[q] = dq_word(wb[q], sb[q >> 1]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER_MFMA, 0);   // then VALU
        }
        __builtin_amdgcn_sched_barrier(0);                       // keep sub-steps apart
    }
}

// C[M][N] = f * gA * gB * sum_k A[m][k] * B[n][k].  Grid: (ceil(N/256), ceil(M/256)),
// 512 threads.  M and N multiples of 32, K a multiple of 64.
//
// The K loop is software-pipelined over two LDS stages (kstep): the waves run the MFMAs of
// slice k from one stage while dequantizing slice k + 1 into the other and loading slice
// k + 2; one barrier per slice.
__global__ void __launch_bounds__(512, 1) k_gemm(Operand A, Operand B, int64_t M, int64_t N,
                                                 int64_t K, float f, float *__restrict__ C)
{
    __shared__ _Float16 lds[2 * STAGE];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int wm = (w >> 1) * 64, wn = (w & 1) * 128;      // this wave's 64 x 128 sub-tile
    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    const Frame fr{A, B, M, N, K, m0, n0, K / BK, wm, wn, lane};
    if (fr.nk > 0) {
        Raw ra = load_raw(A, M, K, m0, 0), rb = load_raw(B, N, K, n0, 0);
        store_dequant(ra, lds);
        store_dequant(rb, lds + BM * LDS_ROW);
        const int64_t k1 = fr.nk > 1 ? BK : 0;
        ra = load_raw(A, M, K, m0, k1);
        rb = load_raw(B, N, K, n0, k1);
        for (int64_t kt = 0; kt < fr.nk; ++kt)
            kstep(fr, lds + (kt & 1) * STAGE, lds + ((kt + 1) & 1) * STAGE, ra, rb, kt, acc);
    }

    // a wave's 64 rows and 128 columns each lie inside one 128-row strip of their operand
    const int64_t mw = m0 + wm, nw = n0 + wn;
    const float ga = mw < M ? A.g[mw >> A.g_shift] : 0.0f;
    const float gb = nw < N ? B.g[nw >> B.g_shift] : 0.0f;
    const float scale = (ga * gb) * f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < M && n < N) C[m * N + n] = acc[i][j][r] * scale;
            }
        }
    }
}

}  // namespace nvfp4g

extern "C" hipError_t nvfp4k_gemm(int local, const uint8_t *a_codes, const uint8_t *a_scales,
                                  const float *a_g, const uint8_t *b_codes,
                                  const uint8_t *b_scales, const float *b_g, int64_t M,
                                  int64_t N, int64_t K, int rotated_pair, float *c,
                                  hipStream_t st)
{
    using namespace nvfp4g;
    if (M == 0 || N == 0) return hipSuccess;
    const int shift = local ? 7 : 62;
    const Operand A{a_codes, a_scales, a_g, shift}, B{b_codes, b_scales, b_g, shift};
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    k_gemm<<<grid, 512, 0, st>>>(A, B, M, N, K, rotated_pair ? 0.0078125f : 1.0f, c);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------ MXFP4 GEMM
// The native FP4 consumer: C = f * A * B^T of two MXFP4 operands (E2M1 codes, one E8M0 scale
// per 32 elements along K) on gfx950's scaled matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in FP4: the matrix core multiplies the
// codes' grid values exactly, applies each lane's power-of-two block scales, and accumulates
// in FP32.  f = 2^-7 when both operands carry the same random-sign Hadamard rotation along K.
//
// Lane layout of the instruction (32 x 32 x 64): lane l supplies row l%32 of A (column l%32 of
// B) and its elements k = 32*(l/32) .. +31, 16 bytes of packed codes (low nibble first, as
// the quantizers store them), and the E8M0 scale of exactly that 32-block; accumulator r of
// lane l is C[8*(r/4) + 4*(l/32) + r%4][l%32], as for the other 32 x 32 instructions.
//
// Tiling: a C tile of 256 x 256 per workgroup of 8 waves, each wave a 64 x 128 sub-tile (2 x 4
// instructions, 128 FP32 accumulators per lane); K in steps of 128 (two instructions deep).
// Each step's codes, 64 bytes per row of A and of B, go straight from memory into one of four
// LDS stages (global_load_lds_dwordx4, 16 bytes per lane), three steps ahead of the stage that
// feeds the matrix cores, together with the rows' 4 scale bytes per step; chunk c of row i sits
// in slot 4 i + (c ^ ((i >> 2) & 3)).  A 16-byte LDS read serves 16 lanes at a time from 64
// banks (256 bytes); its lanes read 16 consecutive rows at one chunk, whose slots then cover
// all 16 residues mod 16, i.e. 16 distinct bank groups (the bank-conflict counter reads 0).
// The only wait on memory is at the top of each step, for that step's own loads.  This
// kernel serves K-tiled operands (its fastest form: every load reads one contiguous piece)
// and row-major operands whose K is not a multiple of 512; row-major operands with K a
// multiple of 512 take k_gemm_mx2 below.
namespace nvfp4g {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int MX_BK = 128;                    // K elements per step
constexpr int MX_ROW = MX_BK / 2;             // code bytes per row and step
constexpr int MX_CODES = (BM + BN) * MX_ROW;  // code bytes of one A + B stage (32 KiB)
constexpr int MX_STAGE = MX_CODES + 4 * (BM + BN);   // + 4 scale bytes per row and step

// Row-major operands: codes [rows][K/2], scales [rows][K/32].  K-tiled operands (the layout
// the MXFP4 producer writes on request): codes [K/128][rows][64], scales [K/128][rows][4], so
// that one K step of 256 rows is 16 KiB of codes and 1 KiB of scales in one piece.
struct MxOperand {
    const uint8_t *codes;
    const uint8_t *scales;
};

#define MX_LDS(p) ((__attribute__((address_space(3))) void *)(p))

__device__ __forceinline__ int mx_slot(int i, int c) { return 4 * i + (c ^ ((i >> 2) & 3)); }

// Where one thread's loads of a stage come from and go to.  The codes of A's and B's 256 rows
// (from m0, n0) are 1024 slots of 16 bytes per operand: lane L of wave w fills slot
// 512 k + 64 w + L in round k, i.e. chunk c of row i with mx_slot(i, c) that slot.  Every
// row's 4 scale bytes come in one 4-byte load per lane (waves 0..3 A's rows 64 w + L,
// waves 4..7 B's).  Rows past an operand re-read its last row (they feed only entries of C
// that are not stored).  The sources are those of step 0; step kt adds kt times a step to
// them: 64 bytes of codes and 4 of scales in a row-major operand, a whole K step of the
// operand's rows (64 or 4 bytes per row) in a K-tiled one.  With K-tiled operands the 64 lanes
// of a code load read 16 consecutive rows' 64 bytes, 1 KiB in one piece, where a row-major
// operand spreads them over 16 rows of K/2 bytes each; that difference alone makes the loads
// markedly cheaper.  The destinations are offsets in a stage, the same for every lane of a
// wave (the load writes lane L's 16 bytes at offset + 16 L).
struct MxLoads {
    const uint8_t *src[4];       // [2 op + k]: codes
    const uint8_t *ssrc;         // scales
    int64_t cstep[2], sstep;     // bytes per K step: codes of A, of B; this thread's scales
    uint32_t dst[4], sdst;       // offsets in a stage (wave-uniform)
};

template <bool TILED>
__device__ __forceinline__ MxLoads mx_loads(const MxOperand &A, const MxOperand &B, int64_t M,
                                            int64_t N, int64_t K, int64_t m0, int64_t n0)
{
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    MxLoads l;
#pragma unroll
    for (int op = 0; op < 2; ++op) {
        const uint8_t *codes = op ? B.codes : A.codes;
        const int64_t rows = op ? N : M, row0 = op ? n0 : m0;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int s = 512 * k + 64 * w + lane;
            const int i = s >> 2, c = (s & 3) ^ ((i >> 2) & 3);
            const int64_t row = row0 + i < rows ? row0 + i : rows - 1;
            l.src[2 * op + k] = codes + row * (TILED ? MX_ROW : (K >> 1)) + 16 * c;
            l.dst[2 * op + k] = (uint32_t)(op * BM * MX_ROW + 16 * (512 * k + 64 * w));
        }
        l.cstep[op] = TILED ? rows * MX_ROW : MX_ROW;
    }
    const bool on_b = w >= 4;
    const int64_t rows = on_b ? N : M, row0 = on_b ? n0 : m0;
    const int i = 64 * (w & 3) + lane;
    const int64_t row = row0 + i < rows ? row0 + i : rows - 1;
    l.ssrc = (on_b ? B.scales : A.scales) + row * (TILED ? 4 : (K >> 5));
    l.sstep = TILED ? rows * 4 : 4;
    l.sdst = (uint32_t)(MX_CODES + 4 * (on_b ? BM : 0) + 4 * 64 * (w & 3));
    return l;
}

// Start loading step kt into a stage: five loads per lane, no branch.
__device__ __forceinline__ void mx_stage(const MxLoads &l, int64_t kt, uint8_t *stage)
{
#pragma unroll
    for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_global_load_lds(l.src[q] + kt * l.cstep[q >> 1],
                                         MX_LDS(stage + l.dst[q]), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(l.ssrc + kt * l.sstep, MX_LDS(stage + l.sdst), 4, 0, 0);
}

__device__ __forceinline__ v8i mx_frag(const uint8_t *p)
{
    const v4i v = *reinterpret_cast<const v4i *>(p);
    return v8i{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
}

// Stages in flight: while the matrix cores work on one stage, the loads of the next
// MX_NSTAGE - 1 are outstanding.  Each wave issues exactly MX_LOADS loads per stage (two
// 16-byte code loads per operand and one scale load), one stage per step, and the vector
// memory counter retires in issue order, so waiting until at most MX_LOADS loads are
// outstanding waits for every stage but the one issued last.
constexpr int MX_NSTAGE = 4;
constexpr int MX_LOADS = 5;

// Wait for this wave's loads of every stage but the newest, then for every wave: the stage
// after the current one is complete in LDS.  `all` waits for every load (the prologue).
__device__ __forceinline__ void mx_barrier(bool all)
{
    // s_waitcnt fields (gfx9): vmcnt bits 3:0 and 15:14, expcnt 6:4 (7 = no wait), lgkmcnt
    // 11:8 (0: this wave's LDS reads are done too)
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("" ::: "memory");
    if (all) __builtin_amdgcn_s_waitcnt(0x0070);
    else __builtin_amdgcn_s_waitcnt(0x0070 | MX_LOADS);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// A lane's offsets in a stage of its fragments (sub-step q: A rows wm + 32 i + lane % 32, B
// rows wn + 32 j + lane % 32, 16-byte chunk 2 q + lane / 32) and of its rows' scale words.
struct MxOffsets {
    uint32_t a[2][2], b[4][2];   // [tile][sub-step]
    uint32_t sa[2], sb[4];
};

__device__ __forceinline__ MxOffsets mx_offsets(int wm, int wn, int lane)
{
    const int half = lane >> 5, r = lane & 31;
    MxOffsets o;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int i = 0; i < 2; ++i) o.a[i][q] = 16 * mx_slot(wm + 32 * i + r, 2 * q + half);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o.b[j][q] = BM * MX_ROW + 16 * mx_slot(wn + 32 * j + r, 2 * q + half);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) o.sa[i] = MX_CODES + 4 * (wm + 32 * i + r);
#pragma unroll
    for (int j = 0; j < 4; ++j) o.sb[j] = MX_CODES + 4 * (BM + wn + 32 * j + r);
    return o;
}

// One sub-step's operands of a wave: 2 fragments of A, 4 of B (sub-step q of a stage).
struct MxFrags {
    v8i a[2], b[4];
};

__device__ __forceinline__ MxFrags mx_read(const uint8_t *stage, const MxOffsets &o, int q)
{
    MxFrags f;
#pragma unroll
    for (int i = 0; i < 2; ++i) f.a[i] = mx_frag(stage + o.a[i][q]);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[j] = mx_frag(stage + o.b[j][q]);
    return f;
}

// Each lane's scale words of a stage; shifted right by 8 (lane / 32), byte 2q is its
// 32-block's in sub-step q.
struct MxScales {
    uint32_t a[2], b[4];
};

__device__ __forceinline__ MxScales mx_read_scales(const uint8_t *stage, const MxOffsets &o)
{
    MxScales r;
#pragma unroll
    for (int i = 0; i < 2; ++i) r.a[i] = *reinterpret_cast<const uint32_t *>(stage + o.sa[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) r.b[j] = *reinterpret_cast<const uint32_t *>(stage + o.sb[j]);
    return r;
}

__device__ __forceinline__ MxScales mx_shift(const MxScales &s, int sh)
{
    MxScales r;
#pragma unroll
    for (int i = 0; i < 2; ++i) r.a[i] = s.a[i] >> sh;
#pragma unroll
    for (int j = 0; j < 4; ++j) r.b[j] = s.b[j] >> sh;
    return r;
}

template <int Q>
__device__ __forceinline__ void mx_mfma(f32x16 (&acc)[2][4], const MxFrags &f, const MxScales &s)
{
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                f.a[i], f.b[j], acc[i][j], 4, 4, 2 * Q, (int)s.a[i], 2 * Q, (int)s.b[j]);
}

// C[M][N] = f * sum_k A[m][k] * B[n][k].  Grid (ceil(N/256), ceil(M/256)), 512 threads.
// M and N multiples of 32, K a multiple of 128; TILED: both operands K-tiled.
//
// The fragment reads run one sub-step ahead of the matrix instructions: a step reads its
// second sub-step's fragments before its first sub-step's instructions issue, then (after the
// barrier that makes the next stage visible) the next step's first fragments and scales
// before its second sub-step's instructions; scheduling barriers keep each group of reads
// ahead of the instructions that run while they are in flight, and the next step's scale
// shifts after them.  Every read of a stage is complete before the barrier of the step after
// it, which is where the loads of a later stage may overwrite it.  The load addresses and the
// LDS offsets are computed once.
template <bool TILED>
__global__ void __launch_bounds__(512, 1) k_gemm_mx(MxOperand A, MxOperand B, int64_t M,
                                                    int64_t N, int64_t K, float f,
                                                    float *__restrict__ C)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[MX_NSTAGE * MX_STAGE];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int wm = (w >> 1) * 64, wn = (w & 1) * 128;
    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    const int64_t nk = K / MX_BK;
    const MxLoads ld = mx_loads<TILED>(A, B, M, N, K, m0, n0);
    const MxOffsets of = mx_offsets(wm, wn, lane);
    const int sh = 8 * (lane >> 5);
    // stage s goes to buffer s % MX_NSTAGE; past the last step the loads repeat the last
    // step's data into buffers nobody reads, so every step issues the same loads
    auto stage = [&](int64_t s) {
        mx_stage(ld, s < nk ? s : nk - 1, lds + (int)(s & (MX_NSTAGE - 1)) * MX_STAGE);
    };
    if (nk > 0) {
        stage(0);
        stage(1);
        stage(2);
        mx_barrier(true);
        MxFrags f0 = mx_read(lds, of, 0);
        MxScales sc = mx_shift(mx_read_scales(lds, of), sh);
        for (int64_t kt = 0; kt < nk; ++kt) {
            const uint8_t *cur = lds + (int)(kt & (MX_NSTAGE - 1)) * MX_STAGE;
            const MxFrags f1 = mx_read(cur, of, 1);
            __builtin_amdgcn_sched_barrier(0);
            mx_mfma<0>(acc, f0, sc);
            // stage kt + 1 landed (its loads were issued before the newest, kt + 2's); the
            // buffer of stage kt - 1 was last read before this barrier
            mx_barrier(false);
            stage(kt + MX_NSTAGE - 1);
            const uint8_t *nxt = lds + (int)((kt + 1) & (MX_NSTAGE - 1)) * MX_STAGE;
            f0 = mx_read(nxt, of, 0);
            const MxScales raw = mx_read_scales(nxt, of);
            __builtin_amdgcn_sched_barrier(0);
            mx_mfma<1>(acc, f1, sc);
            __builtin_amdgcn_sched_barrier(0);
            sc = mx_shift(raw, sh);
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < M && n < N) C[m * N + n] = acc[i][j][r] * f;
            }
        }
    }
}


// ------------------------------------------------------------------------------ MXFP4 GEMM, K % 512 == 0
// The same product on row-major operands with wider K steps, for K a multiple of 512.  Each
// step covers 256 elements of K: 128 code bytes per row of A and B (one 128-byte line per row,
// where the 128-element steps above fetch half a line per row per step), and each row's scale
// bytes come 16 at a time, once every two steps.  Measured with the loads alone, the narrow
// kernel's row-major loads move their bytes at about 0.8 of the rate of these: the number of
// rows a load instruction touches, not its byte count, sets its cost (K-tiled operands, whose
// loads each touch 8 whole lines, do better still).
//
// LDS: two code stages of 64 KiB (256 rows of A then 256 of B, 128 bytes each; chunk c of row
// i in 16-byte slot 8 i + (c ^ ((i >> 1) & 7)), so the 16 rows one 16-byte read serves at a
// time cover all 16 bank groups) and two scale stages of 8 KiB (16 bytes per row: the scale
// bytes of two steps).  A step runs its four sub-steps of 64 elements (8 instructions per
// wave each); the barrier sits before the last sub-step, so that sub-step's instructions
// overlap the wait, the next step's loads and its first reads.
constexpr int MX2_BK = 256;                      // K elements per step
constexpr int MX2_ROW = MX2_BK / 2;              // code bytes per row and step
constexpr int MX2_CODES = (BM + BN) * MX2_ROW;   // 64 KiB
constexpr int MX2_SCALES = (BM + BN) * 16;       // 8 KiB: two steps of scale bytes per row

__device__ __forceinline__ int mx2_slot(int i, int c) { return 8 * i + (c ^ ((i >> 1) & 7)); }

// One thread's loads.  Codes: 4 rounds per operand of 16-byte chunks, lane L of wave w filling
// slot 512 r + 64 w + L of the operand's half of the stage, i.e. row i = 64 r + i0 (i0 =
// 8 w + L / 8) at chunk c = (L & 7) ^ ((i0 >> 1) & 7), the same chunk in every round.  Rows past
// an operand re-read its last row (they feed only entries of C that are not stored); the row
// is clamped per load, so a thread keeps one pointer per operand.  Scales: one 16-byte load
// for row t (A's rows for t < 256, then B's).
struct Mx2Loads {
    const uint8_t *p[2];         // codes + (row0 + i0) ... : operand base at chunk c
    int i0, lim[2];              // first row index; last valid row index - row0 per operand
    const uint8_t *ssrc;         // this thread's scale row
};

__device__ __forceinline__ Mx2Loads mx2_loads(const MxOperand &A, const MxOperand &B, int64_t M,
                                              int64_t N, int64_t K, int64_t m0, int64_t n0)
{
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(t >> 6));
    Mx2Loads l;
    l.i0 = 8 * w + (lane >> 3);
    const int c = (lane & 7) ^ ((l.i0 >> 1) & 7);
    l.p[0] = A.codes + m0 * (K >> 1) + 16 * c;
    l.p[1] = B.codes + n0 * (K >> 1) + 16 * c;
    l.lim[0] = (int)((M - 1 - m0) < 255 ? (M - 1 - m0) : 255);
    l.lim[1] = (int)((N - 1 - n0) < 255 ? (N - 1 - n0) : 255);
    const int op = t >> 8, i = t & 255;
    const int64_t rows = op ? N : M, row0 = op ? n0 : m0;
    const int64_t row = row0 + i < rows ? row0 + i : rows - 1;
    l.ssrc = (op ? B.scales : A.scales) + row * (K >> 5);
    return l;
}

// A lane's fragment rows: A rows wm + 32 i + lane % 32, B rows wn + 32 j + lane % 32.  Chunk
// c = 2 q + lane / 32 of row r sits at byte 128 r + 16 (c ^ ((r >> 1) & 7)); rows 32 apart
// share the xor term, so fragment i of A is at a + 4096 i and the chunk of sub-step q at
// (a ^ 32 q) + 4096 i, with a = 128 r0 + 16 (lane / 32 ^ ((r0 >> 1) & 7)) for the lane's
// first row r0 (the chunk bits 5..6 lie below the row bits).  Likewise for B.  The scale
// words of the lane's rows are at sa + 512 i and sb + 512 j (16 bytes per row).
struct Mx2Offsets {
    uint32_t a, b, sa, sb;
};

__device__ __forceinline__ Mx2Offsets mx2_offsets(int wm, int wn, int lane)
{
    const int half = lane >> 5, r = lane & 31;
    Mx2Offsets o;
    o.a = (uint32_t)(16 * mx2_slot(wm + r, half));
    o.b = (uint32_t)(BM * MX2_ROW + 16 * mx2_slot(wn + r, half));
    o.sa = (uint32_t)(16 * (wm + r));
    o.sb = (uint32_t)(16 * (BM + wn + r));
    return o;
}

__device__ __forceinline__ MxFrags mx2_read(const uint8_t *stage, const Mx2Offsets &o, int q)
{
    const uint8_t *pa = stage + (o.a ^ (uint32_t)(32 * q));
    const uint8_t *pb = stage + (o.b ^ (uint32_t)(32 * q));
    MxFrags f;
#pragma unroll
    for (int i = 0; i < 2; ++i) f.a[i] = mx_frag(pa + 4096 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[j] = mx_frag(pb + 4096 * j);
    return f;
}

// A step's 8 scale bytes per row: word 0 covers sub-steps 0 and 1, word 1 sub-steps 2 and 3.
struct Mx2Scales {
    uint2 a[2], b[4];
};

__device__ __forceinline__ Mx2Scales mx2_read_scales(const uint8_t *sstage, const Mx2Offsets &o,
                                                     int odd)
{
    const uint8_t *pa = sstage + o.sa + 8 * odd, *pb = sstage + o.sb + 8 * odd;
    Mx2Scales s;
#pragma unroll
    for (int i = 0; i < 2; ++i) s.a[i] = *reinterpret_cast<const uint2 *>(pa + 512 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) s.b[j] = *reinterpret_cast<const uint2 *>(pb + 512 * j);
    return s;
}

// The scale words of sub-step q, shifted so that byte 2 (q & 1) is this lane's 32-block's.
__device__ __forceinline__ MxScales mx2_sub_scales(const Mx2Scales &s, int q, int sh)
{
    MxScales r;
#pragma unroll
    for (int i = 0; i < 2; ++i) r.a[i] = (q < 2 ? s.a[i].x : s.a[i].y) >> sh;
#pragma unroll
    for (int j = 0; j < 4; ++j) r.b[j] = (q < 2 ? s.b[j].x : s.b[j].y) >> sh;
    return r;
}

// Wait for all of this wave's loads and LDS reads, then for every wave.
__device__ __forceinline__ void mx2_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// A step's parity as a type, so that each of the two steps of the loop body is compiled with it.
template <int V> struct Mx2Parity { static constexpr int value = V; };

// Hide a value from loop-invariant code motion, so that an address is recomputed where it is
// used (a few instructions per load) instead of being kept in registers across the K loop.
__device__ __forceinline__ int mx2_opaque(int v)
{
    __asm__ volatile("" : "+v"(v));
    return v;
}

// C[M][N] = f * sum_k A[m][k] * B[n][k].  Grid (ceil(N/256), ceil(M/256)), 512 threads.
// M and N multiples of 32, K a multiple of 512.
//
// Step kt computes from code stage kt % 2 and scale stage (kt / 2) % 2.  Its barrier (before
// its last sub-step) finds stage kt + 1 loaded (issued after the previous barrier) and every
// read of stage kt done, so the loads of stage kt + 2 then go into stage kt's buffer; on even
// steps the scale bytes of steps kt + 2 and kt + 3 follow into the scale buffer whose steps
// are over.  The next step's scale words and first fragments are read right after the loads
// are issued, while this step's last instructions run.  The loop body is two steps (K is a
// multiple of 512, so the step count is even) and has no branch: loads past the last step
// re-read the last step's data into buffers nobody reads again, and the reads past it read
// a buffer whose contents go unused.
__global__ void __launch_bounds__(512, 1) k_gemm_mx2(MxOperand A, MxOperand B, int64_t M,
                                                     int64_t N, int64_t K, float f,
                                                     float *__restrict__ C)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * MX2_CODES + 2 * MX2_SCALES];
    uint8_t *const sbase = lds + 2 * MX2_CODES;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int wm = (w >> 1) * 64, wn = (w & 1) * 128;
    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    const int64_t nk = K / MX2_BK;
    const Mx2Loads ld = mx2_loads(A, B, M, N, K, m0, n0);
    const Mx2Offsets of = mx2_offsets(wm, wn, lane);
    const int sh = 8 * (lane >> 5);
    const int64_t Kh = K >> 1;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    // codes of step min(s, nk - 1) into code buffer s % 2
    auto load_codes = [&](int64_t s) {
        uint8_t *st = lds + (int)(s & 1) * MX2_CODES;
        const int64_t src = (s < nk ? s : nk - 1) * MX2_ROW;
        const int i0 = mx2_opaque(ld.i0);
#pragma unroll
        for (int op = 0; op < 2; ++op) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + 64 * r;
                const int row = i < ld.lim[op] ? i : ld.lim[op];
                __builtin_amdgcn_global_load_lds(
                    ld.p[op] + (int64_t)row * Kh + src,
                    MX_LDS(st + op * BM * MX2_ROW + 16 * (512 * r + 64 * wu)), 16, 0, 0);
            }
        }
    };
    // scale bytes of steps 2 ss and 2 ss + 1 (the last pair's past the end) into buffer ss % 2
    auto load_scales = [&](int64_t ss) {
        const int64_t src = 16 * (ss < nk / 2 ? ss : nk / 2 - 1);
        __builtin_amdgcn_global_load_lds(
            ld.ssrc + src, MX_LDS(sbase + (int)(ss & 1) * MX2_SCALES + 16 * 64 * wu), 16, 0, 0);
    };
    // one step; ODD is kt's parity
    auto step = [&](int64_t kt, auto odd_tag, MxFrags &f0, Mx2Scales &sc) {
        constexpr int ODD = decltype(odd_tag)::value;
        const uint8_t *cur = lds + ODD * MX2_CODES;
        const MxFrags f1 = mx2_read(cur, of, 1);
        __builtin_amdgcn_sched_barrier(0);
        mx_mfma<0>(acc, f0, mx2_sub_scales(sc, 0, sh));
        const MxFrags f2 = mx2_read(cur, of, 2);
        __builtin_amdgcn_sched_barrier(0);
        mx_mfma<1>(acc, f1, mx2_sub_scales(sc, 1, sh));
        const MxFrags f3 = mx2_read(cur, of, 3);
        __builtin_amdgcn_sched_barrier(0);
        mx_mfma<0>(acc, f2, mx2_sub_scales(sc, 2, sh));
        const MxScales s3 = mx2_sub_scales(sc, 3, sh);
        mx2_barrier();
        load_codes(kt + 2);
        if constexpr (!ODD) load_scales(kt / 2 + 1);
        f0 = mx2_read(lds + (1 - ODD) * MX2_CODES, of, 0);
        // step kt + 1's scales: the second word pair of this pair's buffer after an even step,
        // the first of the next pair's after an odd one
        sc = mx2_read_scales(sbase + (int)(((kt + 1) >> 1) & 1) * MX2_SCALES, of, 1 - ODD);
        __builtin_amdgcn_sched_barrier(0);
        mx_mfma<1>(acc, f3, s3);
    };
    if (nk > 0) {
        load_codes(0);
        load_codes(1);
        load_scales(0);
        mx2_barrier();
        MxFrags f0 = mx2_read(lds, of, 0);
        Mx2Scales sc = mx2_read_scales(sbase, of, 0);
        for (int64_t kt = 0; kt < nk; kt += 2) {
            step(kt, Mx2Parity<0>{}, f0, sc);
            step(kt + 1, Mx2Parity<1>{}, f0, sc);
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < M && n < N) C[m * N + n] = acc[i][j][r] * f;
            }
        }
    }
}

}  // namespace nvfp4g

extern "C" hipError_t nvfp4k_gemm_mx(const uint8_t *a_codes, const uint8_t *a_scales,
                                     const uint8_t *b_codes, const uint8_t *b_scales,
                                     int64_t M, int64_t N, int64_t K, int tiled,
                                     int rotated_pair, float *c, hipStream_t st)
{
    using namespace nvfp4g;
    if (M == 0 || N == 0) return hipSuccess;
    const MxOperand A{a_codes, a_scales}, B{b_codes, b_scales};
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    const float f = rotated_pair ? 0.0078125f : 1.0f;
    if (tiled) k_gemm_mx<true><<<grid, 512, 0, st>>>(A, B, M, N, K, f, c);
    else if (K % 512 == 0) k_gemm_mx2<<<grid, 512, 0, st>>>(A, B, M, N, K, f, c);
    else k_gemm_mx<false><<<grid, 512, 0, st>>>(A, B, M, N, K, f, c);
    return hipGetLastError();
}
