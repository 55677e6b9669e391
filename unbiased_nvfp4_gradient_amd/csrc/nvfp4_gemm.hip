// nvfp4_gemm.hip -- the GEMM check consumer: C = A * B^T of two NVFP4 operands on gfx950
// matrix cores.
//
// Quartet II runs every linear layer's products on NVFP4 operands (itsolotime.com summary,
// abstract: NVFP4 GEMM kernels up to 4.2x over BF16 on Blackwell).  gfx950's scaled MFMA
// takes power-of-two (E8M0) scales per 32 elements, not E4M3 scales per 16, so this consumer
// dequantizes in LDS instead: a code's value V (<= 2 significant bits) times its block's
// E4M3 scale (<= 4 significant bits) has at most 6 significant bits and an exponent inside
// BF16's range, so the BF16 operand is exact.  v_mfma_f32_32x32x16_bf16 multiplies exactly
// and accumulates in FP32; the two FP32 tensor scales (and 2^-7 when both operands carry
// the same random-sign Hadamard rotation along K, since H H = 128 I) are applied in the
// epilogue.
//
// Tiling: a C tile of 256 x 256 per workgroup of 8 waves, each wave a 64 x 128 sub-tile
// (2 x 4 MFMA 32x32 tiles, 128 FP32 accumulators per lane); K in steps of 64 (four 1x16
// blocks).  Lane layouts of v_mfma_f32_32x32x16_bf16 (checked on
// the device): lane l supplies A row l%32 and B column l%32, elements k = 8*(l/32) .. +7;
// accumulator r of lane l is C[8*(r/4) + 4*(l/32) + r%4][l%32].
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4g {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float float2v __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDS_ROW = BK + 8;          // bf16 per LDS row (16-byte pad against bank conflicts)

struct Operand {
    const uint8_t *codes;    // [rows][K/2]
    const uint8_t *scales;   // [rows][K/16]
    const float *g;
};

__device__ __forceinline__ float e4m3_val(uint32_t c)
{
    const uint32_t e = c >> 3, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Two dequantized values -> one packed BF16 pair.  The products are exact and have at most
// 6 significant bits, so taking the high half of each FP32 is an exact conversion.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return (__float_as_uint(hi) & 0xFFFF0000u) | (__float_as_uint(lo) >> 16);
}

template <int SEL>
__device__ __forceinline__ uint32_t dq_pair(uint32_t w, float s)
{
    const float2v v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
    return pack_bf16(v.x * s, v.y * s);
}

// Dequantize 32 consecutive elements of one operand row (16 code bytes + 2 scales) into
// 16 packed BF16 pairs.
__device__ __forceinline__ void dequant32(uint4 cw, uint32_t s0, uint32_t s1, uint32_t out[16])
{
    const float f0 = e4m3_val(s0), f1 = e4m3_val(s1);
    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float f = k < 2 ? f0 : f1;
        out[4 * k + 0] = dq_pair<0>(w[k], f);
        out[4 * k + 1] = dq_pair<1>(w[k], f);
        out[4 * k + 2] = dq_pair<2>(w[k], f);
        out[4 * k + 3] = dq_pair<3>(w[k], f);
    }
}

// Stage one operand's 256 x 64 K-slice into LDS as BF16.  Thread t handles row t/2, elements
// 32*(t%2) .. +31 of the slice; rows outside [0, rows) are zero.
__device__ __forceinline__ void stage_operand(const Operand &op, int64_t rows, int64_t K,
                                              int64_t row0, int64_t k0, uint16_t *lds)
{
    const int t = threadIdx.x, r = t >> 1, half = t & 1;
    uint32_t packed[16];
    const int64_t row = row0 + r;
    if (row < rows) {
        const uint4 cw = *reinterpret_cast<const uint4 *>(op.codes + row * (K >> 1) +
                                                          (k0 >> 1) + 16 * half);
        const uint8_t *sp = op.scales + row * (K >> 4) + (k0 >> 4) + 2 * half;
        dequant32(cw, sp[0], sp[1], packed);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) packed[i] = 0u;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(lds + r * LDS_ROW + 32 * half);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        dst[i] = make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
}

__device__ __forceinline__ bf16x8 frag(const uint16_t *lds, int row, int k)
{
    const uint4 v = *reinterpret_cast<const uint4 *>(lds + row * LDS_ROW + k);
    return __builtin_bit_cast(bf16x8, v);
}

// C[M][N] = f * gA * gB * sum_k A[m][k] * B[n][k].  Grid: (ceil(N/256), ceil(M/256)),
// 512 threads.  M and N multiples of 32, K a multiple of 64.
__global__ void __launch_bounds__(512, 1) k_gemm(Operand A, Operand B, int64_t M, int64_t N,
                                                 int64_t K, float f, float *__restrict__ C)
{
    __shared__ uint16_t As[BM * LDS_ROW];
    __shared__ uint16_t Bs[BN * LDS_ROW];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int wm = (w >> 1) * 64, wn = (w & 1) * 128;      // this wave's 64 x 128 sub-tile
    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        __syncthreads();                                   // previous slice fully consumed
        stage_operand(A, M, K, m0, k0, As);
        stage_operand(B, N, K, n0, k0, Bs);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            const int kl = kk + 8 * (lane >> 5);
            bf16x8 a[2], b[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = frag(As, wm + 32 * i + (lane & 31), kl);
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = frag(Bs, wn + 32 * j + (lane & 31), kl);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j],
                                                                        0, 0, 0);
        }
    }

    const float scale = (*A.g * *B.g) * f;
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

extern "C" hipError_t nvfp4k_gemm(const uint8_t *a_codes, const uint8_t *a_scales,
                                  const float *a_g, const uint8_t *b_codes,
                                  const uint8_t *b_scales, const float *b_g, int64_t M,
                                  int64_t N, int64_t K, int rotated_pair, float *c,
                                  hipStream_t st)
{
    using namespace nvfp4g;
    if (M == 0 || N == 0) return hipSuccess;
    const Operand A{a_codes, a_scales, a_g}, B{b_codes, b_scales, b_g};
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    k_gemm<<<grid, 512, 0, st>>>(A, B, M, N, K, rotated_pair ? 0.0078125f : 1.0f, c);
    return hipGetLastError();
}
