// VALU issue rate of the instruction kinds the quantizer kernels use, on gfx950.
//
// Each kernel runs a loop whose body is 16 copies of one instruction over 8 independent
// registers (a chain of 2 per register per body), with 8 waves per SIMD on every CU and no
// memory access inside the loop, so the SIMD's issue rate for that instruction is the only
// limit.  Printed per kind: time, wave-lane instructions per second, and SIMD clocks per
// wave instruction at the nominal 2.4 GHz.  The quantizer's roofline takes its peak from
// the published FP32 vector rate (157.3 TFLOP/s = 78.6 T FMA lanes/s: 32 lanes per SIMD per
// clock); this program shows which instructions issue at that width and which at half or a
// quarter of it.
//
// Built by the package's build step as an executable; it takes no arguments.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

constexpr int ITERS = 2048;
constexpr int BLOCKS = 256 * 8;      // 2048 workgroups of 4 waves: 8 waves per SIMD
constexpr int THREADS = 256;

#define STR(x) #x
#define BODY(I) I(0) I(1) I(2) I(3) I(4) I(5) I(6) I(7) I(0) I(1) I(2) I(3) I(4) I(5) I(6) I(7)
#define RATE_KERNEL(NAME, INSTR)                                                             \
    __global__ void __launch_bounds__(THREADS) NAME(const uint32_t *in, uint32_t *out)      \
    {                                                                                        \
        const int t = blockIdx.x * blockDim.x + threadIdx.x;                                 \
        uint32_t a0 = in[(8 * t + 0) & 1023], a1 = in[(8 * t + 1) & 1023];                   \
        uint32_t a2 = in[(8 * t + 2) & 1023], a3 = in[(8 * t + 3) & 1023];                   \
        uint32_t a4 = in[(8 * t + 4) & 1023], a5 = in[(8 * t + 5) & 1023];                   \
        uint32_t a6 = in[(8 * t + 6) & 1023], a7 = in[(8 * t + 7) & 1023];                   \
        const uint32_t b = in[(t + 11) & 1023], c = in[(t + 17) & 1023];                     \
        for (int i = 0; i < ITERS; ++i) {                                                    \
            __asm__ volatile("s_nop 1\n\t" BODY(INSTR)                                       \
                             : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5),   \
                               "+v"(a6), "+v"(a7)                                            \
                             : "v"(b), "v"(c));                                              \
        }                                                                                    \
        out[t] = a0 ^ a1 ^ a2 ^ a3 ^ a4 ^ a5 ^ a6 ^ a7;                                      \
    }

#define I_ADD(k)     "v_add_f32_e32 %" STR(k) ", %" STR(k) ", %8\n\t"
#define I_SUB(k)     "v_sub_f32_e32 %" STR(k) ", %" STR(k) ", %8\n\t"
#define I_ADDABS(k)  "v_add_f32_e64 %" STR(k) ", |%" STR(k) "|, -%8\n\t"
#define I_MUL(k)     "v_mul_f32_e32 %" STR(k) ", %" STR(k) ", %8\n\t"
#define I_FMA(k)     "v_fma_f32 %" STR(k) ", %" STR(k) ", %8, %9\n\t"
#define I_FMAC(k)    "v_fmac_f32_e32 %" STR(k) ", %8, %9\n\t"
#define I_XOR(k)     "v_xor_b32_e32 %" STR(k) ", %8, %" STR(k) "\n\t"
#define I_ADDU(k)    "v_add_u32_e32 %" STR(k) ", %8, %" STR(k) "\n\t"
#define I_BITOP3(k)  "v_bitop3_b32 %" STR(k) ", %8, %9, %" STR(k) " bitop3:0x6c\n\t"
#define I_MAX(k)     "v_max_f32_e32 %" STR(k) ", %" STR(k) ", %8\n\t"
#define I_MAX3(k)    "v_max3_f32 %" STR(k) ", |%" STR(k) "|, |%8|, |%9|\n\t"
#define I_LSHLREV(k) "v_lshlrev_b32_e32 %" STR(k) ", 16, %" STR(k) "\n\t"
#define I_LSHLADD(k) "v_lshl_add_u32 %" STR(k) ", %8, 16, %" STR(k) "\n\t"
#define I_PERM(k)    "v_perm_b32 %" STR(k) ", %8, %" STR(k) ", %9\n\t"
#define I_FMACDPP(k) "v_fmac_f32_dpp %" STR(k) ", %8, %9 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
#define I_ADDDPP(k)  "v_add_f32_dpp %" STR(k) ", %8, %" STR(k) " quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
#define I_MULHI(k)   "v_mul_hi_u32 %" STR(k) ", %" STR(k) ", %8\n\t"
#define I_MULLO(k)   "v_mul_lo_u32 %" STR(k) ", %" STR(k) ", %8\n\t"
#define I_CVTFP4(k)  "v_cvt_scalef32_pk_fp4_f32 %" STR(k) ", %8, %9, %8\n\t"
#define I_CVTFP8(k)  "v_cvt_pk_fp8_f32 %" STR(k) ", %8, %9\n\t"
#define I_RCP(k)     "v_rcp_f32_e32 %" STR(k) ", %" STR(k) "\n\t"
#define I_XORSDWA(k) "v_xor_b32_sdwa %" STR(k) ", %" STR(k) ", %8 dst_sel:WORD_1 dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:WORD_1\n\t"
#define I_PKMAD(k)   "v_pk_mad_u16 %" STR(k) ", %" STR(k) ", %8, %9 op_sel:[0,0,0] op_sel_hi:[0,1,1]\n\t"
#define I_PKADD(k)   "v_pk_add_u16 %" STR(k) ", %" STR(k) ", %8\n\t"
#define I_MADU24(k)  "v_mad_u32_u24 %" STR(k) ", %" STR(k) ", %8, %9\n\t"
#define I_MULU24(k)  "v_mul_u32_u24_e32 %" STR(k) ", %8, %" STR(k) "\n\t"
#define I_CVTBF16(k) "v_cvt_f32_bf16_e32 %" STR(k) ", %" STR(k) "\n\t"
#define I_ANDSDWA(k) "v_and_b32_sdwa %" STR(k) ", %" STR(k) ", %8 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:DWORD\n\t"

RATE_KERNEL(k_add, I_ADD)
RATE_KERNEL(k_sub, I_SUB)
RATE_KERNEL(k_addabs, I_ADDABS)
RATE_KERNEL(k_mul, I_MUL)
RATE_KERNEL(k_fma, I_FMA)
RATE_KERNEL(k_fmac, I_FMAC)
RATE_KERNEL(k_xor, I_XOR)
RATE_KERNEL(k_addu, I_ADDU)
RATE_KERNEL(k_bitop3, I_BITOP3)
RATE_KERNEL(k_max, I_MAX)
RATE_KERNEL(k_max3, I_MAX3)
RATE_KERNEL(k_lshlrev, I_LSHLREV)
RATE_KERNEL(k_lshladd, I_LSHLADD)
RATE_KERNEL(k_perm, I_PERM)
RATE_KERNEL(k_fmacdpp, I_FMACDPP)
RATE_KERNEL(k_adddpp, I_ADDDPP)
RATE_KERNEL(k_mulhi, I_MULHI)
RATE_KERNEL(k_mullo, I_MULLO)
RATE_KERNEL(k_cvtfp4, I_CVTFP4)
RATE_KERNEL(k_cvtfp8, I_CVTFP8)
RATE_KERNEL(k_rcp, I_RCP)
RATE_KERNEL(k_xorsdwa, I_XORSDWA)
RATE_KERNEL(k_andsdwa, I_ANDSDWA)
RATE_KERNEL(k_pkmad, I_PKMAD)
RATE_KERNEL(k_pkadd, I_PKADD)
RATE_KERNEL(k_madu24, I_MADU24)
RATE_KERNEL(k_mulu24, I_MULU24)
RATE_KERNEL(k_cvtbf16, I_CVTBF16)

typedef void (*Kernel)(const uint32_t *, uint32_t *);
struct Entry { const char *instr; Kernel k; };

const Entry ENTRIES[] = {
    {"v_add_f32_e32", k_add},
    {"v_sub_f32_e32", k_sub},
    {"v_add_f32_e64 |a|, -b", k_addabs},
    {"v_mul_f32_e32", k_mul},
    {"v_fma_f32", k_fma},
    {"v_fmac_f32_e32", k_fmac},
    {"v_xor_b32_e32", k_xor},
    {"v_add_u32_e32", k_addu},
    {"v_bitop3_b32", k_bitop3},
    {"v_max_f32_e32", k_max},
    {"v_max3_f32 |a|,|b|,|c|", k_max3},
    {"v_lshlrev_b32_e32", k_lshlrev},
    {"v_lshl_add_u32", k_lshladd},
    {"v_perm_b32", k_perm},
    {"v_fmac_f32_dpp quad_perm", k_fmacdpp},
    {"v_add_f32_dpp quad_perm", k_adddpp},
    {"v_mul_hi_u32", k_mulhi},
    {"v_mul_lo_u32", k_mullo},
    {"v_cvt_scalef32_pk_fp4_f32", k_cvtfp4},
    {"v_cvt_pk_fp8_f32", k_cvtfp8},
    {"v_rcp_f32_e32", k_rcp},
    {"v_xor_b32_sdwa dst_sel:WORD_1 src0_sel:WORD_0", k_xorsdwa},
    {"v_and_b32_sdwa src0_sel:WORD_1", k_andsdwa},
    {"v_pk_mad_u16 op_sel_hi:[0,1,1]", k_pkmad},
    {"v_pk_add_u16", k_pkadd},
    {"v_mad_u32_u24", k_madu24},
    {"v_mul_u32_u24_e32", k_mulu24},
    {"v_cvt_f32_bf16_e32", k_cvtbf16},
};

#define CHECK(x)                                                                             \
    do {                                                                                     \
        hipError_t e_ = (x);                                                                 \
        if (e_ != hipSuccess) {                                                              \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);      \
            return 1;                                                                        \
        }                                                                                    \
    } while (0)

}  // namespace

int main()
{
    uint32_t *in = nullptr, *out = nullptr;
    CHECK(hipMalloc(&in, 1024 * sizeof(uint32_t)));
    CHECK(hipMalloc(&out, size_t(BLOCKS) * THREADS * sizeof(uint32_t)));
    uint32_t host[1024];
    for (int i = 0; i < 1024; ++i) host[i] = 0x3F800000u ^ ((i * 2654435761u) & 0x007FFFFFu);
    CHECK(hipMemcpy(in, host, sizeof host, hipMemcpyHostToDevice));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    // wave instructions of one launch: 16 per body plus the s_nop, per wave and iteration
    const double wave_instr = double(BLOCKS) * (THREADS / 64) * ITERS * 16;
    std::printf("| instruction | ms (best of 3) | T lane-instr/s | SIMD clocks per wave instr at 2.4 GHz |\n");
    std::printf("|---|---|---|---|\n");
    for (const Entry &e : ENTRIES) {
        float best = 1e30f;
        for (int rep = 0; rep < 4; ++rep) {           // the first launch warms the clocks
            CHECK(hipEventRecord(e0));
            hipLaunchKernelGGL(e.k, dim3(BLOCKS), dim3(THREADS), 0, 0, in, out);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e1));
            CHECK(hipEventSynchronize(e1));
            float ms = 0.0f;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            if (rep > 0 && ms < best) best = ms;
        }
        const double rate = wave_instr * 64 / (best * 1e-3) / 1e12;
        const double clocks = best * 1e-3 * 2.4e9 * 1024 / wave_instr;   // 1024 SIMDs
        std::printf("| `%s` | %.3f | %.1f | %.2f |\n", e.instr, best, rate, clocks);
        std::fflush(stdout);
    }
    CHECK(hipFree(in));
    CHECK(hipFree(out));
    return 0;
}
