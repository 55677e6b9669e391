// conv_check.hip -- test helper: runs the quantizers' own scalar device functions
// (unbiased_nvfp4_gradient_amd/csrc/nvfp4_device.h) over ranges of inputs on the GPU so that
// the tests can compare every result with the CPU oracle.  Built into libconv_check.so next
// to this file; only tests load it.
//
// Every launcher takes device pointers sized by the caller for `count` results and checks
// nothing else: the tests size the buffers.  All grids are bounds-checked grid-stride loops.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.h"

using namespace nvfp4k;

namespace {

constexpr int THREADS = 256;

unsigned grid_for(uint64_t n)
{
    const uint64_t b = (n + THREADS - 1) / THREADS;
    return (unsigned)(b < 8192 ? (b ? b : 1) : 8192);
}

// E2M1 codes of the floats with bits start + i, i < count (count even), two per byte (low
// nibble = even i), by the packed conversion the RTN path uses, cycling through the four
// byte positions of the destination word as the quantizer does.  *touched counts the
// conversions that changed any of the other three bytes of their word.
__global__ void k_fp4_encode(uint32_t start, uint64_t count, uint8_t *out, uint32_t *touched)
{
    const uint64_t pairs = count / 2;
    uint32_t bad = 0;
    for (uint64_t p = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; p < pairs;
         p += (uint64_t)gridDim.x * blockDim.x) {
        const float y0 = __uint_as_float(start + (uint32_t)(2 * p));
        const float y1 = __uint_as_float(start + (uint32_t)(2 * p + 1));
        uint32_t w = 0x5A5A5A5Au;             // bytes the conversion must leave alone
        uint32_t byte;
        switch (p & 3) {
        case 0: w = CVT_FP4(w, y0, y1, 0); byte = w & 0xFFu; break;
        case 1: w = CVT_FP4(w, y0, y1, 1); byte = (w >> 8) & 0xFFu; break;
        case 2: w = CVT_FP4(w, y0, y1, 2); byte = (w >> 16) & 0xFFu; break;
        default: w = CVT_FP4(w, y0, y1, 3); byte = w >> 24; break;
        }
        const uint32_t keep = ~(0xFFu << (8 * (p & 3)));
        bad += (w & keep) != (0x5A5A5A5Au & keep);
        out[p] = (uint8_t)byte;
    }
    if (bad) atomicAdd(touched, bad);
}

// E4M3 nearest-even (saturating) of the floats with bits start + i.
__global__ void k_e4m3_rne(uint32_t start, uint64_t count, uint8_t *out)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (uint64_t)gridDim.x * blockDim.x)
        out[i] = (uint8_t)e4m3_rne_hw(__uint_as_float(start + (uint32_t)i));
}

// E4M3 round-up (capped) of the floats with bits start + i.
__global__ void k_e4m3_up(uint32_t start, uint64_t count, uint8_t *out)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (uint64_t)gridDim.x * blockDim.x)
        out[i] = (uint8_t)e4m3_up(__uint_as_float(start + (uint32_t)i));
}

// Grid values of every code byte at every byte position: out[(sel * 256 + byte) * 2 + k].
__global__ void k_fp4_decode(float *out)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= 1024) return;
    const int sel = t >> 8;
    const uint32_t byte = (uint32_t)(t & 255);
    const uint32_t w = (byte << (8 * sel)) | (0xA5A5A5A5u & ~(0xFFu << (8 * sel)));
    float2v v;
    switch (sel) {
    case 0: v = DEC_FP4(w, 0); break;
    case 1: v = DEC_FP4(w, 1); break;
    case 2: v = DEC_FP4(w, 2); break;
    default: v = DEC_FP4(w, 3); break;
    }
    out[2 * t] = v.x;
    out[2 * t + 1] = v.y;
}

// E4M3 values of the 128 codes.
__global__ void k_e4m3_val(float *out)
{
    if (threadIdx.x < 128) out[threadIdx.x] = e4m3_val(threadIdx.x);
}

// Scale SR of normal c in [2^-6, 448) with word w.
__global__ void k_scale_sr(const float *c, const uint32_t *w, uint64_t n, uint8_t *out)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        out[i] = (uint8_t)e4m3_sr_normal(__float_as_uint(c[i]), w[i]);
}

// Element SR code (sign and magnitude) of y[i] with word w[i], eight at a time through the
// quantizers' packing routine (so both element positions of the conversion are exercised);
// out[i] is one code per byte.  n is a multiple of 8.
__global__ void k_elem_sr(const float *y, const uint32_t *w, uint64_t n, uint8_t *out)
{
    for (uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n / 8;
         g += (uint64_t)gridDim.x * blockDim.x) {
        float yy[8];
        uint32_t ww[8];
        for (int k = 0; k < 8; ++k) { yy[k] = y[8 * g + k]; ww[k] = w[8 * g + k]; }
        const uint32_t d = e2m1_sr_pack8(yy, ww);
        for (int k = 0; k < 8; ++k) out[8 * g + k] = (uint8_t)((d >> (4 * k)) & 15u);
    }
}

// MXFP4 scale byte (e + 127) of the floats with bits start + i.
__global__ void k_mx_exp(uint32_t start, uint64_t count, uint8_t *out)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (uint64_t)gridDim.x * blockDim.x)
        out[i] = (uint8_t)(mx_scale_exp(__uint_as_float(start + (uint32_t)i)) + 127);
}

// Philox4x32-10 words of (key, counter) pairs: ctr [n][4], out [n][4].
__global__ void k_philox(const uint64_t *key, const uint32_t *ctr, uint64_t n, uint32_t *out)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x) {
        const Word4 r = philox(key[i], ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]);
        for (int k = 0; k < 4; ++k) out[4 * i + k] = r.w[k];
    }
}

int status(void) { return hipGetLastError() == hipSuccess ? 0 : -6; }

}  // namespace

extern "C" {

int conv_fp4_encode(uint32_t start, uint64_t count, uint8_t *out, uint32_t *touched,
                    void *stream)
{
    k_fp4_encode<<<grid_for(count / 2), THREADS, 0, (hipStream_t)stream>>>(start, count, out,
                                                                           touched);
    return status();
}

int conv_e4m3_rne(uint32_t start, uint64_t count, uint8_t *out, void *stream)
{
    k_e4m3_rne<<<grid_for(count), THREADS, 0, (hipStream_t)stream>>>(start, count, out);
    return status();
}

int conv_e4m3_up(uint32_t start, uint64_t count, uint8_t *out, void *stream)
{
    k_e4m3_up<<<grid_for(count), THREADS, 0, (hipStream_t)stream>>>(start, count, out);
    return status();
}

int conv_fp4_decode(float *out, void *stream)
{
    k_fp4_decode<<<4, 256, 0, (hipStream_t)stream>>>(out);
    return status();
}

int conv_e4m3_val(float *out, void *stream)
{
    k_e4m3_val<<<1, 128, 0, (hipStream_t)stream>>>(out);
    return status();
}

int conv_scale_sr(const float *c, const uint32_t *w, uint64_t n, uint8_t *out, void *stream)
{
    k_scale_sr<<<grid_for(n), THREADS, 0, (hipStream_t)stream>>>(c, w, n, out);
    return status();
}

int conv_elem_sr(const float *y, const uint32_t *w, uint64_t n, uint8_t *out, void *stream)
{
    if (n % 8) return -1;
    k_elem_sr<<<grid_for(n / 8), THREADS, 0, (hipStream_t)stream>>>(y, w, n, out);
    return status();
}

int conv_mx_exp(uint32_t start, uint64_t count, uint8_t *out, void *stream)
{
    k_mx_exp<<<grid_for(count), THREADS, 0, (hipStream_t)stream>>>(start, count, out);
    return status();
}

int conv_philox(const uint64_t *key, const uint32_t *ctr, uint64_t n, uint32_t *out,
                void *stream)
{
    k_philox<<<grid_for(n), THREADS, 0, (hipStream_t)stream>>>(key, ctr, n, out);
    return status();
}

}  // extern "C"
