// nvfp4_api.cpp -- C ABI of libnvfp4.so: argument validation and dispatch to the gfx950
// kernels in nvfp4_kernels.hip.  The declarations, with the meaning, layout, ownership and
// error behaviour of every argument, are in include/nvfp4.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

extern "C" hipError_t nvfp4k_amax(int rht, int layouts, const void *x, int64_t R, int64_t C,
                                  float *amax, uint64_t rht_seed, hipStream_t st);
extern "C" hipError_t nvfp4k_quant(int mode, int rht, int layouts, const void *x, int64_t R,
                                   int64_t C, uint8_t *codes0, uint8_t *scales0, float *g0,
                                   uint8_t *codes1, uint8_t *scales1, float *g1,
                                   const float *amax, uint64_t seed, uint64_t rht_seed,
                                   hipStream_t st);
extern "C" size_t nvfp4k_workspace(void);
extern "C" hipError_t nvfp4k_scratch(void **ptr, size_t *bytes);
extern "C" hipError_t nvfp4k_quantize(int mode, int rht, int layouts, const void *x, int64_t R,
                                      int64_t C, uint8_t *codes0, uint8_t *scales0, float *g0,
                                      uint8_t *codes1, uint8_t *scales1, float *g1,
                                      void *workspace, uint64_t seed, uint64_t rht_seed,
                                      hipStream_t st);
extern "C" size_t nvfp4k_strip_workspace(int64_t R, int64_t C);
extern "C" hipError_t nvfp4k_quant_strips(int mode, int rht, int layouts, const void *x,
                                          int64_t R, int64_t C, uint8_t *codes0,
                                          uint8_t *scales0, float *g0, uint8_t *codes1,
                                          uint8_t *scales1, float *g1, void *workspace,
                                          uint64_t seed, uint64_t rht_seed, hipStream_t st);
extern "C" hipError_t nvfp4k_gemm(int local, const uint8_t *a_codes, const uint8_t *a_scales,
                                  const float *a_g, const uint8_t *b_codes,
                                  const uint8_t *b_scales, const float *b_g, int64_t M,
                                  int64_t N, int64_t K, int rotated_pair, float *c,
                                  hipStream_t st);
extern "C" hipError_t nvfp4k_quant_mx(int sr, int rht, int layouts, const void *x, int64_t R,
                                      int64_t C, uint8_t *codes0, uint8_t *scales0, int tiled0,
                                      uint8_t *codes1, uint8_t *scales1, int tiled1,
                                      uint64_t seed, uint64_t rht_seed, hipStream_t st);
extern "C" hipError_t nvfp4k_gemm_mx(const uint8_t *a_codes, const uint8_t *a_scales,
                                     const uint8_t *b_codes, const uint8_t *b_scales,
                                     int64_t M, int64_t N, int64_t K, int tiled,
                                     int rotated_pair, float *c, hipStream_t st);
extern "C" hipError_t nvfp4k_dequantize(int local, const uint8_t *codes, const uint8_t *scales,
                                        const float *g, int64_t vecs, int64_t n, int rht,
                                        uint64_t rht_seed, float *out, hipStream_t st);

namespace {

enum { MODE_RTN = 0, MODE_SR = 1, MODE_EDEN = 2, MODE_FP46 = 3 };

constexpr size_t MIN_WORKSPACE_BYTES = 256;   // smallest workspace any quantizer asks for
constexpr int64_t MAX_DIM = (int64_t)1 << 31; // each dimension is below this
constexpr int64_t MAX_ELEMS = (int64_t)1 << 40; // and so is each product of two

// a < MAX_DIM and b < MAX_DIM and a * b < MAX_ELEMS (a, b >= 0)
bool fits(int64_t a, int64_t b)
{
    return a < MAX_DIM && b < MAX_DIM && (a == 0 || b <= (MAX_ELEMS - 1) / a);
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_device()
{
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return NVFP4_ERR_HIP;
    }
    return NVFP4_OK;
}

// A layout with no elements may pass NULL codes and scales (its tensor scale is still set).
int check_layout(const nvfp4_tensor *t, bool empty)
{
    if (!t) return NVFP4_OK;
    if (!t->tensor_scale || (!empty && (!t->codes || !t->scales))) return NVFP4_ERR_NULL;
    if (!aligned(t->codes, 16) || !aligned(t->scales, 8) || !aligned(t->tensor_scale, 4))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// Checks shared by every quantizer entry point (everything but the workspace and amax).
int check_input(int mode, const void *x, int64_t rows, int64_t cols, int group, int block, int rht,
                bool want_row, bool want_col)
{
    if (!x && rows > 0 && cols > 0) return NVFP4_ERR_NULL;
    if (group != 128 || block != 16) return NVFP4_ERR_GROUP;
    if (rht != 0 && rht != 1) return NVFP4_ERR_ARG;
    if (mode < MODE_RTN || mode > MODE_FP46) return NVFP4_ERR_ARG;
    if (rows < 0 || cols < 0) return NVFP4_ERR_SHAPE;
    if (!fits(rows, cols)) return NVFP4_ERR_ARG;
    const bool rotated = rht || mode == MODE_EDEN;
    const int64_t unit = rotated ? 128 : 16;
    if (cols % 8) return NVFP4_ERR_SHAPE;
    if (want_row && cols % unit) return NVFP4_ERR_SHAPE;
    if (want_col && rows % unit) return NVFP4_ERR_SHAPE;
    if (!aligned(x, 16)) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

int check_outputs(const nvfp4_tensor *row_out, const nvfp4_tensor *col_out, int64_t rows,
                  int64_t cols)
{
    if (!row_out && !col_out) return NVFP4_ERR_NULL;
    const bool empty = rows == 0 || cols == 0;
    int rc = check_layout(row_out, empty);
    return rc ? rc : check_layout(col_out, empty);
}

int launch_quant(int mode, const void *x, int64_t rows, int64_t cols, uint64_t seed, int rht,
                 uint64_t rht_seed, const float *amax, const nvfp4_tensor *row_out,
                 const nvfp4_tensor *col_out, void *stream)
{
    const int layouts = (row_out ? 1 : 0) | (col_out ? 2 : 0);
    const bool rotated = rht || mode == MODE_EDEN;
    hipError_t e = nvfp4k_quant(
        mode, rotated ? 1 : 0, layouts, x, rows, cols, row_out ? row_out->codes : nullptr,
        row_out ? row_out->scales : nullptr, row_out ? row_out->tensor_scale : nullptr,
        col_out ? col_out->codes : nullptr, col_out ? col_out->scales : nullptr,
        col_out ? col_out->tensor_scale : nullptr, amax, seed, rht_seed,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// Workspace of the strip-local quantizer (a scale table per strip, wave maxima per tile),
// padded to 256 bytes.
size_t strip_workspace_bytes(int64_t rows, int64_t cols)
{
    if (rows < 0 || cols < 0 || !fits(rows, cols)) return MIN_WORKSPACE_BYTES;
    const size_t b = nvfp4k_strip_workspace(rows, cols);
    return b < MIN_WORKSPACE_BYTES ? MIN_WORKSPACE_BYTES : (b + 255) / 256 * 256;
}

int quantize_common(int local, int mode, const void *x, int64_t rows, int64_t cols, int group,
                    int block, uint64_t seed, int rht, uint64_t rht_seed,
                    const nvfp4_tensor *row_out, const nvfp4_tensor *col_out, void *workspace,
                    size_t workspace_bytes, void *stream, bool own_scratch = false)
{
    int rc = check_outputs(row_out, col_out, rows, cols);
    if (rc) return rc;
    rc = check_input(mode, x, rows, cols, group, block, rht, row_out != nullptr,
                     col_out != nullptr);
    if (rc) return rc;
    if (own_scratch) {
        // the library's own device scratch (eden_quantize_noalloc), once the arguments are
        // known to be good: looked up on the current device, never allocated
        rc = check_device();
        if (rc) return rc;
        if (nvfp4k_scratch(&workspace, &workspace_bytes) != hipSuccess) {
            (void)hipGetLastError();
            return NVFP4_ERR_HIP;
        }
    }
    const size_t need = local ? strip_workspace_bytes(rows, cols) : nvfp4k_workspace();
    if (!workspace || workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
    rc = check_device();
    if (rc) return rc;
    const int layouts = (row_out ? 1 : 0) | (col_out ? 2 : 0);
    const bool rotated = rht || mode == MODE_EDEN;
    const hipError_t e = (local ? nvfp4k_quant_strips : nvfp4k_quantize)(
        mode, rotated ? 1 : 0, layouts, x, rows, cols, row_out ? row_out->codes : nullptr,
        row_out ? row_out->scales : nullptr, row_out ? row_out->tensor_scale : nullptr,
        col_out ? col_out->codes : nullptr, col_out ? col_out->scales : nullptr,
        col_out ? col_out->tensor_scale : nullptr, workspace, seed, rht_seed,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int dequantize_common(int local, const nvfp4_tensor *in, int64_t vecs, int64_t n, int group,
                      int block, int rht, uint64_t rht_seed, float *out, void *stream)
{
    if (!in || !in->tensor_scale) return NVFP4_ERR_NULL;
    if ((vecs > 0 && n > 0) && (!out || !in->codes || !in->scales)) return NVFP4_ERR_NULL;
    if (group != 128 || block != 16) return NVFP4_ERR_GROUP;
    if (rht != 0 && rht != 1) return NVFP4_ERR_ARG;
    if (vecs < 0 || n < 0) return NVFP4_ERR_SHAPE;
    if (!fits(vecs, n)) return NVFP4_ERR_ARG;
    if (n % (rht ? 128 : 16)) return NVFP4_ERR_SHAPE;
    if (!aligned(in->codes, 8) || !aligned(in->scales, 1) || !aligned(in->tensor_scale, 4) ||
        !aligned(out, 16))
        return NVFP4_ERR_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = nvfp4k_dequantize(local, in->codes, in->scales, in->tensor_scale, vecs, n,
                                     rht, rht_seed, out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int gemm_common(int local, const nvfp4_tensor *a, const nvfp4_tensor *b, int64_t M, int64_t N,
                int64_t K, int rotated_pair, float *c, void *stream)
{
    if (!a || !b || !a->tensor_scale || !b->tensor_scale) return NVFP4_ERR_NULL;
    if (rotated_pair != 0 && rotated_pair != 1) return NVFP4_ERR_ARG;
    if (M < 0 || N < 0 || K < 0) return NVFP4_ERR_SHAPE;
    if (!fits(M, N) || !fits(M, K) || !fits(N, K)) return NVFP4_ERR_ARG;
    if (M % 32 || N % 32 || K % 64) return NVFP4_ERR_SHAPE;
    if (M > 0 && N > 0 && (!c || (K > 0 && (!a->codes || !a->scales || !b->codes || !b->scales))))
        return NVFP4_ERR_NULL;
    if (!aligned(a->codes, 16) || !aligned(b->codes, 16) || !aligned(a->scales, 2) ||
        !aligned(b->scales, 2) || !aligned(c, 4) || !aligned(a->tensor_scale, 4) ||
        !aligned(b->tensor_scale, 4))
        return NVFP4_ERR_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = nvfp4k_gemm(local, a->codes, a->scales, a->tensor_scale, b->codes, b->scales,
                               b->tensor_scale, M, N, K, rotated_pair, c,
                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace

extern "C" {

size_t nvfp4_workspace_bytes(int64_t rows, int64_t cols, int layouts_mask)
{
    (void)rows;
    (void)cols;
    (void)layouts_mask;
    return nvfp4k_workspace();
}

const char *nvfp4_strerror(int status)
{
    switch (status) {
    case NVFP4_OK: return "success";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "unsupported shape (negative size, cols % 8, or n not a multiple of 128/16)";
    case NVFP4_ERR_GROUP: return "group must be 128 and block must be 16";
    case NVFP4_ERR_ALIGN: return "misaligned pointer";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_HIP: return "HIP error (launch failure or no device)";
    case NVFP4_ERR_ARG: return "invalid argument";
    default: return "unknown status";
    }
}

int eden_quantize(const void *x_bf16, int64_t rows, int64_t cols, int group, int block,
                  uint64_t seed, uint64_t rht_seed, const nvfp4_tensor *row_out,
                  const nvfp4_tensor *col_out, void *workspace, size_t workspace_bytes,
                  void *stream)
{
    return quantize_common(0, MODE_EDEN, x_bf16, rows, cols, group, block, seed, 1, rht_seed,
                           row_out, col_out, workspace, workspace_bytes, stream);
}

int eden_quantize_noalloc(const void *x_bf16, int64_t rows, int64_t cols, int group, int block,
                          uint64_t seed, uint64_t rht_seed, const nvfp4_tensor *row_out,
                          const nvfp4_tensor *col_out, void *stream)
{
    return quantize_common(0, MODE_EDEN, x_bf16, rows, cols, group, block, seed, 1, rht_seed,
                           row_out, col_out, nullptr, 0, stream, true);
}

int sr_quantize(const void *x_bf16, int64_t rows, int64_t cols, int group, int block,
                uint64_t seed, int rht, uint64_t rht_seed, const nvfp4_tensor *row_out,
                const nvfp4_tensor *col_out, void *workspace, size_t workspace_bytes,
                void *stream)
{
    return quantize_common(0, MODE_SR, x_bf16, rows, cols, group, block, seed, rht, rht_seed,
                           row_out, col_out, workspace, workspace_bytes, stream);
}

int rtn_quantize(const void *x_bf16, int64_t rows, int64_t cols, int group, int block, int rht,
                 uint64_t rht_seed, const nvfp4_tensor *row_out, const nvfp4_tensor *col_out,
                 void *workspace, size_t workspace_bytes, void *stream)
{
    return quantize_common(0, MODE_RTN, x_bf16, rows, cols, group, block, 0, rht, rht_seed,
                           row_out, col_out, workspace, workspace_bytes, stream);
}

int fp46_quantize(const void *x_bf16, int64_t rows, int64_t cols, int group, int block, int rht,
                  uint64_t rht_seed, const nvfp4_tensor *row_out, const nvfp4_tensor *col_out,
                  void *workspace, size_t workspace_bytes, void *stream)
{
    return quantize_common(0, MODE_FP46, x_bf16, rows, cols, group, block, 0, rht, rht_seed,
                           row_out, col_out, workspace, workspace_bytes, stream);
}

int nvfp4_amax(const void *x_bf16, int64_t rows, int64_t cols, int group, int block, int rht,
               uint64_t rht_seed, int layouts_mask, float *amax, void *stream)
{
    if (!amax) return NVFP4_ERR_NULL;
    if (layouts_mask < 1 || layouts_mask > 3) return NVFP4_ERR_ARG;
    int rc = check_input(MODE_RTN, x_bf16, rows, cols, group, block, rht, layouts_mask & 1,
                         layouts_mask & 2);
    if (rc) return rc;
    if (!aligned(amax, 4)) return NVFP4_ERR_ALIGN;
    rc = check_device();
    if (rc) return rc;
    hipError_t e = nvfp4k_amax(rht, layouts_mask, x_bf16, rows, cols, amax, rht_seed,
                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int nvfp4_quantize_amax(int mode, const void *x_bf16, int64_t rows, int64_t cols, int group,
                        int block, uint64_t seed, int rht, uint64_t rht_seed, const float *amax,
                        const nvfp4_tensor *row_out, const nvfp4_tensor *col_out, void *stream)
{
    if (!amax) return NVFP4_ERR_NULL;
    int rc = check_outputs(row_out, col_out, rows, cols);
    if (rc) return rc;
    rc = check_input(mode, x_bf16, rows, cols, group, block, rht, row_out != nullptr,
                     col_out != nullptr);
    if (rc) return rc;
    if (!aligned(amax, 4)) return NVFP4_ERR_ALIGN;
    rc = check_device();
    if (rc) return rc;
    return launch_quant(mode, x_bf16, rows, cols, seed, rht, rht_seed, amax, row_out, col_out,
                        stream);
}

int dequantize(const nvfp4_tensor *in, int64_t vecs, int64_t n, int group, int block, int rht,
               uint64_t rht_seed, float *out, void *stream)
{
    return dequantize_common(0, in, vecs, n, group, block, rht, rht_seed, out, stream);
}

int nvfp4_gemm_check(const nvfp4_tensor *a, const nvfp4_tensor *b, int64_t M, int64_t N,
                     int64_t K, int rotated_pair, float *c, void *stream)
{
    return gemm_common(0, a, b, M, N, K, rotated_pair, c, stream);
}

size_t nvfp4_strip_workspace_bytes(int64_t rows, int64_t cols, int layouts_mask)
{
    (void)layouts_mask;
    return strip_workspace_bytes(rows, cols);
}

int nvfp4_quantize_strips(int mode, const void *x_bf16, int64_t rows, int64_t cols, int group,
                          int block, uint64_t seed, int rht, uint64_t rht_seed,
                          const nvfp4_tensor *row_out, const nvfp4_tensor *col_out,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    return quantize_common(1, mode, x_bf16, rows, cols, group, block, seed, rht, rht_seed,
                           row_out, col_out, workspace, workspace_bytes, stream);
}

int dequantize_strips(const nvfp4_tensor *in, int64_t vecs, int64_t n, int group, int block,
                      int rht, uint64_t rht_seed, float *out, void *stream)
{
    return dequantize_common(1, in, vecs, n, group, block, rht, rht_seed, out, stream);
}

int nvfp4_gemm_check_strips(const nvfp4_tensor *a, const nvfp4_tensor *b, int64_t M, int64_t N,
                            int64_t K, int rotated_pair, float *c, void *stream)
{
    return gemm_common(1, a, b, M, N, K, rotated_pair, c, stream);
}

int mxfp4_quantize(const void *x_bf16, int64_t rows, int64_t cols, int block, int sr,
                   uint64_t seed, int rht, uint64_t rht_seed, const mxfp4_tensor *row_out,
                   const mxfp4_tensor *col_out, void *stream)
{
    if (!row_out && !col_out) return NVFP4_ERR_NULL;
    const bool empty = rows == 0 || cols == 0;
    for (const mxfp4_tensor *t : {row_out, col_out}) {
        if (!t) continue;
        if (!empty && (!t->codes || !t->scales)) return NVFP4_ERR_NULL;
        if (!aligned(t->codes, 16) || !aligned(t->scales, 4)) return NVFP4_ERR_ALIGN;
        if (t->k_tiled != 0 && t->k_tiled != 1) return NVFP4_ERR_ARG;
    }
    if (!x_bf16 && !empty) return NVFP4_ERR_NULL;
    if (block != 32) return NVFP4_ERR_GROUP;
    if ((sr != 0 && sr != 1) || (rht != 0 && rht != 1)) return NVFP4_ERR_ARG;
    if (rows < 0 || cols < 0) return NVFP4_ERR_SHAPE;
    if (!fits(rows, cols)) return NVFP4_ERR_ARG;
    if (cols % 8) return NVFP4_ERR_SHAPE;
    if (row_out && cols % (rht || row_out->k_tiled ? 128 : 32)) return NVFP4_ERR_SHAPE;
    if (col_out && rows % (rht || col_out->k_tiled ? 128 : 32)) return NVFP4_ERR_SHAPE;
    if (!aligned(x_bf16, 16)) return NVFP4_ERR_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    const int layouts = (row_out ? 1 : 0) | (col_out ? 2 : 0);
    const hipError_t e = nvfp4k_quant_mx(
        sr, rht, layouts, x_bf16, rows, cols, row_out ? row_out->codes : nullptr,
        row_out ? row_out->scales : nullptr, row_out ? row_out->k_tiled : 0,
        col_out ? col_out->codes : nullptr, col_out ? col_out->scales : nullptr,
        col_out ? col_out->k_tiled : 0, seed, rht_seed, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int mxfp4_gemm(const mxfp4_tensor *a, const mxfp4_tensor *b, int64_t M, int64_t N, int64_t K,
               int rotated_pair, float *c, void *stream)
{
    if (!a || !b) return NVFP4_ERR_NULL;
    if (rotated_pair != 0 && rotated_pair != 1) return NVFP4_ERR_ARG;
    if ((a->k_tiled != 0 && a->k_tiled != 1) || a->k_tiled != b->k_tiled) return NVFP4_ERR_ARG;
    if (M < 0 || N < 0 || K < 0) return NVFP4_ERR_SHAPE;
    if (!fits(M, N) || !fits(M, K) || !fits(N, K)) return NVFP4_ERR_ARG;
    if (M % 32 || N % 32 || K % 128) return NVFP4_ERR_SHAPE;
    if (M > 0 && N > 0 && (!c || (K > 0 && (!a->codes || !a->scales || !b->codes || !b->scales))))
        return NVFP4_ERR_NULL;
    if (!aligned(a->codes, 16) || !aligned(b->codes, 16) || !aligned(a->scales, 4) ||
        !aligned(b->scales, 4) || !aligned(c, 4))
        return NVFP4_ERR_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    const hipError_t e = nvfp4k_gemm_mx(a->codes, a->scales, b->codes, b->scales, M, N, K,
                                        a->k_tiled, rotated_pair, c,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // extern "C"
