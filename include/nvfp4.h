/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 quantizer library libnvfp4.so.
 *
 * The library implements the hot path of Quartet II, the MS-EDEN unbiased NVFP4 quantizer,
 * with the plain stochastic-rounding (SR) baseline, round-to-nearest (RTN), the forward-pass
 * "4/6" grid choice, a producer that emits both packed layouts in one pass, a dequantizer,
 * a GEMM check consumer, the strip-local ("CTA-local") scaling variant of each, and a native
 * FP4 recipe (MXFP4 producer and GEMM on the FP4 matrix cores).  Definitions follow the pages
 * summarising "Quartet II: Accurate LLM Pre-Training in NVFP4 by Improved Unbiased Gradient
 * Estimation":
 *   - Telegram digest quant_prune_distill post 640, section "Method": SR; EDEN (random
 *     Hadamard rotation, then multiplication by <x,x> / <Q(Rx), Rx>); stochastic rounding of
 *     the scales to FP8; the 4/6 choice between the (-6,6) and (-4,4) grids; 1x16 groups.
 *   - itsolotime.com summary, Q1 "theory vs hardware compromises": fixed 128-dim rotation
 *     groups, one rotation per tensor, no SR for scales below about 1/32000 of the max.
 *   - rit.work note on "Format-Aware Fusion for Fast FP4 Pretraining": the global NVFP4 max
 *     is a synchronisation point; one producer writes both layouts a GEMM pair needs.
 * The arithmetic is fixed in binary32 (one rounding per operation, no FMA contraction) and
 * in a fixed order (the rotation's butterfly stages by ascending span, every scalar product
 * and sum of squares as per-term products joined by a balanced pairwise sum in natural
 * order), so that results are reproducible bit for bit.
 *
 * Conventions shared by every entry point
 *   Pointers.   Every data pointer is a DEVICE pointer allocated by the caller (e.g. a torch
 *               CUDA/HIP tensor).  The library never allocates.  Its only state is per
 *               device and fixed once looked up (the compute-unit count, and for
 *               eden_quantize_noalloc the address of its device scratch), so calls that
 *               bring their own workspace are thread-safe; calls on one stream are ordered.
 *   Stream.     `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *               work is enqueued asynchronously on it; results are valid once it is
 *               synchronised.  Nothing is copied to the host: the tensor scale stays on the
 *               device.
 *   Errors.     Return 0 on success, a negative NVFP4_ERR_* code otherwise.  Argument
 *               errors are detected synchronously, before anything is enqueued, and leave
 *               every output untouched.  NVFP4_ERR_HIP reports a failed launch or no device.
 *   Input.      x is a row-major BF16 matrix [rows][cols], 16-byte aligned, cols % 8 == 0.
 *               Values must be finite with |x| < 2^56; other values give unspecified
 *               codes but no fault.  rows, cols < 2^31 and rows * cols < 2^40.
 *   Layouts.    The row layout quantizes the rows of X (vectors = rows, n = cols); the
 *               column layout quantizes the columns (vectors = cols, n = rows), i.e. it is
 *               the row layout of X^T, with its own tensor scale and random stream.
 *               Pass NULL for a layout that is not wanted; at least one is required.
 *               Each layout's n must be a multiple of 128 when the rotation is on (always
 *               for MS-EDEN) and of 16 otherwise.
 *   Output.     nvfp4_tensor for a layout with vecs vectors of length n:
 *                 codes  [vecs][n/2] bytes, byte j = code(2j) | code(2j+1) << 4, where a
 *                        code is sign << 3 | magnitude index into {0,.5,1,1.5,2,3,4,6},
 *                        the sign bit set iff the rotated value is negative (an exact
 *                        zero encodes as 0); 16-byte aligned;
 *                 scales [vecs][n/16] OCP E4M3FN bytes (one per 1x16 block), 8-byte aligned;
 *                 tensor_scale: one float g, 4-byte aligned.
 *               A value decodes as sign * (E4M3(scale) * g) * magnitude; with the rotation
 *               on, the decoded vector is in the rotated domain (see dequantize).
 *   group/block Must be 128 and 16 (NVFP4 1x16 blocks; 128-element rotation groups).
 *   Aliasing.   Output buffers must not overlap one another, the input or the workspace;
 *               overlapping buffers give undefined results.
 *   Workspace.  Device scratch of at least nvfp4_workspace_bytes() bytes, 256-byte aligned,
 *               owned by the caller.  On the stream, the library writes every byte of it
 *               that it reads before reading it; its contents between calls do not matter.
 *               Concurrent calls need distinct workspaces.
 *   Seeds.      rht_seed selects the rotation's random signs, shared by every group and both
 *               layouts; both operands of one GEMM must use the same rht_seed.  seed drives
 *               stochastic rounding (Philox4x32-10 counter streams).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_OK 0
#define NVFP4_ERR_NULL (-1)      /* a required pointer is NULL */
#define NVFP4_ERR_SHAPE (-2)     /* negative size, or n not a multiple of 128 / 16, cols % 8 */
#define NVFP4_ERR_GROUP (-3)     /* group != 128 or block != 16 */
#define NVFP4_ERR_ALIGN (-4)     /* a pointer violates the alignment stated above */
#define NVFP4_ERR_WORKSPACE (-5) /* workspace NULL or smaller than nvfp4_workspace_bytes() */
#define NVFP4_ERR_HIP (-6)       /* HIP launch failure or no usable device */
#define NVFP4_ERR_ARG (-7)       /* other invalid argument (flag value, size too large) */

/* Quantizer selector of the two-phase entry points. */
#define NVFP4_MODE_RTN 0
#define NVFP4_MODE_SR 1
#define NVFP4_MODE_EDEN 2
#define NVFP4_MODE_FP46 3

typedef struct nvfp4_tensor {
    uint8_t *codes;      /* [vecs][n/2]  packed E2M1 codes, low nibble first */
    uint8_t *scales;     /* [vecs][n/16] E4M3FN block scales */
    float *tensor_scale; /* [1]          FP32 tensor scale g */
} nvfp4_tensor;

/* Bytes of workspace the quantizers need for a rows x cols input and the layouts in
 * layouts_mask (bit 0 = row, bit 1 = column).  Never fails; 0 means none needed.  Today a
 * fixed 16 KiB: the two partial maxima (row, column) of each phase-1 workgroup (at most
 * 2048), which every phase-2 workgroup reduces before it rounds a scale. */
size_t nvfp4_workspace_bytes(int64_t rows, int64_t cols, int layouts_mask);

/* Human-readable text for a status code (static storage). */
const char *nvfp4_strerror(int status);

/* MS-EDEN (Telegram digest "Method"; itsolotime Q1): per 128-group random-sign Hadamard
 * rotation r = H(sigma * x); FP32 tensor scale g = amax|r| / 2688; 1x16 E4M3 scales by
 * round-to-nearest of max|r| / (6g); elements rounded to nearest on the E2M1 grid; EDEN ratio
 * S = <r,r>/<r,q> per group; each scale replaced by a stochastic rounding of S * scale to
 * E4M3 (no SR below 2^-6; saturating at 448).  Codes stay the RTN codes.  Decoding gives an
 * unbiased estimate of r in the rotated domain.  Both layouts in one pass when both given. */
int eden_quantize(const void *x_bf16, int64_t rows, int64_t cols, int group, int block,
                  uint64_t seed, uint64_t rht_seed, const nvfp4_tensor *row_out,
                  const nvfp4_tensor *col_out, void *workspace, size_t workspace_bytes,
                  void *stream);

/* eden_quantize() for callers that cannot allocate device memory or bring a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments (without the workspace), outputs, errors and results, bit for bit, as
 * eden_quantize.  The phase-1 maxima go to a 16 KiB array in device memory that the library
 * owns (one copy per GPU, held until the process ends); 16 KiB covers every shape the
 * library accepts, and a call that needed more would be rejected with NVFP4_ERR_WORKSPACE.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library routine); its
 * first call on a device looks up that device's copy of the array.  Every call on one GPU
 * shares that array and finds it as the last call left it (nothing in it needs clearing):
 * calls that overlap on one GPU -- on different streams, or from different threads -- race
 * and give undefined results; calls on one stream are ordered and safe. */
int eden_quantize_noalloc(const void *x_bf16, int64_t rows, int64_t cols, int group, int block,
                          uint64_t seed, uint64_t rht_seed, const nvfp4_tensor *row_out,
                          const nvfp4_tensor *col_out, void *stream);

/* Plain stochastic rounding (itsolotime opening paragraph; Telegram "Method"): tensor scale
 * amax / 2688, block scale rounded UP to E4M3 (no element clips), each element rounded to
 * one of its two E2M1 neighbours with probability given by its distance to them: the top 22
 * bits v of element e's Philox word (word e mod 4 of Philox(seed, (e/4 lo, e/4 hi, 3,
 * layout)), e = vector * n + position) are added to its fraction as v * 2^-22 and the sum is
 * rounded down, so the probability of rounding up is floor(frac * 2^22) / 2^22.
 * rht != 0 rotates first (random-sign Hadamard, as MS-EDEN), rht == 0 quantizes x as is. */
int sr_quantize(const void *x_bf16, int64_t rows, int64_t cols, int group, int block,
                uint64_t seed, int rht, uint64_t rht_seed, const nvfp4_tensor *row_out,
                const nvfp4_tensor *col_out, void *workspace, size_t workspace_bytes,
                void *stream);

/* Round-to-nearest NVFP4 (no randomness; denisavetisyan.com paraphrase, "NVFP4 and
 * micro-scaling": E2M1 elements under an FP8 scale per 16 and an FP32 tensor scale; Telegram
 * "Method": round-to-nearest is the biased baseline MS-EDEN corrects): tensor scale
 * amax / 2688, block scale and elements rounded to nearest (ties to even), optional rotation
 * as above. */
int rtn_quantize(const void *x_bf16, int64_t rows, int64_t cols, int group, int block,
                 int rht, uint64_t rht_seed, const nvfp4_tensor *row_out,
                 const nvfp4_tensor *col_out, void *workspace, size_t workspace_bytes,
                 void *stream);

/* Forward-pass 4/6 (Telegram "Method"): tensor scale amax / 1792; per 1x16 block, RTN on
 * the full +-6 grid (scale max/(6g)) and on the clipped +-4 grid (scale max/(4g)); the block
 * keeps whichever has the lower sum of squared errors (ties keep +-6).  Optional rotation. */
int fp46_quantize(const void *x_bf16, int64_t rows, int64_t cols, int group, int block,
                  int rht, uint64_t rht_seed, const nvfp4_tensor *row_out,
                  const nvfp4_tensor *col_out, void *workspace, size_t workspace_bytes,
                  void *stream);

/* The two phases of every quantizer above, for callers that must act on the tensor-wide
 * maximum between them.  The rit.work note on "Format-Aware Fusion for Fast FP4 Pretraining"
 * ("speedup is lost between matmuls") names the global NVFP4 maximum as the one
 * synchronisation point of the producer: no scale can be rounded before the partial maxima
 * of the whole tensor are collected.  A tensor sharded over several GPUs runs phase 1 on
 * each shard, combines the two floats with an all-reduce(MAX), then runs phase 2.
 *
 * Phase 1: amax[0] = max |r| over the row layout, amax[1] = over the column layout, where
 * r is x rotated per 128-group when rht != 0 (always rotate for MS-EDEN) and x itself
 * otherwise.  amax is a device float[2] (4-byte aligned) written on `stream`; the slot of a
 * layout not in layouts_mask (bit 0 row, bit 1 column) is set to 0.  Shape rules as for the
 * quantizers.  The tensor scale phase 2 derives is amax / 2688 (amax / 1792 for 4/6). */
int nvfp4_amax(const void *x_bf16, int64_t rows, int64_t cols, int group, int block, int rht,
               uint64_t rht_seed, int layouts_mask, float *amax, void *stream);

/* Phase 2: quantizer `mode` (NVFP4_MODE_*) of x given the phase-1 maxima in amax (device
 * float[2], read on `stream`).  Same arguments, outputs and rules as the one-call entry
 * points (rht is ignored and taken as 1 for MS-EDEN; seed is unused by RTN and 4/6).  With
 * amax from nvfp4_amax on the same inputs, the result is bit-identical to the one-call
 * quantizer's. */
int nvfp4_quantize_amax(int mode, const void *x_bf16, int64_t rows, int64_t cols, int group,
                        int block, uint64_t seed, int rht, uint64_t rht_seed, const float *amax,
                        const nvfp4_tensor *row_out, const nvfp4_tensor *col_out, void *stream);

/* Decode vecs vectors of length n from `in` into out [vecs][n] FP32 (device, 16-byte
 * aligned; codes 8-byte aligned): the value the NVFP4 format assigns to a code
 * (denisavetisyan.com paraphrase, "NVFP4 and micro-scaling": element times block scale times
 * tensor scale), sign * (E4M3(scale) * g) * magnitude.  With rht != 0 the rotation is undone,
 * x_j = sigma_j * (H q)_j * 2^-7 (H H = 128 I), using the signs of rht_seed, so the output
 * is in the original domain; n must then be a multiple of 128 (else of 16). */
int dequantize(const nvfp4_tensor *in, int64_t vecs, int64_t n, int group, int block,
               int rht, uint64_t rht_seed, float *out, void *stream);

/* GEMM check consumer (itsolotime.com summary, abstract: every linear layer's products run
 * on NVFP4 operands): C[m][n] = f * gA * gB * sum_k a(m,k) * b(n,k), where a(m,k) =
 * sign * E4M3(scale) * magnitude of code (m,k) of `a` and likewise for `b`, and f = 2^-7
 * when rotated_pair != 0 (both operands rotated along K with the same rht_seed, so
 * H H = 128 I cancels the rotation) else 1.  a is [M][K] and b is [N][K], both in the
 * row layout (K contiguous, as the quantizers emit; codes 16-byte and scales 2-byte
 * aligned); c is FP32 [M][N] row-major (device, 4-byte aligned).  Operand values are dequantized exactly to FP16 and multiplied on the
 * matrix cores with FP32 accumulation (summation order unspecified).  M and N must be
 * multiples of 32 and K a multiple of 64. */
int nvfp4_gemm_check(const nvfp4_tensor *a, const nvfp4_tensor *b, int64_t M, int64_t N,
                     int64_t K, int rotated_pair, float *c, void *stream);

/* ------------------------------------------------------------------ strip-local scales
 * The CTA-local variant in the rit.work note on "Format-Aware Fusion for Fast FP4
 * Pretraining" (section "speedup is lost between matmuls"): the maximum behind the FP32
 * second-level scale is taken inside one block of work instead of over the whole tensor, so
 * no block waits for the tensor-wide maximum, and the GEMM applies separate row and column
 * corrections after its sum over K.  The note's closing section adds that this changes the
 * numerical contract and has to be evaluated as a training recipe of its own.  Reading taken here: a correction that stays
 * fixed during the sum over K covers whole vectors, so each layout's vectors form strips of
 * 128 consecutive vectors (one tile row of X for the row layout, one tile column for the
 * column layout), and strip s has its own g_s = max |r| over the strip / 2688 (/ 1792 for
 * 4/6).  Every vector is then quantized exactly as by the quantizer of the same mode with
 * g_s in place of g; random streams keep the vector's index in the whole layout.
 *
 * Outputs differ from nvfp4_tensor's global form in one field: tensor_scale points to
 * ceil(vecs / 128) floats (4-byte aligned), g of vector v being tensor_scale[v / 128]. */

/* Workspace bytes of nvfp4_quantize_strips for a rows x cols input: a 2 KiB scale table per
 * row strip and per column strip, plus 32 bytes per 128 x 128 tile (the maxima the strip
 * reduction reads), rounded up to a multiple of 256.  Never fails. */
size_t nvfp4_strip_workspace_bytes(int64_t rows, int64_t cols, int layouts_mask);

/* Quantizer `mode` (NVFP4_MODE_*) with strip-local scales.  Arguments, shapes, seeds, errors
 * and the two layouts as for the one-call quantizers (rht is taken as 1 for MS-EDEN; seed is
 * unused by RTN and 4/6); the workspace must hold nvfp4_strip_workspace_bytes() bytes.  Three
 * launches on `stream`: the rotated maxima of every tile, one reduction per strip (which
 * writes g and the strip's scale table into the workspace), then the quantization. */
int nvfp4_quantize_strips(int mode, const void *x_bf16, int64_t rows, int64_t cols, int group,
                          int block, uint64_t seed, int rht, uint64_t rht_seed,
                          const nvfp4_tensor *row_out, const nvfp4_tensor *col_out,
                          void *workspace, size_t workspace_bytes, void *stream);

/* dequantize() for strip-local outputs: vector v decodes with tensor_scale[v / 128]. */
int dequantize_strips(const nvfp4_tensor *in, int64_t vecs, int64_t n, int group, int block,
                      int rht, uint64_t rht_seed, float *out, void *stream);

/* nvfp4_gemm_check() for strip-local operands: C[m][n] = f * gA[m / 128] * gB[n / 128] *
 * sum_k a(m,k) * b(n,k), the row correction of A and the column correction of B applied after
 * the sum over K.  a and b are row layouts of nvfp4_quantize_strips ([M][K] and [N][K]). */
int nvfp4_gemm_check_strips(const nvfp4_tensor *a, const nvfp4_tensor *b, int64_t M, int64_t N,
                            int64_t K, int rotated_pair, float *c, void *stream);

/* ------------------------------------------------------------------ MXFP4 (native FP4)
 * The recipe of the native FP4 matrix-core consumer.  Quartet II runs its linear layers on
 * FP4 matrix cores (itsolotime.com summary, abstract: NVFP4 GEMM kernels up to 4.2x over
 * BF16).  gfx950's scaled matrix instructions multiply E2M1 elements that carry one power-of-
 * two (E8M0) scale per 32 elements along K; an NVFP4 operand's E4M3 scales per 16 (3 mantissa
 * bits) cannot ride on them, so this recipe has a block contract of its own ("MXFP4"): the
 * vectors, layouts, rotation (rht, rht_seed as for the NVFP4 quantizers) and random streams of
 * the NVFP4 quantizers; blocks of 32; block scale 2^e with e the smallest integer such that
 * 6 * 2^e >= max |r| over the block (nothing clips, so SR stays unbiased), clamped to
 * [-127, 127]; elements y = r * 2^-e rounded to the E2M1 grid by round-to-nearest-even
 * (sr == 0; Telegram digest "Method") or stochastically (sr == 1; itsolotime opening
 * paragraph; the draw of element e of a layout is the top 22 bits of word e mod 4 of
 * Philox(seed, (e/4 lo, e/4 hi, 3, layout)), added to the fraction and rounded down as for
 * sr_quantize).  MS-EDEN has no MXFP4 form here: stochastic rounding of its corrected
 * scales onto powers of two would add several percent of variance.  No tensor scale. */
typedef struct mxfp4_tensor {
    uint8_t *codes;      /* packed E2M1 codes, low nibble first; 16-byte aligned */
    uint8_t *scales;     /* E8M0 bytes, scale = 2^(byte - 127); 4-byte aligned */
    int32_t k_tiled;     /* 0: codes [vecs][n/2], scales [vecs][n/32] (row-major).
                          * 1: K-tiled, n a multiple of 128: codes [n/128][vecs][64] and
                          *    scales [n/128][vecs][4], i.e. code byte j of vector v at
                          *    (j / 64) * vecs * 64 + v * 64 + j % 64 and scale byte s at
                          *    (s / 4) * vecs * 4 + v * 4 + s % 4.  The same values as the
                          *    row-major form, stored so that a GEMM's K step of many rows is
                          *    one contiguous piece. */
} mxfp4_tensor;

/* MXFP4 quantization of x (as for the NVFP4 quantizers: BF16 row-major, 16-byte aligned,
 * cols % 8 == 0) in one or both layouts, one pass (no tensor-wide maximum is needed).
 * block must be 32; each requested layout's n a multiple of 32 (128 with the rotation or when
 * that layout is K-tiled; k_tiled must be 0 or 1).  No workspace; errors as in the
 * conventions above. */
int mxfp4_quantize(const void *x_bf16, int64_t rows, int64_t cols, int block, int sr,
                   uint64_t seed, int rht, uint64_t rht_seed, const mxfp4_tensor *row_out,
                   const mxfp4_tensor *col_out, void *stream);

/* C[m][n] = f * sum_k a(m,k) * b(n,k) on the FP4 matrix cores (v_mfma_scale_f32_32x32x64_
 * f8f6f4), a(m,k) = sign * magnitude * 2^(scale byte - 127) of `a` [M][K] and likewise of `b`
 * [N][K] (row layouts: K is each vector's n); f = 2^-7 when rotated_pair != 0 (both operands
 * rotated along K with the same rht_seed) else 1.  Products exact, FP32 accumulation over K in
 * ascending 64-element steps (so row-major and K-tiled operands give the same bits).  c is
 * FP32 [M][N] row-major (device, 4-byte aligned).  M and N multiples of 32, K a multiple of
 * 128; a and b both row-major or both K-tiled (else NVFP4_ERR_ARG); K-tiled operands take the
 * faster kernel. */
int mxfp4_gemm(const mxfp4_tensor *a, const mxfp4_tensor *b, int64_t M, int64_t N, int64_t K,
               int rotated_pair, float *c, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
