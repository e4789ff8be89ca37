/*
 * bsq.h -- block-scaled quantization and expert GEMMs for AMD MI355X (gfx950).
 *
 * C ABI of libbsq.so. The operations follow "End-to-End 4-Bit Training"
 * (Thinking Machines Lab): NVFP4 (E2M1 values, one E4M3 scale per 1x16
 * block, one FP32 outer scale) and MXFP8 (E4M3 values, one E8M0 scale per
 * 1x32 block) from the section "Low-precision formats on Blackwell"; the
 * dequantize-transpose-requantize with stochastic rounding from the section
 * "Re-quantization with stochastic rounding" and its quantized linear layer
 * figure; the block-scaled forward and backward products from the section
 * "Block-scaled backward passes"; routing of tokens to experts from the
 * section "Quantized communications".
 *
 * Conventions for every entry point:
 *  - Buffers are device memory owned by the caller, except where a parameter
 *    is marked HOST. The library never allocates, frees or synchronizes, and
 *    keeps no state between calls beyond a per-device cache of the
 *    compute-unit count (sizes persistent grids); calls are thread-safe.
 *  - Work is enqueued on `stream` (0 = the null stream) and runs
 *    asynchronously. The return value reports argument validation (checked on
 *    the host before any HIP call) and launch errors only.
 *  - Device pointers must be 16-byte aligned unless stated otherwise.
 *  - Inputs are never modified; outputs are fully overwritten.
 *  - NaN or infinite inputs give unspecified (but memory-safe) results.
 *  - Layouts are row-major. NVFP4 codes hold two elements per byte, element
 *    2k in the low nibble. E4M3 is the OCP "FN" variant (max 448, no
 *    infinities). E8M0 code c means 2^(c-127).
 */
#ifndef BSQ_H
#define BSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* bsq_stream_t; /* a hipStream_t */

typedef enum {
  BSQ_OK = 0,
  BSQ_E_NULL = 1,      /* a required pointer is NULL */
  BSQ_E_SHAPE = 2,     /* a size is negative, not a multiple of the block, or too large */
  BSQ_E_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  BSQ_E_DTYPE = 4,     /* unknown element type */
  BSQ_E_ENUM = 5,      /* unknown mode, rounding or format value */
  BSQ_E_WORKSPACE = 6, /* workspace smaller than the size query returns */
  BSQ_E_LAUNCH = 7     /* a kernel launch failed (hipGetLastError) */
} bsq_status;

typedef enum { BSQ_F32 = 0, BSQ_BF16 = 1 } bsq_dtype;

/* Granularity of the FP32 outer scale ("Recipe details": per-expert for
 * weights, per-token for activations). */
typedef enum {
  BSQ_OUTER_TENSOR = 0, /* one per batch item (a tensor, or one expert's weights) */
  BSQ_OUTER_ROW = 1,    /* one per row (a token) */
  BSQ_OUTER_GIVEN = 2   /* one per batch item, read from outer_in */
} bsq_outer_mode;
/* Flag OR'ed into bsq_quantize_nvfp4's mode: Four Over Six block scales. */
enum { BSQ_NVFP4_FOUR_OVER_SIX = 16 };

typedef enum { BSQ_RN = 0, BSQ_SR = 1 } bsq_round;
typedef enum { BSQ_NVFP4 = 0, BSQ_MXFP8 = 1 } bsq_format;

/* Human-readable name of a status value. Never NULL. */
const char* bsq_status_string(int status);

/* ABI version of this header (major * 100 + minor). */
int bsq_version(void);

/* ------------------------------------------------------------------------
 * Round-to-nearest NVFP4 quantization ("Low-precision formats on Blackwell";
 * block scale from the block's largest magnitude, e.g. -54 -> -6 with scale
 * 9; x_i = q_i * s_{i//16} * s_t).
 *
 * x        [batch, rows, cols] of `dtype` (F32 or BF16), cols % 16 == 0.
 * mode     outer-scale granularity (bsq_outer_mode), optionally OR'ed with
 *          BSQ_NVFP4_FOUR_OVER_SIX.
 * outer_in [batch] FP32, required only for BSQ_OUTER_GIVEN (positive, normal).
 * codes    [batch, rows, cols/2] u8 (two E2M1 codes per byte).
 * scales   [batch, rows, cols/16] u8 (E4M3). 1-byte alignment suffices.
 * outer_out[batch] (TENSOR, GIVEN) or [batch*rows] (ROW) FP32; receives s_t.
 * ws       workspace of at least bsq_quantize_nvfp4_workspace() bytes
 *          (NULL when that is 0).
 * Per group: s_t = f32(amax/2688) (1 for an all-zero group). Per block:
 * r = f32(a_b / f32(6 s_t)), s_b = E4M3 round-to-nearest-even of r saturating
 * at 448; D = f32(s_b s_t); a block with D below 2^-126 stores magnitude 0;
 * else each element rounds f32(x * f32(1/D)) to the nearest E2M1 value (ties
 * to even, saturating at 6, sign kept).
 * Four Over Six ("Recipe details": for activations, each block chooses
 * between two scale factors to reduce quantization error; the quantized
 * linear layer figure applies it to the per-token activation quantize): the
 * block also forms s_b4 from r4 = f32(a_b / f32(4 s_t)) with its codes, and
 * keeps it when its squared error is strictly smaller; the error is
 * sum_i f32(e_i^2), e_i = f32(x_i - f32(f32(q_i s_b) s_t)), summed in float32
 * in element order (ties keep the 6 scale).
 * Limits: cols <= 32768. x and codes 16-byte aligned; outer_in, outer_out
 * and ws 4-byte aligned; scales 1-byte.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, ENUM, WORKSPACE, LAUNCH.
 * ---------------------------------------------------------------------- */
size_t bsq_quantize_nvfp4_workspace(int64_t batch, int64_t rows, int64_t cols, int mode);
int bsq_quantize_nvfp4(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                       int mode, const float* outer_in, uint8_t* codes, uint8_t* scales,
                       float* outer_out, void* ws, size_t ws_bytes, bsq_stream_t stream);

/* ------------------------------------------------------------------------
 * The quantization step of the expert chain ("Quantized communications",
 * Figure 5: w13 GEMM, quantize, w2 GEMM): SwiGLU of the w13 output, then
 * NVFP4 with one outer scale per row (a dispatched token row), as
 * bsq_quantize_nvfp4 with BSQ_OUTER_ROW.
 *
 * h13      [rows, 2*ffn] of `dtype` (F32 or BF16): gate columns [0, ffn), up
 *          columns [ffn, 2*ffn).
 * flags    0 or BSQ_NVFP4_FOUR_OVER_SIX.
 * codes    [rows, ffn/2] u8; scales [rows, ffn/16] u8; outer_out [rows] FP32.
 * h = silu(g) * u with silu(g) = g / (1 + e^-g), each step rounded to float32;
 * e^x = p(r) 2^n with n = round-half-even(f32(x * f32(1/ln 2))) clamped to
 * [-300, 300], r = f32(f32(x - n * 0.693145751953125) - f32(n * f32(ln 2 -
 * 0.693145751953125))) and p(r) = sum_{k<=7} r^k/k! in Horner form with every
 * product and sum rounded separately (coefficients f32 of c_k = c_(k-1)/k
 * formed in double precision).
 * ffn % 16 == 0, ffn <= 32768. h13 and codes 16-byte aligned, outer_out 4.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, ENUM, LAUNCH.
 * ---------------------------------------------------------------------- */
int bsq_swiglu_quantize_nvfp4(const void* h13, int dtype, int64_t rows, int64_t ffn, int flags,
                              uint8_t* codes, uint8_t* scales, float* outer_out, bsq_stream_t stream);

/* ------------------------------------------------------------------------
 * Square-tile NVFP4 quantization ("Block-scaled backward passes": the
 * alternative the pages compare against, one scale per 16x16 tile, shown in
 * the row-vs-column and outlier figures). Because the tile is square, the
 * quantization of the transpose is bitwise the transpose of the quantization;
 * the call can write both layouts from one read of x.
 *
 * x         [batch, rows, cols] of `dtype` (F32 or BF16); rows % 16 == 0 and
 *           cols % 16 == 0.
 * mode      BSQ_OUTER_TENSOR (s_t = f32(amax/2688) per batch item, 1 for an
 *           all-zero item) or BSQ_OUTER_GIVEN (outer_in [batch], positive).
 * codes     [batch, rows, cols/2] u8, two E2M1 codes per byte (element 2k in
 *           the low nibble), as bsq_quantize_nvfp4.
 * scales    [batch, rows, cols/16] u8 (E4M3): the 1x16 layout, each tile's
 *           scale repeated in its 16 rows, so the 1x16 consumers (the grouped
 *           GEMM, dequantize, requantize) read it unchanged.
 * codes_t   [batch, cols, rows/2] u8 and scales_t [batch, cols, rows/16] u8:
 *           the same quantization of x transposed (per item); both NULL to
 *           skip, else both non-NULL.
 * outer_out [batch] FP32, receives s_t.
 * ws        bsq_quantize_nvfp4_square_workspace() bytes (0 for GIVEN).
 * Per tile: a_t = max |x|; s_b = E4M3 round-to-nearest-even of
 * f32(a_t / f32(6 s_t)), saturating at 448; each element rounds as in
 * bsq_quantize_nvfp4 with that s_b.
 * Alignment: x, codes, codes_t 16 bytes; outer_in, outer_out, ws 4 bytes.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, ENUM (BSQ_OUTER_ROW or a flag),
 * WORKSPACE, LAUNCH.
 * ---------------------------------------------------------------------- */
size_t bsq_quantize_nvfp4_square_workspace(int64_t batch, int64_t rows, int64_t cols, int mode);
int bsq_quantize_nvfp4_square(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                              int mode, const float* outer_in, uint8_t* codes, uint8_t* scales,
                              uint8_t* codes_t, uint8_t* scales_t, float* outer_out, void* ws,
                              size_t ws_bytes, bsq_stream_t stream);

/* ------------------------------------------------------------------------
 * MXFP8 quantization of a gradient (quantized linear layer figure: the BF16
 * output gradient is quantized to MXFP8 with stochastic rounding, row-wise
 * for DGRAD and transposed for WGRAD).
 *
 * x          [rows, cols] of `dtype` (F32 or BF16).
 * transpose  0: blocks of 32 along cols; cols % 32 == 0; output codes
 *              [rows, cols], scales [rows, cols/32]; element index r*cols+c.
 *            1: rows are dispatched token rows grouped into num_segments
 *              expert segments by seg_offsets (device, int64 [num_segments+1],
 *              seg_offsets[0] == 0, nondecreasing, last == rows,
 *              1 <= num_segments <= 1024); segment e of length M_e is written
 *              as its transpose [cols, Mp_e], Mp_e = M_e rounded up to 32,
 *              zero padded, the segments one after another (the "padded
 *              per-segment transposed layout"); blocks of 32 run along tokens
 *              from the segment start; element index of (e, c, m) is
 *              cols * sum_{e'<e} Mp_e' + c * Mp_e + m. cols % 64 == 0,
 *              cols <= 4194304.
 *              seg_offsets == NULL means one segment covering all rows.
 *              Needs bsq_quantize_mxfp8_workspace() bytes of workspace. The
 *              caller sizes codes for cols * sum_e Mp_e bytes and scales for
 *              a 32nd of that; cols * (rows + 31 * num_segments) bounds the sum
 *              for any seg_offsets (the sizes are not checked: they depend on
 *              the device-side offsets). Malformed offsets are read as
 *              clamped to [0, rows] and then replaced by their running
 *              maximum (a decreasing offset ends the earlier segments'
 *              coverage: [0, R, 0, R] acts as [0, R, R, R]), so segments
 *              never overlap and the bound holds.
 * rnd        BSQ_RN (nearest-even) or BSQ_SR.
 * seed, stream_id  select the random stream (SR only).
 * E8M0 rule: the smallest 2^e with a_b <= 448 * 2^e (e clamped to [-127,127];
 * a zero block gets code 0); y = f32(x * 2^-e), so |y| <= 448.
 * SR: u = (r + 1/2) / 2^16 with r the 16 Philox4x32-10 bits of the element's
 * output index (see bsq_rng_bits16); the magnitude rounds up iff u < delta,
 * delta the position of |y| between its two E4M3 neighbours.
 * Codes and x must be 16-byte aligned, ws 16-byte aligned, scales 1-byte.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, ENUM, WORKSPACE, LAUNCH.
 * ---------------------------------------------------------------------- */
size_t bsq_quantize_mxfp8_workspace(int64_t rows, int transpose, int64_t num_segments);
int bsq_quantize_mxfp8(const void* x, int dtype, int64_t rows, int64_t cols, int transpose,
                       const int64_t* seg_offsets, int64_t num_segments, int rnd, uint64_t seed,
                       uint64_t stream_id, uint8_t* codes, uint8_t* scales, void* ws,
                       size_t ws_bytes, bsq_stream_t stream);

/* Both MXFP8 quantizations of the gradient from one read of x (the quantized
 * linear layer figure quantizes the BF16 output gradient row-wise for DGRAD
 * and transposed for WGRAD; both consume the same gradient).
 * Outputs are those of bsq_quantize_mxfp8 with transpose = 0 (codes, scales;
 * random stream stream_rows) and with transpose = 1 (codes_t, scales_t;
 * stream_t, the padded per-segment transposed layout), bit for bit, for every
 * row inside a segment (all rows when seg_offsets[0] == 0 and the last offset
 * == rows, or seg_offsets == NULL). Rows outside every segment (only with
 * offsets that do not cover [0, rows)) are not written in codes/scales.
 * cols % 64 == 0, cols <= 4194304; workspace bsq_quantize_mxfp8_workspace(rows, 1, num_segments);
 * x, codes, codes_t, ws 16-byte aligned. Errors: NULL, SHAPE, ALIGN, DTYPE,
 * ENUM, WORKSPACE, LAUNCH. */
int bsq_quantize_mxfp8_dual(const void* x, int dtype, int64_t rows, int64_t cols,
                            const int64_t* seg_offsets, int64_t num_segments, int rnd, uint64_t seed,
                            uint64_t stream_rows, uint64_t stream_t, uint8_t* codes, uint8_t* scales,
                            uint8_t* codes_t, uint8_t* scales_t, void* ws, size_t ws_bytes,
                            bsq_stream_t stream);

/* ------------------------------------------------------------------------
 * Dequantize -> transpose -> requantize with stochastic rounding ("Re-
 * quantization with stochastic rounding"; E[w_q] = E[(w_q^T)^T]).
 *
 * Input NVFP4 codes [in_rows, cols/2] (16-byte aligned), scales
 * [in_rows, cols/16] (u8), outer per in_mode: BSQ_OUTER_ROW -> outer[in_rows];
 * BSQ_OUTER_TENSOR -> outer[batch] (one per batch item; outer[0] in gather
 * mode). Dequantized value x^ = f32(f32(q * s_b) * s_t). cols % 64 == 0.
 *
 * Batch mode (row_gather == NULL, seg_offsets == NULL): the input is
 *   [batch, rows, cols] (in_rows == batch*rows) and the output is the
 *   transpose [batch, cols, rows] with blocks along rows; rows % 32 == 0 for
 *   MXFP8, rows % 16 == 0 for NVFP4. Element index b*cols*rows + c*rows + r.
 * Gather mode (row_gather and seg_offsets both given, batch == 1,
 *   out_fmt == BSQ_MXFP8): dispatched row m (0 <= m < rows) reads input row
 *   row_gather[m] (int32, < in_rows); rows are grouped into num_segments
 *   expert segments and written in the padded per-segment transposed layout
 *   of bsq_quantize_mxfp8(transpose=1), sized by the caller as described
 *   there (cols * (rows + 31 * num_segments) bounds it).
 * out_fmt BSQ_MXFP8: E8M0/E4M3 as in bsq_quantize_mxfp8 (no outer scale).
 * out_fmt BSQ_NVFP4: new outer s_t' = f32(max|x^|/2688) per batch item
 *   (written to out_outer[batch]); block scale r = f32(a_b / f32(6 s_t'))
 *   rounded UP to E4M3 (capped at 448), so no element exceeds 6; then
 *   y = f32(z * f32(1/D)) rounded onto the E2M1 grid.
 * rnd BSQ_SR (the method) or BSQ_RN (nearest-even, for comparison).
 * Workspace: bsq_requant_workspace(batch, rows, num_segments, out_fmt, gather)
 * bytes, 16-byte aligned (0 bytes for batch-mode MXFP8).
 * Errors: NULL, SHAPE, ALIGN, ENUM, WORKSPACE, LAUNCH.
 * ---------------------------------------------------------------------- */
size_t bsq_requant_workspace(int64_t batch, int64_t rows, int64_t num_segments, int out_fmt,
                             int gather);
int bsq_requant_transpose_sr(const uint8_t* codes, const uint8_t* scales, const float* outer,
                             int in_mode, int64_t batch, int64_t rows, int64_t cols,
                             int64_t in_rows, const int32_t* row_gather,
                             const int64_t* seg_offsets, int64_t num_segments, int out_fmt,
                             int rnd, uint64_t seed, uint64_t stream_id, uint8_t* out_codes,
                             uint8_t* out_scales, float* out_outer, void* ws, size_t ws_bytes,
                             bsq_stream_t stream);

/* ------------------------------------------------------------------------
 * NVFP4 x NVFP4 expert grouped GEMM, forward pass ("Block-scaled backward
 * passes": y = x_q w_q^T with 16-value blocks paired and each block sum
 * multiplied by both block scales).
 *
 * For dispatched row r of expert e (seg_offsets[e] <= r < seg_offsets[e+1]):
 *   y[r, n] = a_outer[t] * b_outer[e] * sum_k xq[t, k] * wq[e, n, k]
 * with t = a_row_index[r] (identity when NULL), xq = q * s_b and
 * wq = q * s_b (block values, each exact), accumulated in FP32; the sum is
 * multiplied by f32(a_outer * b_outer) and stored as out_dtype: BSQ_BF16
 * (round to nearest even) or BSQ_F32 (the same value before rounding).
 * a_codes [a_rows, K/2], a_scales [a_rows, K/16]; a_outer [a_rows] when
 * a_outer_per_row != 0, else [1].
 * b_codes [E, N, K/2], b_scales [E, N, K/16], b_outer [E].
 * seg_offsets device int64 [E+1]; M_total = seg_offsets[E] rows of output,
 * M_total < 2^31 - 1.
 * out [M_total, N] of out_dtype. Rows of a segment past M_total are not
 * written (malformed offsets never reach outside the buffers).
 * Constraints: K % 64 == 0, N % 256 == 0, 1 <= E <= 1024 (BSQ_E_SHAPE).
 * a_codes, b_codes and out 16-byte aligned; scale arrays 4-byte aligned.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, LAUNCH.
 * ---------------------------------------------------------------------- */
int bsq_grouped_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                           int a_outer_per_row, int64_t a_rows, const int32_t* a_row_index,
                           const uint8_t* b_codes, const uint8_t* b_scales, const float* b_outer,
                           const int64_t* seg_offsets, int64_t E, int64_t M_total, int64_t N,
                           int64_t K, void* out, int out_dtype, bsq_stream_t stream);

/* The w2 GEMM of the expert chain with the combine codec in its epilogue
 * ("Quantized communications": the RHT and S2F6 quantization run in the
 * epilogue of the w2 grouped GEMM): the same product as
 * bsq_grouped_gemm_nvfp4 (float32 sums times the two outer scales), written
 * as bsq_rht_s2f6_encode would encode its float32 output:
 *   out_codes  [M_total, N] u8 (S2F6), out_scales [M_total, N/32] u8 (UE8M0),
 *   signs      the RHT's sign mask.
 * Rows past a segment's end are not written. Arguments, limits and errors
 * otherwise as bsq_grouped_gemm_nvfp4 (out_codes 16-byte aligned). */
int bsq_grouped_gemm_nvfp4_s2f6(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                                int a_outer_per_row, int64_t a_rows, const int32_t* a_row_index,
                                const uint8_t* b_codes, const uint8_t* b_scales, const float* b_outer,
                                const int64_t* seg_offsets, int64_t E, int64_t M_total, int64_t N,
                                int64_t K, uint32_t signs, uint8_t* out_codes, uint8_t* out_scales,
                                bsq_stream_t stream);

/* ------------------------------------------------------------------------
 * MXFP8 expert grouped GEMMs of the backward pass (quantized linear layer
 * figure: DGRAD and WGRAD as MXFP8 GEMMs).
 *
 * wgrad == 0 (DGRAD, segments along M): for row r of expert e
 *   out[r, n] = sum_k A[r, k] * B[e, n, k]
 *   (M_total < 2^31 - 1)
 *   A codes [M_total, K], scales [M_total, K/32]; B codes [E, N, K], scales
 *   [E, N, K/32]; out [M_total, N]. K % 64 == 0, N % 256 == 0.
 * wgrad == 1 (WGRAD, segments along K): for expert e with padded token count
 *   Kp_e = seg length rounded up to 32,
 *   out[e, m, n] = sum_t A_e[m, t] * B_e[n, t]
 *   with A and B in the padded per-segment transposed layout written by
 *   bsq_quantize_mxfp8(transpose=1) and bsq_requant_transpose_sr (gather
 *   mode): A_e [M, Kp_e], B_e [N, Kp_e]; here M is the `M_total` argument
 *   and K is ignored. out [E, M, N]. M % 256 == 0, N % 256 == 0.
 * Values are E4M3 times the E8M0 block scale. Every product is formed
 * exactly and accumulated in FP32: each value is decoded to bf16 (subnormals
 * kept), which is exact for every E4M3 value under scale codes 3..246 (the
 * MXFP8 quantizer's codes for any block maximum up to 1.75 * 2^127). Under
 * codes 0..2 a decoded value rounds to the nearest multiple of 2^-133 (error
 * at most 2^-134 per value); under codes 247..254 a decoded magnitude of
 * 2^128 or more becomes infinite; code 255 (NaN) propagates.
 * out_dtype BSQ_BF16 (round to nearest even) or BSQ_F32.
 * Codes and out 16-byte aligned. Scales are read in aligned 4-byte words:
 * A's scale array (M_total * K / 32 bytes, not a multiple of 4 only when
 * K % 128 == 64 and M_total is odd) must stay readable up to the next 4-byte
 * boundary past its end, as any allocation of whole 4-byte words is.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, ENUM, LAUNCH.
 * ---------------------------------------------------------------------- */
/* bsq_gemm_nvfp4_inreg_scale: the NVFP4 product with the block scales
 * applied in registers instead of decoded into the operands ("Kernels for
 * low-precision training": the two ways to handle NVFP4 scales without a
 * native NVFP4 MMA), kept to measure that choice against
 * bsq_grouped_gemm_nvfp4 on the same data. Dense, one expert:
 *   out[m, n] = a_outer[m] * b_outer[0] * sum_k xq[m, k] * wq[n, k]
 * Each 16-value block pair is one FP8 MFMA over the E2M1 values (exact
 * partial sum), scaled by s_a * s_w and accumulated in FP32.
 * a_codes [M, K/2], a_scales [M, K/16], a_outer [M]; b_codes [N, K/2],
 * b_scales [N, K/16], b_outer [1]; out float32 [M, N].
 * M % 128 == 0 (M / 128 <= 65535), N % 128 == 0, K % 64 == 0; codes and out
 * 16-byte aligned, scales 4-byte aligned.
 * Errors: NULL, SHAPE, ALIGN, LAUNCH.
 * ---------------------------------------------------------------------- */
int bsq_gemm_nvfp4_inreg_scale(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                               const uint8_t* b_codes, const uint8_t* b_scales, const float* b_outer,
                               int64_t M, int64_t N, int64_t K, float* out, bsq_stream_t stream);

/* ------------------------------------------------------------------------ */
int bsq_grouped_gemm_mxfp8(int wgrad, const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* b_codes, const uint8_t* b_scales,
                           const int64_t* seg_offsets, int64_t E, int64_t M_total, int64_t N,
                           int64_t K, void* out, int out_dtype, bsq_stream_t stream);

/* ------------------------------------------------------------------------
 * Routing of tokens to expert segments ("Quantized communications": a router
 * picks experts per token and tokens are dispatched to them; on one GPU the
 * dispatch is a permutation into per-expert row segments).
 *
 * topk_ids   int32 [tokens, k], expert ids in [0, E), distinct per token.
 * row_index  int32 [tokens*k]: token of each dispatched row.
 * seg_offsets int64 [E+1].
 * pair_row   int32 [tokens*k]: dispatched row of pair t*k+j.
 * Rows of a segment are ordered by (token, slot). Deterministic.
 * ws         at least bsq_route_workspace(tokens, E) bytes.
 * Errors: NULL, SHAPE (k < 1 or > 64, E < 1 or > 1024), ALIGN (ws),
 * WORKSPACE, LAUNCH.
 * ---------------------------------------------------------------------- */
size_t bsq_route_workspace(int64_t tokens, int64_t E);
int bsq_route(const int32_t* topk_ids, int64_t tokens, int64_t k, int64_t E, int32_t* row_index,
              int64_t* seg_offsets, int32_t* pair_row, void* ws, size_t ws_bytes,
              bsq_stream_t stream);

/* bsq_route_noalloc: bsq_route for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments and outputs as bsq_route minus the
 * workspace: the per-chunk counts live in a library-owned device array of
 * BSQ_ROUTE_NOALLOC_MAX_BYTES per GPU (held until the process ends). Makes
 * no hipMalloc/hipFree call. Every slot it reads is written earlier in the
 * same call, so nothing carries over between calls; all calls on one GPU
 * share the array, so calls that overlap in time on one GPU (other streams,
 * other host threads) race and must be serialised by the caller.
 * Errors: as bsq_route; WORKSPACE when bsq_route_workspace(tokens, E)
 * exceeds BSQ_ROUTE_NOALLOC_MAX_BYTES (e.g. E = 64 allows 1,048,576 tokens).
 * ---------------------------------------------------------------------- */
#define BSQ_ROUTE_NOALLOC_MAX_BYTES ((size_t)1 << 20)
int bsq_route_noalloc(const int32_t* topk_ids, int64_t tokens, int64_t k, int64_t E,
                      int32_t* row_index, int64_t* seg_offsets, int32_t* pair_row,
                      bsq_stream_t stream);

/* ------------------------------------------------------------------------
 * Combine codec ("Quantized communications": before the combine exchange an
 * expert output row is rotated by a 32-dimensional random Hadamard transform
 * and quantized to block-scaled S2F6, one UE8M0 scale per 32 values, 8.25
 * bits per value; the receiver dequantizes and aggregates a token's copies
 * and inverts the transform).
 *
 * Transform: z = H D x / sqrt(32) per block of 32 along a row; D = diag of
 * signs (bit i of `signs` set: element i negated), H the Sylvester Hadamard
 * matrix (H_2n = [[H, H], [H, -H]]); float32 butterfly of spans 1, 2, 4, 8, 16
 * ((a, b) -> (a + b, a - b)) and one multiply by f32(1/sqrt(32)).
 * S2F6: values k/64, k in [-128, 127] (two's-complement byte). Scale: the
 * smallest 2^e with max|z| <= (127/64) 2^e, e in [-127, 127] (-127 for a zero
 * block), byte e + 127; k = round-half-even(z 2^(6-e)) saturated.
 *
 * bsq_rht_s2f6_encode
 *   x       [rows, cols] of `dtype` (F32 or BF16), cols % 32 == 0.
 *   codes   [rows, cols] u8; scales [rows, cols/32] u8.
 *   Alignment: x and codes 16 bytes. Errors: NULL, SHAPE, ALIGN, DTYPE, LAUNCH.
 * bsq_rht_s2f6_combine
 *   codes, scales  as written by the encoder for `rows` rows of `cols`.
 *   pair_row int32 [tokens*k]: row of copy j of token t at t*k + j (as
 *            bsq_route writes it); indices outside [0, rows) are clamped.
 *   out      [tokens, cols] of out_dtype (F32, or BF16 rounded to nearest
 *            even): D H / sqrt(32) applied to the float32 sum, in slot order j,
 *            of the dequantized blocks k/64 * 2^e (exact) of the token's rows.
 *   1 <= k <= 64. Alignment: codes and out 16 bytes, pair_row 4 bytes.
 *   Errors: NULL, SHAPE, ALIGN, DTYPE, LAUNCH.
 * NaN and infinite inputs give unspecified codes (memory-safe).
 * ---------------------------------------------------------------------- */
int bsq_rht_s2f6_encode(const void* x, int dtype, int64_t rows, int64_t cols, uint32_t signs,
                        uint8_t* codes, uint8_t* scales, bsq_stream_t stream);
int bsq_rht_s2f6_combine(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                         const int32_t* pair_row, int64_t tokens, int64_t k, uint32_t signs, void* out,
                         int out_dtype, bsq_stream_t stream);

/* ------------------------------------------------------------------------
 * Test support: dequantization and the raw random bits.
 * bsq_dequantize_nvfp4: out[b, r, c] = f32(f32(q * s_b) * s_t) (FP32),
 *   outer per mode as in bsq_requant_transpose_sr's batch mode.
 * bsq_dequantize_mxfp8: out[r, c] = q * 2^(s-127) (FP32), cols % 32 == 0.
 * bsq_rng_bits16: out[i] = the 16 stochastic-rounding bits of output index
 *   first + i (Philox4x32-10; key = seed, counter = (idx>>3, stream_id), half
 *   idx&1 of word (idx>>1)&3), as uint16.
 * ---------------------------------------------------------------------- */
int bsq_dequantize_nvfp4(const uint8_t* codes, const uint8_t* scales, const float* outer,
                         int mode, int64_t batch, int64_t rows, int64_t cols, float* out,
                         bsq_stream_t stream);
int bsq_dequantize_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                         float* out, bsq_stream_t stream);
int bsq_rng_bits16(uint64_t seed, uint64_t stream_id, uint64_t first, int64_t n, uint16_t* out,
                   bsq_stream_t stream);

/* ------------------------------------------------------------------------
 * Measurement support: per-instruction MFMA throughput ("Kernels for
 * low-precision training": the matrix instructions set the GEMMs' rate).
 * Launches `workgroups` workgroups of 256 threads; every wave runs `iters`
 * rounds of four independent accumulator chains of one MFMA instruction on
 * operands held in registers (nothing but MFMAs in the loop):
 *   kind 0 v_mfma_f32_32x32x16_f16, 1 ..._bf16, 2 ..._fp8_fp8 (2*32*32*16
 *   FLOP each); 3 v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3, 4 the same on
 *   E2M1 (2*32*32*64 FLOP each; E8M0 scales of one).
 *   data 0 random finite operands, 1 zeros, 2 values with at most two
 *   significant bits (the GEMMs run at the chip's power limit, so the rate
 *   depends on how many operand bits switch).
 * Total FLOP = workgroups * 4 waves * iters * 4 * FLOP per instruction; the
 * caller times the launch. out: workgroups * 256 floats (one accumulator
 * element per thread, so no MFMA is dead code; the values are not meaningful).
 * 1 <= iters <= 2^24, 1 <= workgroups <= 65535. Errors: NULL, SHAPE, ALIGN,
 * ENUM, LAUNCH.
 * ---------------------------------------------------------------------- */
int bsq_mfma_rate_probe(int kind, int data, int64_t iters, int64_t workgroups, float* out, bsq_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BSQ_H */
