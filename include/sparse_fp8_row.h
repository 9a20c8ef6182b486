/*
 * sparse_fp8_row.h -- C ABI of the MI355X (gfx950) row-wise-scaled FP8 linear
 * layer with a 2:4 semi-structured sparse weight.
 *
 * The operation (pytorch/ao PR #1671, "Add CUTLASS-based row-wise scaled
 * sparse FP8 kernel", ready-for-review comment, item 1: a converter of FP8
 * data to a 2:4 sparse format, and a row-wise scaled linear operator for a
 * sparse FP8 weight and an FP8 activation; item 4: the activation is quantized
 * dynamically) is, with torch `linear` conventions (weight [N, K]):
 *
 *     out[m, n] = bf16( xs[m] * ws[n] * sum_k xq[m, k] * wq[n, k]  (+ bias[n]) )
 *
 * where xq/xs is the FP8 activation with one binary32 scale per row, wq/ws the
 * FP8 weight with one binary32 scale per output row, and wq keeps at most two
 * non-zeros in every group of four consecutive k.  Either operand may be OCP
 * e4m3 ("fn": max 448, no infinities) or e5m2 (max 57344); the four dtype
 * pairs are the four instantiations the pages list (pytorch/ao issue #3516,
 * "Making torchao ABI compatible ...", file table).  A plain C ABI, free of
 * any framework's C++ types, is the point that issue makes.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers to contiguous row-major data and
 *    must be 16-byte aligned.  The caller owns all memory; the library never
 *    allocates, frees or synchronizes.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it and the call returns without waiting.  The library keeps no state
 *    between calls and may be called from several host threads at once.
 *  - Arguments are validated on the host before anything is launched.  On an
 *    error nothing is launched and no output is touched.  Device faults (bad
 *    pointers that pass validation) surface at the caller's next
 *    synchronization, as usual in HIP.
 *  - Outputs must not alias inputs.
 *  - Inputs must be finite.  NaN or infinite inputs give unspecified results.
 */
#ifndef SPARSE_FP8_ROW_H
#define SPARSE_FP8_ROW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* FP8 formats (OCP 8-bit floating point). */
typedef enum { SFR_E4M3 = 0, SFR_E5M2 = 1 } sfr_fp8_t;

/* Output formats of the linear layer.  SFR_OUT_F32 writes the binary32 value
 * before the final bf16 rounding (for accuracy checks). */
typedef enum { SFR_OUT_BF16 = 0, SFR_OUT_F32 = 1 } sfr_out_t;

/* Scale granularity of one operand of sparse_fp8_scaled_linear: one binary32
 * scale per row (per token for the activation, per output row for the
 * weight), or one for the whole operand. */
typedef enum { SFR_SCALE_ROW = 0, SFR_SCALE_TENSOR = 1 } sfr_scale_t;

typedef enum {
    SFR_OK = 0,
    SFR_ERR_NULL = 1,   /* a required pointer is NULL                         */
    SFR_ERR_SHAPE = 2,  /* a size is negative, too large or not a multiple    */
    SFR_ERR_ALIGN = 3,  /* a pointer is not 16-byte aligned                   */
    SFR_ERR_DTYPE = 4,  /* an enum argument is out of range                   */
    SFR_ERR_LAUNCH = 5  /* the HIP runtime rejected a kernel launch           */
} sfr_status;

/* Version of the compressed-weight layout described at compress_2to4_fp8. */
#define SFR_FORMAT_VERSION 1

/* Largest accepted row count / column count / K of any entry point. */
#define SFR_MAX_DIM ((int64_t)1 << 30)

/*
 * quantize_rowwise_fp8 -- dynamic row-wise FP8 quantization.
 * Source: PR #1671 (row-wise scaled FP8 activation, quantized dynamically;
 * FP16->FP8 quantization must not produce NaN) and pytorch/ao PR #1455
 * ("[float8nocompile] ... atomic_max-based algo ...", review thread: the split
 * reduction is worth keeping because it is deterministic).
 *
 * For every row r of x (bf16 bits, [rows, cols]):
 *     amax     = max_k |x[r, k]|                      (exact)
 *     scale[r] = fl32(amax / fmax)                    (IEEE binary32 division;
 *                                                      fmax 448 or 57344)
 *     q[r, k]  = sat_rne_fp8(fl32(x[r, k] / scale[r]))
 * sat_rne_fp8 rounds to nearest, ties to even, keeps the sign of zero, and
 * clamps magnitudes above fmax to fmax.  A row whose amax is 0 gets
 * scale 0 and codes 0x00 / 0x80 that keep each zero's sign.  The result is
 * deterministic and exact: the same bytes on every run and every launch shape.
 *
 *   x      [rows, cols] bf16 bits, device, read.
 *   dt     format of q.
 *   q      [rows, cols] FP8 bytes, device, written.
 *   scale  [rows] binary32, device, written.
 * Sizes: 0 <= rows <= SFR_MAX_DIM, 0 < cols <= SFR_MAX_DIM, cols % 8 == 0.
 * rows == 0 is a no-op; cols == 0 is rejected (SFR_ERR_SHAPE) because a row
 * without elements has no amax.
 */
sfr_status quantize_rowwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, sfr_fp8_t dt,
                                uint8_t* q, float* scale, void* stream);

/*
 * quantize_tensorwise_fp8 -- dynamic tensor-wise FP8 quantization: the
 * quantization of quantize_rowwise_fp8 with one scale for the whole tensor
 * (as if the tensor were a single row of rows*cols elements).  Source:
 * pytorch/ao PR #1455 ("[float8nocompile] Add alternate Triton kernels for
 * FP8 conversion which use atomic_max-based algo instead of reduction-based
 * algo", review thread): tensor-wise FP8 conversion whose global amax must
 * stay a deterministic reduction.  Here it is computed in two launches --
 * per-block maxima written to fixed workspace slots, then every block of the
 * cast kernel reduces all slots itself -- with no atomics; the amax is an
 * exact integer maximum, so the result is bit-exact and deterministic.
 *
 *     amax     = max_{r,k} |x[r, k]|                   (exact)
 *     scale[0] = fl32(amax / fmax)                     (IEEE binary32 division)
 *     q[r, k]  = sat_rne_fp8(fl32(x[r, k] / scale[0]))
 * An all-zero tensor gets scale 0 and sign-keeping zero codes.
 *
 *   x          [rows, cols] bf16 bits, device, read.
 *   dt         format of q.
 *   q          [rows, cols] FP8 bytes, device, written.
 *   scale      [1] binary32, device, written.
 *   workspace  device scratch of at least workspace_bytes =
 *              sfr_quantize_tensorwise_workspace_bytes(rows, cols) bytes,
 *              owned by the caller, overwritten; calls that may run at the
 *              same time need distinct workspaces.
 * Sizes as quantize_rowwise_fp8.  rows == 0 is a no-op; a workspace smaller
 * than required is SFR_ERR_SHAPE.
 */
sfr_status quantize_tensorwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, sfr_fp8_t dt,
                                   uint8_t* q, float* scale, void* workspace, int64_t workspace_bytes,
                                   void* stream);

/* Workspace bytes quantize_tensorwise_fp8 needs for a [rows, cols] tensor
 * (at most 4 KB); 0 for sizes it rejects. */
int64_t sfr_quantize_tensorwise_workspace_bytes(int64_t rows, int64_t cols);

/*
 * quantize_tensorwise_fp8_noalloc -- quantize_tensorwise_fp8 for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): no workspace argument, and the
 * call allocates nothing.  The workspace is the library's own 4 KB device
 * array, one copy per GPU, held until the process ends; its address is
 * looked up on the first call on each device.  Results are bit-identical to
 * quantize_tensorwise_fp8's.
 *
 * Every call on one GPU uses that GPU's array, which keeps the last call's
 * contents (each call writes every slot it reads before reading it).  Calls
 * that may overlap on one GPU (different streams, or host threads) race on
 * the array and must be serialized by the caller.
 *
 * Arguments, sizes and errors as quantize_tensorwise_fp8 without the
 * workspace; a size whose workspace would exceed the array is SFR_ERR_SHAPE
 * (no accepted size does), and a failed lookup of the array SFR_ERR_LAUNCH.
 */
sfr_status quantize_tensorwise_fp8_noalloc(const uint16_t* x, int64_t rows, int64_t cols, sfr_fp8_t dt,
                                           uint8_t* q, float* scale, void* stream);

/*
 * compress_2to4_fp8 -- 2:4 semi-structured compression of an FP8 matrix.
 * Source: PR #1671 (converter to the 2:4 sparse format; testing found that
 * the compressor must treat -0.0 as zero, the issue the PR works around in
 * `from_plain()` and fixes upstream).
 *
 * For every row n and every group g of four consecutive k (k = 4g .. 4g+3)
 * of w ([n, k] FP8 bytes), the two entries of largest magnitude are kept;
 * ties go to the lower index and +0 / -0 have equal (zero) magnitude.  With
 * i0 < i1 the kept positions:
 *     values[n, 2g]   = w[n, 4g + i0]     values[n, 2g+1] = w[n, 4g + i1]
 *     (a kept -0.0, byte 0x80, is stored as 0x00)
 *     meta[n, g / 2]  bits 4*(g%2) .. 4*(g%2)+3  =  i0 | (i1 << 2)
 * so a little-endian 32-bit word of meta holds the nibbles of eight
 * consecutive groups, even group in the low nibble (layout version
 * SFR_FORMAT_VERSION).  Magnitude order is the unsigned order of the low
 * seven bits, identical for e4m3 and e5m2; `dt` is validated and otherwise
 * does not change the result.  Output is bit-exact and deterministic.
 *
 *   w      [n, k] FP8 bytes, device, read.
 *   values [n, k/2] bytes, device, written.
 *   meta   [n, k/8] bytes, device, written.
 * Sizes: 0 <= n <= SFR_MAX_DIM, 0 < k <= SFR_MAX_DIM, k % 128 == 0.
 * n == 0 is a no-op.
 */
sfr_status compress_2to4_fp8(const uint8_t* w, int64_t n, int64_t k, sfr_fp8_t dt,
                             uint8_t* values, uint8_t* meta, void* stream);

/*
 * prune_2to4_bf16 -- 2:4 magnitude pruning of a bf16 matrix, the weight's
 * first preparation step (before FP8 quantization and compress_2to4_fp8).
 * Source: PR #1671 (the weight is 2:4 semi-structured sparse; zeros of
 * either sign count as zero, the -0.0 issue that PR fixes in the converter).
 *
 * For every row and every group of four consecutive k of w ([n, k] bf16
 * bits), the two entries of largest magnitude keep their bits and the other
 * two become +0.0 (0x0000); ties go to the lower index and +0.0 / -0.0 have
 * equal (zero) magnitude.  A row's largest magnitude always survives, so its
 * row-wise FP8 scale is the same before and after pruning.  Finite inputs
 * only.  Output is bit-exact and deterministic.
 *
 *   w    [n, k] bf16 bits, device, read.
 *   out  [n, k] bf16 bits, device, written; may be w (in place).
 * Sizes: 0 <= n <= SFR_MAX_DIM, 0 < k <= SFR_MAX_DIM, k % 8 == 0.
 * n == 0 is a no-op.
 */
sfr_status prune_2to4_bf16(const uint16_t* w, int64_t n, int64_t k, uint16_t* out, void* stream);

/*
 * sparse_fp8_rowwise_linear -- the row-wise scaled linear layer with a 2:4
 * sparse FP8 weight.  Source: PR #1671 (row-wise scaled linear operator for a
 * sparse FP8 weight and an FP8 activation, one instantiation per dtype pair,
 * issue #3516's file table).
 *
 *     acc[m, n] = sum_k xq[m, k] * wq[n, k]          (binary32-grade accumulation
 *                                                    of exact products, any order)
 *     y[m, n]   = acc[m, n] * (xs[m] * ws[n]) (+ bias[n])   (binary32)
 *     out[m, n] = bf16_rne(y[m, n])   or   y[m, n] with SFR_OUT_F32
 * wq is the weight that (values, meta) encode in the compress_2to4_fp8
 * layout.  Any accumulation order is a correct result; the library's order is
 * fixed, so repeated calls give identical bits.
 *
 *   xq     [m, k] FP8 bytes (format x_dt), device, read.
 *   xs     [m] binary32, device, read.
 *   values [n, k/2], meta [n, k/8]: compressed weight (format w_dt), device, read.
 *   ws     [n] binary32, device, read.
 *   bias   [n] bf16 bits, device, read; may be NULL (no bias).
 *   out    [m, n] bf16 bits (SFR_OUT_BF16) or binary32 (SFR_OUT_F32), device, written.
 * Sizes: 0 <= m <= SFR_MAX_DIM, 0 <= n <= SFR_MAX_DIM, n % 16 == 0,
 * 0 < k <= SFR_MAX_DIM, k % 128 == 0.  m == 0 or n == 0 is a no-op.
 */
sfr_status sparse_fp8_rowwise_linear(const uint8_t* xq, sfr_fp8_t x_dt, const float* xs,
                                     int64_t m, int64_t k,
                                     const uint8_t* values, const uint8_t* meta, sfr_fp8_t w_dt,
                                     const float* ws, int64_t n, const uint16_t* bias,
                                     void* out, sfr_out_t out_dt, void* stream);

/*
 * sparse_fp8_scaled_linear -- sparse_fp8_rowwise_linear with the scale
 * granularity of each operand chosen: xs_kind / ws_kind SFR_SCALE_ROW reads
 * xs[m] / ws[n] as above, SFR_SCALE_TENSOR reads the single xs[0] / ws[0] for
 * every row (the tensor-wise scaling of quantize_tensorwise_fp8).  Everything
 * else -- arguments, sizes, accumulation, epilogue, errors -- is as
 * sparse_fp8_rowwise_linear, which is this call with both kinds
 * SFR_SCALE_ROW.  An unknown kind is SFR_ERR_DTYPE.
 */
sfr_status sparse_fp8_scaled_linear(const uint8_t* xq, sfr_fp8_t x_dt, const float* xs,
                                    sfr_scale_t xs_kind, int64_t m, int64_t k,
                                    const uint8_t* values, const uint8_t* meta, sfr_fp8_t w_dt,
                                    const float* ws, sfr_scale_t ws_kind, int64_t n,
                                    const uint16_t* bias, void* out, sfr_out_t out_dt,
                                    void* stream);

/*
 * Accumulation.  The products xq * wq are exact in binary32 (at most 8
 * significant bits each).  By default the library widens the FP8 codes
 * exactly to bf16 in registers and multiplies them on gfx950's 16-bit sparse
 * matrix instruction, which adds each product 24 bits below the largest term
 * of the instruction (the running sum included) and truncates toward zero:
 * a binary32-grade sum, whose error is that of a binary32 sum with
 * truncation in place of rounding.  An algorithm id with
 * SFR_ALGO_ACC_F8 set (see below) runs the FP8 sparse matrix instruction
 * instead, at twice the instruction rate; that instruction adds the 64
 * products of one 128-k step 13 bits below the largest of them, so a product
 * under 2^-13 of the step's largest is dropped.  On dot products that cancel
 * heavily next to large products (outlier channels, short K) its error can
 * exceed the bound above.
 */

/*
 * sparse_fp8_rowwise_linear_dynamic -- the layer from the bf16 activation:
 * quantize_rowwise_fp8 of x into (xq, xs), then sparse_fp8_scaled_linear with
 * row activation scales.  Source: PR #1671, item 4 (the activation is
 * quantized dynamically, per call).  xq and xs receive exactly the bytes
 * quantize_rowwise_fp8 writes; out is as sparse_fp8_scaled_linear.
 *
 * For 1 to 4 activation rows with k a multiple of 1024, both steps run in
 * ONE launch where that is faster: every workgroup quantizes the rows itself
 * (no workgroup waits for another), so the redundant work grows with rows x
 * workgroups.  One launch is taken for 1 or 2 rows with k up to 4096, or up
 * to 16384 while n / 16 does not exceed the device's CU count; for 3 or 4
 * rows with k up to 4096 and n / 16 at most the CU count.  Other shapes
 * take two launches (quantization, then the linear layer).  Both paths write
 * the same bytes.
 *
 *   x      [m, k] bf16 bits, device, read.
 *   xq     [m, k] FP8 bytes (format x_dt), device, written.
 *   xs     [m] binary32, device, written.
 * Other arguments, sizes and errors as sparse_fp8_scaled_linear (ws_kind
 * selects row or tensor weight scales).
 */
sfr_status sparse_fp8_rowwise_linear_dynamic(const uint16_t* x, sfr_fp8_t x_dt, int64_t m, int64_t k,
                                             const uint8_t* values, const uint8_t* meta, sfr_fp8_t w_dt,
                                             const float* ws, sfr_scale_t ws_kind, int64_t n,
                                             const uint16_t* bias, void* out, sfr_out_t out_dt,
                                             uint8_t* xq, float* xs, void* stream);

/*
 * sparse_fp8_rowwise_linear_dynamic_algo -- sparse_fp8_rowwise_linear_dynamic
 * with the linear layer's algorithm id given (SFR_ALGO_DEFAULT = the built-in
 * choice; ids as for sparse_fp8_scaled_linear_algo below).  The single-launch
 * path runs when the id's kernel configuration is the built-in one for the
 * shape; the accumulation follows the id.  Errors as
 * sparse_fp8_scaled_linear_algo.
 */
sfr_status sparse_fp8_rowwise_linear_dynamic_algo(const uint16_t* x, sfr_fp8_t x_dt, int64_t m, int64_t k,
                                                  const uint8_t* values, const uint8_t* meta, sfr_fp8_t w_dt,
                                                  const float* ws, sfr_scale_t ws_kind, int64_t n,
                                                  const uint16_t* bias, void* out, sfr_out_t out_dt,
                                                  uint8_t* xq, float* xs, int algo, void* stream);

/*
 * Kernel configurations ("algorithms") of the linear layer, and the choice
 * among them.  Source: pytorch/ao PR #4432 ("Add algorithm search to FP8
 * sparse linear benchmark": the best kernel configuration depends on the
 * shape, so it is searched per shape) and PR #1671 (remaining tasks: a
 * meaningful config selection).  Every algorithm computes the same function
 * (same result rules; the order of the binary32 sum differs between them).
 *
 * An algorithm id is a kernel configuration (low 8 bits) optionally or-ed
 * with SFR_ALGO_ACC_F8 (FP8 matrix-instruction accumulation, see
 * "Accumulation" above); without the flag the accumulation is binary32-grade.
 *
 *   sfr_linear_algo_count()      number of kernel configurations (ids
 *                                0 .. count-1, each with or without the flag).
 *   sfr_linear_algo_valid(a)     1 if a names an algorithm, else 0.
 *   sfr_linear_algo_name(a)      static name (configurations with the flag
 *                                end in "+f8acc"), NULL for an unknown id.
 *   sfr_linear_algo_supported(a, m, n, k)
 *                                1 if algorithm a can run the shape, else 0.
 *   sfr_linear_default_algo(m, n, k)
 *                                the library's built-in choice for the shape
 *                                on the current device (it counts rounds of
 *                                tiles over the device's compute units, so it
 *                                can differ between GPUs; 256 units are
 *                                assumed when no device is present).
 *   sparse_fp8_scaled_linear_algo(..., algo, stream)
 *                                sparse_fp8_scaled_linear with the given
 *                                algorithm; SFR_ALGO_DEFAULT (-1) = built-in
 *                                choice.  An unknown id is SFR_ERR_DTYPE; an
 *                                algorithm that cannot run the shape is
 *                                SFR_ERR_SHAPE.
 * Configurations: 0 decode_lds (m <= 64, k % 1024 == 0), 1 decode_reg
 * (m <= 16), 2 tiled_64x64, 3 tiled_128x128, 4 tiled_256x256,
 * 5 wide_256x256 (k >= 512, only with SFR_ALGO_ACC_F8), 6 decode_lds_32
 * (m <= 64, k % 1024 == 0, n % 32 == 0), 7 tiled_256x128 (tiles of 256
 * output columns n by 128 rows m).
 */
#define SFR_ALGO_DEFAULT (-1)
#define SFR_ALGO_ACC_F8 0x100
int sfr_linear_algo_count(void);
int sfr_linear_algo_valid(int algo);
const char* sfr_linear_algo_name(int algo);
int sfr_linear_algo_supported(int algo, int64_t m, int64_t n, int64_t k);
int sfr_linear_default_algo(int64_t m, int64_t n, int64_t k);
sfr_status sparse_fp8_scaled_linear_algo(const uint8_t* xq, sfr_fp8_t x_dt, const float* xs,
                                         sfr_scale_t xs_kind, int64_t m, int64_t k,
                                         const uint8_t* values, const uint8_t* meta, sfr_fp8_t w_dt,
                                         const float* ws, sfr_scale_t ws_kind, int64_t n,
                                         const uint16_t* bias, void* out, sfr_out_t out_dt, int algo,
                                         void* stream);

/*
 * Block-sparse (BSR) bf16 weight and its linear layer.
 * Source: pytorch/ao PR #1734 ("promote blocksparse from prototype, make it
 * faster"): the weight is stored in blocks of 64 x 64, most of them zero
 * (its measurements use sparsity level 0.9), and multiplied by a dense
 * activation whose row count is padded to 16 for decode.  The page names no
 * number format; here weight, activation and output are bf16, the sum is
 * binary32 (every bf16 product is exact in it), the result rounded once to
 * bf16 (nearest, ties to even) or returned in binary32.
 *
 * Layout (compressed-sparse-row over blocks, as torch's BSR tensors):
 *   crow   int32 [n/64 + 1]: crow[0] = 0, crow[i+1] - crow[i] = kept blocks of
 *          block row i (rows 64 i .. 64 i + 63); nnz = crow[n/64].
 *   col    int32 [nnz]: block column of each kept block, ascending within a
 *          block row.
 *   values bf16 bits [nnz][64][64]: each kept block, row-major.
 * A block is kept when any element is non-zero by value (+0.0 and -0.0 are
 * zero; NaN, infinities and subnormals are non-zero).
 *
 * bsr_count_bf16(w, n, k, crow, stream): two launches write crow for the
 *   dense bf16 w [n, k] (row-major, 16-byte aligned).  The caller reads
 *   crow[n/64] (nnz) to size col and values.
 * bsr_fill_bf16(w, n, k, crow, col, values, stream): writes col and values
 *   for the crow that bsr_count_bf16 wrote for the same w.  col and values
 *   may be NULL only when nnz = 0.
 * bsr_linear_bf16(x, m, k, crow, col, values, n, bias, out, out_dt, stream):
 *   out[m, n] = sum_k x[i, k] W[j, k] (+ bias[j]) for bf16 x [m, k]
 *   (row-major), the BSR weight W [n, k] and optional bf16 bias [n]; out is
 *   bf16 or binary32 [m, n], row-major.  Deterministic (fixed summation
 *   order).  Every block column index is clamped to the matrix, but crow and
 *   the values array must be the ones bsr_count_bf16 / bsr_fill_bf16 wrote
 *   (they are read as given).
 * Sizes: 0 <= n, m <= SFR_MAX_DIM; 0 < k <= SFR_MAX_DIM; n % 64 == 0,
 * k % 64 == 0.  Alignment: w, x, values, bias, out 16 bytes; crow, col 4.
 * Errors: SFR_ERR_SHAPE, SFR_ERR_NULL, SFR_ERR_ALIGN, SFR_ERR_DTYPE (out_dt),
 * SFR_ERR_LAUNCH.  All pointers are device memory owned by the caller; the
 * calls are asynchronous on `stream` (NULL = the default stream).
 */
#define SFR_BSR_BLOCK 64
sfr_status bsr_count_bf16(const uint16_t* w, int64_t n, int64_t k, int32_t* crow, void* stream);
sfr_status bsr_fill_bf16(const uint16_t* w, int64_t n, int64_t k, const int32_t* crow, int32_t* col,
                         uint16_t* values, void* stream);
sfr_status bsr_linear_bf16(const uint16_t* x, int64_t m, int64_t k, const int32_t* crow, const int32_t* col,
                           const uint16_t* values, int64_t n, const uint16_t* bias, void* out, sfr_out_t out_dt,
                           void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* sfr_status_string(sfr_status s);

/* The compressed-weight layout version this library reads and writes. */
int sfr_format_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_FP8_ROW_H */
