/*
 * fp8dsl.h -- C ABI of the delayed-scaling FP8 linear library for AMD MI355X
 * (gfx950 / CDNA4).
 *
 * The library implements the data-parallel hot path of an FP8 linear layer
 * trained with delayed scaling:
 *
 *   fp8_cast_transpose_amax  scaled, saturating cast of a bf16/fp32 tensor to
 *                            OCP E4M3 or E5M2, writing the row-major codes, the
 *                            cached transpose, the per-tensor amax and the
 *                            scale-inverse snapshot in one pass;
 *   fp8_scale_update         the amax-history "max" recipe for every scaled
 *                            tensor of a model in one launch;
 *   fp8_linear_fwd           Y  = X W^T (+ bias)  E4M3 x E4M3 -> bf16
 *   fp8_linear_dgrad         dX = dY W            E5M2 x E4M3 -> bf16
 *   fp8_linear_wgrad         dW = dY^T X          E5M2 x E4M3 -> fp32 / bf16
 *
 * and around it: several casts in one launch (fp8_cast_transpose_amax_group),
 * the gradient cast with the bias gradient fused
 * (fp8_cast_transpose_amax_dbias, also as a no-allocation entry point), the
 * toy block's elementwise producers fused into the cast and the modulation's
 * gradient (fp8_produce_cast_transpose_amax, fp8_produce_modulate_backward),
 * dynamic scaling as the comparator (fp8_cast_transpose_dynamic), the
 * forward with FP8 output and output amax (fp8_linear_fwd_fp8out), the three
 * products split over K through a caller workspace for shapes that alone
 * leave compute units idle (fp8_linear_{fwd,dgrad,wgrad}_ws,
 * fp8_gemm_workspace_bytes), the cast with cached source loads, and a device
 * copy that serves as the bandwidth yardstick (fp8_reference_copy).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer to tensor data is a DEVICE pointer (memory the caller got
 *    from hipMalloc or from a framework allocator on the current device).
 *    The fp8_tensor_t descriptors themselves live in HOST memory and are read
 *    during the call only.
 *  - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *    the default stream).  No entry point synchronises, allocates, frees, or
 *    reads device memory from the host, so every call can be captured in a
 *    HIP graph.
 *  - The caller owns every buffer.  The library keeps no state between calls
 *    beyond per-device caches of immutable device facts (compute-unit count,
 *    kernel attributes set once), filled on first use and safe to fill from
 *    several threads at once, and the per-device scratch array of
 *    fp8_cast_transpose_amax_dbias_noalloc (described there).
 *  - Return value: FP8_OK (0) or a negative fp8_status_t.  On an argument
 *    error nothing has been enqueued.  The kernels are built for gfx950 only:
 *    on any other device the runtime rejects the launch and the call returns
 *    FP8_ERR_DEVICE.  Faults inside a kernel surface later, as HIP reports
 *    them, on the stream.
 *  - Layouts are row-major with unit stride in the last dimension.
 *  - FP8 codes are OCP float8_e4m3fn / float8_e5m2 bytes.
 */
#ifndef FP8DSL_H
#define FP8DSL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8DSL_ABI_VERSION 11

/* A hipStream_t, passed as an opaque pointer so that this header needs no
 * HIP include. */
typedef void *fp8_stream_t;

typedef enum {
    FP8_OK = 0,
    FP8_ERR_NULL = -1,      /* a required pointer is NULL                       */
    FP8_ERR_SHAPE = -2,     /* negative size, or a size rule below is broken    */
    FP8_ERR_ALIGN = -3,     /* a tensor pointer is not 16-byte aligned          */
    FP8_ERR_FORMAT = -4,    /* an FP8 format this entry point does not accept   */
    FP8_ERR_ARG = -5,       /* another argument out of range (dtype, algo, ...) */
    FP8_ERR_LAUNCH = -6,    /* the HIP runtime rejected a kernel launch         */
    FP8_ERR_DEVICE = -7,    /* no gfx950 code object for the current device     */
    FP8_ERR_SCRATCH = -8    /* more scratch than a no-allocation call holds     */
} fp8_status_t;

/* OCP 8-bit float formats ("Accelerating PyTorch Training Workloads with FP8
 * -- Part 2", PyTorch-native FP8 data types: float8_e4m3fn with 3 mantissa
 * bits, max 448; float8_e5m2 with 2 mantissa bits, max 57344).  Under the
 * HYBRID recipe of "CPU Overhead of te.Linear FP8 Layers" forward tensors use
 * E4M3 and gradients E5M2. */
typedef enum { FP8_E4M3 = 0, FP8_E5M2 = 1 } fp8_format_t;

/* Element type of a cast source or of a GEMM output. */
typedef enum { FP8_DTYPE_BF16 = 0, FP8_DTYPE_FP32 = 1 } fp8_dtype_t;

/* Amax-history reduction; "max" is the only one the recipe on the pages uses. */
typedef enum { FP8_AMAX_ALGO_MAX = 0 } fp8_amax_algo_t;

/* Elementwise producer fused in front of a cast (fp8_produce_cast_transpose_amax). */
typedef enum {
    FP8_PRODUCE_MODULATE = 1,
    FP8_PRODUCE_ADD = 2,
    FP8_PRODUCE_ADD2 = 3,
    FP8_PRODUCE_MODULATE_FINITE = 4
} fp8_produce_op_t;

/*
 * An FP8 tensor: codes, optional cached transpose and the scale-inverse that
 * was in force when the codes were written.  This is the plain-memory form of
 * the Float8Tensor of "[PyTorch] Refactor FP8 workspaces in linear modules":
 * it holds a private copy of the FP8 scale-inverse that later scale updates
 * do not touch (first motivation of that change) and a transpose cache filled
 * by the cast rather than lazily by a separate transpose kernel.
 */
typedef struct fp8_tensor {
    uint8_t *data;       /* [rows, cols] codes, or NULL                        */
    uint8_t *data_t;     /* [cols, rows] codes (transpose of data), or NULL    */
    float *scale_inv;    /* 1 float: 1/scale at cast time                      */
    int32_t fmt;         /* fp8_format_t                                       */
    int32_t reserved;    /* must be 0                                          */
    int64_t rows;
    int64_t cols;
} fp8_tensor_t;

/*
 * fp8_scale_update -- delayed-scaling update of T scaled tensors in one launch.
 *
 * Defined by the DelayedScaling recipe (amax_history_len = 16,
 * amax_compute_algo = "max") in "CPU Overhead of te.Linear FP8 Layers", by the
 * scale update that "[PyTorch] Refactor FP8 workspaces in linear modules" runs
 * for every FP8 tensor each forward pass, and by the single packed amax
 * tensor that "support delayed scaling of weight in float8 all-gather" syncs
 * once per step.  The pages do not print the scale formula; this library uses
 * the conventional one.  For every t in [0, T):
 *
 *   amax_history[t, 1:H] = amax_history[t, 0:H-1]    (roll by one)
 *   amax_history[t, 0]   = amax_cur[t]
 *   m = max_i |amax_history[t, i]|   (ordered by the sign-cleared fp32 pattern)
 *   if m is finite and m > 0:
 *       s = fp8_max(fmt[t]) / ldexp(m, margin)         (fp32, correctly rounded)
 *       if s is finite and s > 0: scale[t] = s          (else scale is kept)
 *   scale_inv[t] = 1 / scale[t]                        (fp32, correctly rounded)
 *   amax_cur[t]  = 0
 *
 * amax_history [T, H] fp32 (in/out), amax_cur [T] fp32 (in/out), scale [T]
 * fp32 (in/out), scale_inv [T] fp32 (out), fmt [T] uint8 (fp8_format_t).
 * Constraints: T >= 0 (T == 0 is a no-op), 1 <= H <= 1024, -126 <= margin <= 126,
 * algo == FP8_AMAX_ALGO_MAX.  An fmt entry that is not a valid format leaves
 * that record unchanged (the host cannot read device memory to reject it).
 * Errors: FP8_ERR_NULL, FP8_ERR_ARG, FP8_ERR_LAUNCH.
 */
int fp8_scale_update(float *amax_history, float *amax_cur, float *scale, float *scale_inv,
                     const uint8_t *fmt, int32_t T, int32_t H, int32_t margin, int32_t algo,
                     fp8_stream_t stream);

/*
 * fp8_cast_transpose_amax -- one HBM pass over a bf16/fp32 tensor.
 *
 * Defined by the FP8 casts of "Accelerating PyTorch Training Workloads with
 * FP8 -- Part 2" (round to nearest even onto the float8_e4m3fn / float8_e5m2
 * grids of its finfo table), by the transpose cache and scale-inverse copy of
 * "[PyTorch] Refactor FP8 workspaces in linear modules", by the noop flag that
 * change passes to its transpose for CUDA-graph weight caching, and by the
 * per-tensor amax buffers of "support delayed scaling of weight in float8
 * all-gather".  For every element:
 *
 *   v = fp32(x[r, c]) * (*scale)                 one fp32 multiply, RNE
 *   code = NaN(v)            ? 0x7F | (sign(x) ^ sign(*scale))
 *        : |v| >= fp8_max    ? sign(v) | max code (0x7E E4M3, 0x7B E5M2)
 *        :                   round v to the FP8 grid, ties to even
 *   out->data[r, c] = code;  out->data_t[c, r] = code     (each if non-NULL)
 *   *amax_cur = max(*amax_cur, |x[r, c]|)    (sign-cleared fp32 bit order; the
 *                                             UNSCALED source)
 * and *out->scale_inv = 1 / *scale (if out->scale_inv is non-NULL).
 *
 * x       device, [rows, cols] with row stride ld elements; src selects bf16 or
 *         fp32.  ld >= cols.
 * scale   device, 1 float (the delayed scale recorded by fp8_scale_update).
 * out     host descriptor; out->rows == rows, out->cols == cols, out->fmt the
 *         target format; data and/or data_t non-NULL.
 * amax_cur device, 1 float, max-accumulated (atomically, so several casts of
 *         one tensor in a step combine); must hold a non-negative value, e.g.
 *         0 after fp8_scale_update.  May be NULL to skip the amax.
 * noop_flag NULL, or a device int32: when it is non-zero at kernel time the
 *         call does nothing (weight caching under graph replay).
 * Constraints: rows, cols >= 0 and multiples of 16; x, data, data_t 16-byte
 * aligned; ld a multiple of 8 (bf16) or 4 (fp32); 128 * ld * element size
 * below 2^31 bytes.
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_ALIGN, FP8_ERR_FORMAT,
 * FP8_ERR_ARG, FP8_ERR_LAUNCH.
 */
int fp8_cast_transpose_amax(const void *x, int32_t src, int64_t rows, int64_t cols, int64_t ld,
                            const float *scale, const fp8_tensor_t *out, float *amax_cur,
                            const int32_t *noop_flag, fp8_stream_t stream);

/* Tensors per fp8_cast_transpose_amax_group call. */
#define FP8DSL_CAST_GROUP_MAX 8

/* One tensor of a grouped cast: the arguments of fp8_cast_transpose_amax. */
typedef struct fp8_cast_group_item {
    const void *x;              /* device source [rows, cols], row stride ld   */
    int64_t rows;
    int64_t cols;
    int64_t ld;
    const float *scale;         /* device, 1 float                             */
    const fp8_tensor_t *out;    /* host descriptor of the codes                */
    float *amax_cur;            /* device, 1 float, or NULL                    */
} fp8_cast_group_item_t;

/*
 * fp8_cast_transpose_amax_group -- several casts in one launch.
 *
 * The launches a model spends on casts are what the pages' fused layers
 * remove ("CPU Overhead of te.Linear FP8 Layers": fewer kernel launches when
 * casts are fused); a block's weights are cast together here.  Each item is
 * cast exactly as fp8_cast_transpose_amax(item.x, src, item.rows, item.cols,
 * item.ld, item.scale, item.out, item.amax_cur, noop_flag) casts it (the same
 * codes, transpose, amax and scale-inverse snapshot), all in one kernel
 * launch with one workgroup per 128 x 128 tile.
 *
 * src        FP8_DTYPE_BF16 or FP8_DTYPE_FP32, for every item.
 * items      host array of `count` items, 1 <= count <= FP8DSL_CAST_GROUP_MAX;
 *            read during the call only.  Every item's out->fmt must be the
 *            same, and so must the outputs it asks for (data, data_t or both:
 *            NULL or not alike across the items); items may not share
 *            outputs.  An item with no rows or columns only takes its
 *            scale-inverse snapshot (one more small launch).
 * noop_flag  as fp8_cast_transpose_amax: skips every item.
 * Constraints per item as fp8_cast_transpose_amax.
 * Errors: those of fp8_cast_transpose_amax for any item (nothing is enqueued
 * then); FP8_ERR_ARG for a count out of range or items that differ in
 * format or outputs; FP8_ERR_NULL for a NULL item array.
 */
int fp8_cast_transpose_amax_group(int32_t src, const fp8_cast_group_item_t *items, int32_t count,
                                  const int32_t *noop_flag, fp8_stream_t stream);

/*
 * fp8_cast_transpose_amax_cached -- fp8_cast_transpose_amax reading its
 * source through the caches.
 *
 * fp8_cast_transpose_amax reads the source with non-temporal loads: the
 * source is read once, and keeping it out of the last-level cache leaves the
 * codes it writes there for the products that read them next (a whole
 * forward + backward step of a linear is faster that way).  This variant
 * reads the source with ordinary loads, for a source that is read again soon
 * or a cast whose codes are not read next; a cast on its own is faster with
 * it.  Results are identical.  Arguments, constraints and errors as
 * fp8_cast_transpose_amax.
 */
int fp8_cast_transpose_amax_cached(const void *x, int32_t src, int64_t rows, int64_t cols,
                                   int64_t ld, const float *scale, const fp8_tensor_t *out,
                                   float *amax_cur, const int32_t *noop_flag,
                                   fp8_stream_t stream);

/*
 * fp8_reference_copy -- a measurement reference, not part of the method: a
 * plain device copy of `bytes` (a multiple of 16) from src to dst with
 * 16-byte accesses, `workgroups` workgroups of 256 threads (1 .. 65536)
 * striding over 16 KiB slabs, loads non-temporal when `nontemporal` is 1.
 * The cast moves exactly the bytes of a copy (its source read once, its
 * codes and their transpose written once), so the best copy rate of the
 * same volume on the same device is the ceiling the cast is measured
 * against.  src and dst: device, 16-byte aligned, not overlapping.
 * Errors: FP8_ERR_ARG, FP8_ERR_NULL, FP8_ERR_ALIGN, FP8_ERR_LAUNCH.
 */
int fp8_reference_copy(const void *src, void *dst, int64_t bytes, int32_t workgroups,
                       int32_t nontemporal, fp8_stream_t stream);

/*
 * fp8_cast_dbias_workspace_bytes -- device workspace (bytes) that
 * fp8_cast_transpose_amax_dbias needs for a [rows, cols] source:
 * ceil(rows / 128) * ceil(cols / 128) * 128 * sizeof(float).  Returns a
 * negative status for negative or oversized sizes.
 */
int64_t fp8_cast_dbias_workspace_bytes(int64_t rows, int64_t cols);

/*
 * fp8_cast_transpose_amax_dbias -- fp8_cast_transpose_amax plus the bias
 * gradient in the same pass over the source.
 *
 * The training loop of "CPU Overhead of te.Linear FP8 Layers" (reproduction
 * script: biased linears, fp32 parameters in its FP8 run, loss.backward())
 * needs, for a biased linear y = x W^T + b, the gradient of b, i.e. the
 * column sums of the output gradient dY:
 *
 *   dbias[c] = sum over r of x[r, c]       (unscaled source, fp32 result)
 *
 * Everything fp8_cast_transpose_amax writes is written identically (same
 * codes, transpose, amax, scale-inverse).  The sum is taken in fp32 in a
 * fixed order: per 128 x 128 tile, then over tiles in tile-row order (a
 * second small kernel), so repeated calls give identical bits; its error is
 * at most (ceil(rows / 128) + 12) * 2^-24 * sum over r of |x[r, c]|.
 *
 * dbias     device, [cols] fp32, overwritten; 4-byte aligned.
 * workspace device scratch of at least
 *           fp8_cast_dbias_workspace_bytes(rows, cols) bytes, 16-byte
 *           aligned, owned by the caller; its contents on entry do not
 *           matter and on return are unspecified.  Two calls that overlap
 *           on one workspace race.
 * rows == 0 writes dbias = 0 (cols > 0) and the scale-inverse snapshot;
 * noop_flag skips the whole call, dbias included.
 * Other arguments, constraints and errors as fp8_cast_transpose_amax.
 */
int fp8_cast_transpose_amax_dbias(const void *x, int32_t src, int64_t rows, int64_t cols,
                                  int64_t ld, const float *scale, const fp8_tensor_t *out,
                                  float *amax_cur, float *dbias, void *workspace,
                                  int64_t workspace_bytes, const int32_t *noop_flag,
                                  fp8_stream_t stream);

/* Bytes of the device scratch array behind fp8_cast_transpose_amax_dbias_noalloc
 * (one per GPU the library runs on, held until the process ends). */
#define FP8DSL_NOALLOC_SCRATCH_BYTES (4 << 20)

/*
 * fp8_cast_transpose_amax_dbias_noalloc -- fp8_cast_transpose_amax_dbias
 * without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.
 *
 * Same kernels, same results (codes, transpose, amax, scale-inverse and dbias
 * bit for bit) as fp8_cast_transpose_amax_dbias; the per-tile column sums go
 * into a file-scope device array of FP8DSL_NOALLOC_SCRATCH_BYTES bytes
 * instead of a caller workspace.  The call allocates and frees nothing.  The
 * first call on a device looks up that device's copy of the array once.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or several host threads) race and must be ordered
 * by the caller.  Nothing in the array needs to start at zero (every sum the
 * second pass reads is written by the first).
 *
 * Limit: fp8_cast_dbias_workspace_bytes(rows, cols) must not exceed
 * FP8DSL_NOALLOC_SCRATCH_BYTES (4 MiB: e.g. [8192, 16384] or [16384, 8192]);
 * larger sources return FP8_ERR_SCRATCH before anything is enqueued.
 * Other arguments, constraints and errors as fp8_cast_transpose_amax_dbias.
 */
int fp8_cast_transpose_amax_dbias_noalloc(const void *x, int32_t src, int64_t rows, int64_t cols,
                                          int64_t ld, const float *scale, const fp8_tensor_t *out,
                                          float *amax_cur, float *dbias,
                                          const int32_t *noop_flag, fp8_stream_t stream);

/*
 * fp8_produce_cast_transpose_amax -- the elementwise operation that produces
 * a linear's input, fused with that input's cast.
 *
 * In the toy block of "CPU Overhead of te.Linear FP8 Layers" (reproduction
 * script, TEBlock.forward) the input of a linear is made by torch elementwise
 * code right before the linear: the modulation (the block input times one
 * column slice of the modulation linear's output, divided by another slice)
 * and the residual adds onto the stream.  This call computes it and casts it
 * in one pass:
 *
 *   op FP8_PRODUCE_MODULATE: y = bf16(a * x / b)   (fp32 multiply, correctly
 *                            rounded fp32 division, round to nearest even);
 *                            nothing is sanitised: a zero divisor gives
 *                            +-inf, 0/0 a NaN written as 0x7FC0, and the
 *                            cast then saturates the infinities and codes the
 *                            NaN as 0x7F (the amax records the NaN)
 *   op FP8_PRODUCE_ADD:      y = bf16(x + a)       (fp32 add, round to nearest
 *                            even); a NaN y is written as 0x7FC0
 *   op FP8_PRODUCE_ADD2:     y = bf16(bf16(x + a) + b)   (the block's residual
 *                            add of the two cross-attention outputs, one term
 *                            at a time as torch adds them, each sum rounded;
 *                            a NaN at either step is written as 0x7FC0)
 *
 *   op FP8_PRODUCE_MODULATE_FINITE: this library's addition, on no page:
 *                            FP8_PRODUCE_MODULATE, then a y that is not
 *                            finite becomes +0.  For models whose divisor
 *                            can be exactly zero: under delayed scaling a
 *                            record whose amax is infinite keeps its scale,
 *                            so without it one zero divisor keeps a model at
 *                            its initial scales and spreads NaNs
 *
 * then writes y (bf16, row-major [rows, cols], ld = cols) and exactly what
 * fp8_cast_transpose_amax writes for the bf16 source y with this scale.
 *
 * x, a, b   device bf16 [rows, cols] with row strides ldx, lda, ldb
 *           (elements, each >= cols and a multiple of 8; 16-byte aligned); b
 *           is read by MODULATE and ADD2 (NULL for ADD).  Column slices of a
 *           wider tensor are fine.
 * y         device bf16 [rows, cols], 16-byte aligned; must not overlap the
 *           inputs.
 * Other arguments, constraints (rows, cols multiples of 16) and errors as
 * fp8_cast_transpose_amax; FP8_ERR_ARG for an unknown op.
 */
int fp8_produce_cast_transpose_amax(int32_t op, const uint16_t *x, int64_t ldx,
                                    const uint16_t *a, int64_t lda, const uint16_t *b,
                                    int64_t ldb, uint16_t *y, int64_t rows, int64_t cols,
                                    const float *scale, const fp8_tensor_t *out, float *amax_cur,
                                    const int32_t *noop_flag, fp8_stream_t stream);

/*
 * fp8_produce_modulate_backward -- the gradient of the modulation producer
 * (op FP8_PRODUCE_MODULATE or FP8_PRODUCE_MODULATE_FINITE above) with respect
 * to its three inputs, in one pass: the backward of the toy block's
 * modulation that the training loop of "CPU Overhead of te.Linear FP8
 * Layers" runs through autograd, whose da and db form the modulation
 * linear's output gradient (cast next, to E5M2 with the bias gradient).
 *
 * For y = a * x / b and the gradient dy of y, with fp32 arithmetic on the
 * exactly widened bf16 inputs and every step rounded to nearest even:
 *   u  = (a * x) / b          (the forward's quotient before its rounding)
 *   t  = dy / b
 *   dx = bf16(t * a),  da = bf16(t * x),  db = bf16(-(t * u))
 * a NaN result is written as 0x7FC0.  Op FP8_PRODUCE_MODULATE_FINITE: where
 * the forward's bf16(u) is infinite or NaN (the forward wrote +0 there, a
 * constant) dx, da and db are +0.
 *
 * dy, x, a, b   device bf16 [rows, cols], row strides lddy, ldx, lda, ldb
 * dx, da, db    device bf16 [rows, cols], row strides lddx, ldda, lddb;
 *               column slices of wider tensors are fine for all seven.  The
 *               outputs must not overlap each other or the inputs.
 * rows >= 0; cols a multiple of 8; every stride >= cols and a multiple of 8
 * elements; every pointer 16-byte aligned.  Allocates nothing.
 * Errors: FP8_ERR_ARG (another op), FP8_ERR_SHAPE, FP8_ERR_NULL,
 * FP8_ERR_ALIGN, FP8_ERR_LAUNCH / FP8_ERR_DEVICE.  rows or cols 0: no work.
 */
int fp8_produce_modulate_backward(int32_t op, const uint16_t *dy, int64_t lddy,
                                  const uint16_t *x, int64_t ldx, const uint16_t *a, int64_t lda,
                                  const uint16_t *b, int64_t ldb, uint16_t *dx, int64_t lddx,
                                  uint16_t *da, int64_t ldda, uint16_t *db, int64_t lddb,
                                  int64_t rows, int64_t cols, fp8_stream_t stream);

/*
 * fp8_cast_transpose_dynamic -- dynamic scaling, the comparator of delayed
 * scaling ("support delayed scaling of weight in float8 all-gather" contrasts
 * them: dynamic scaling reads the tensor twice, delayed scaling once).
 *
 *   *amax  = max |x|  of this tensor (sign-cleared fp32 bit order)
 *   *scale = fp8_max / (*amax * 2^margin)   -- the fp8_scale_update formula;
 *            the value in *scale on entry is kept when *amax is zero or not
 *            finite or the quotient is not a finite positive number
 * then exactly fp8_cast_transpose_amax with that scale (without amax
 * accumulation).  Four launches on `stream`: clear *amax, an amax-only pass
 * over x, the scale, the cast.
 *
 * scale   device, 1 float, in: fallback scale, out: the scale used.
 * amax    device, 1 float, out.
 * margin  -126 .. 126.
 * Other arguments, constraints and errors as fp8_cast_transpose_amax.
 */
int fp8_cast_transpose_dynamic(const void *x, int32_t src, int64_t rows, int64_t cols,
                               int64_t ld, int32_t margin, float *scale, const fp8_tensor_t *out,
                               float *amax, const int32_t *noop_flag, fp8_stream_t stream);

/*
 * fp8_linear_fwd -- Y = X W^T + bias on FP8 operands.
 *
 * Defined by torch._scaled_mm in "Accelerating PyTorch Training Workloads with
 * FP8 -- Part 2" (first operand row-major, second transposed, per-tensor
 * scales held on the device, optional bf16 bias, chosen output type) and by
 * the te.Linear forward of "CPU Overhead of te.Linear FP8 Layers":
 *
 *   y[m, n] = bf16_rne( (sum_k dec(x[m,k]) dec(w[n,k])) * x_sinv * w_sinv + bias[n] )
 *
 * with fp32 accumulation.  x->data [M, K] and w->data [N, K] (E4M3 or E5M2
 * each), their scale_inv snapshots, bias device bf16 [N] or NULL, y device
 * bf16 [M, N].
 * Constraints: M, N >= 0 (0 is a no-op), K >= 0 and a multiple of 16, 16-byte
 * aligned pointers, N a multiple of 8.
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_ALIGN, FP8_ERR_FORMAT,
 * FP8_ERR_LAUNCH.
 */
int fp8_linear_fwd(const fp8_tensor_t *x, const fp8_tensor_t *w, const uint16_t *bias,
                   uint16_t *y, fp8_stream_t stream);

/*
 * fp8_linear_fwd_fp8out -- Y = X W^T + bias with an FP8 output and its amax.
 *
 * torch._scaled_mm called with an FP8 out_dtype returns the FP8 output
 * together with the output's amax ("Accelerating PyTorch Training Workloads
 * with FP8 -- Part 2", the torch._scaled_mm example).  The product is the one
 * of fp8_linear_fwd, kept in fp32, and then cast as fp8_cast_transpose_amax
 * casts, with the output tensor's own delayed scale:
 *
 *   v[m, n]  = fp32( (sum_k dec(x[m,k]) dec(w[n,k])) * x_sinv * w_sinv + bias[n] )
 *   y->data[m, n] = the cast of v with *scale_y (one fp32 multiply, saturating
 *                   round to nearest even, NaN -> 0x7F | sign)
 *   *amax_y  = max(*amax_y, |v[m, n]|)   (UNSCALED v, sign-cleared fp32 bit
 *                                          order: the value the output's amax
 *                                          history records)
 *   *y->scale_inv = 1 / *scale_y          (if y->scale_inv is non-NULL)
 *
 * x, w, bias as fp8_linear_fwd.  scale_y device, 1 float.  y host descriptor:
 * y->data device [M, N] codes in y->fmt (E4M3 or E5M2), y->rows == M,
 * y->cols == N, y->data_t must be NULL (no transposed output).  amax_y device,
 * 1 float, max-accumulated atomically; must hold a non-negative value (e.g. 0
 * after fp8_scale_update); may be NULL to skip the amax.  With M or N zero
 * only the scale-inverse snapshot is written.
 * Constraints: as fp8_linear_fwd, with N a multiple of 16.
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_ALIGN, FP8_ERR_FORMAT,
 * FP8_ERR_ARG (y->data_t set), FP8_ERR_LAUNCH.
 */
int fp8_linear_fwd_fp8out(const fp8_tensor_t *x, const fp8_tensor_t *w, const uint16_t *bias,
                          const float *scale_y, const fp8_tensor_t *y, float *amax_y,
                          fp8_stream_t stream);

/*
 * fp8_linear_dgrad -- dX = dY W on FP8 operands, using W's cached transpose.
 *
 * The backward data product of te.Linear ("CPU Overhead of te.Linear FP8
 * Layers", loss.backward under fp8_autocast with the HYBRID format: gradients
 * in E5M2) reading the transpose cache of "[PyTorch] Refactor FP8 workspaces
 * in linear modules":
 *
 *   dx[m, k] = bf16_rne( (sum_n dec(dy[m,n]) dec(w_t[k,n])) * dy_sinv * w_sinv )
 *
 * dy->data [M, N], w->data_t [K, N] (w->rows = N, w->cols = K), dx device
 * bf16 [M, K].  Constraints as fp8_linear_fwd with the contraction N a
 * multiple of 16 and K a multiple of 8.
 */
int fp8_linear_dgrad(const fp8_tensor_t *dy, const fp8_tensor_t *w, uint16_t *dx,
                     fp8_stream_t stream);

/*
 * fp8_linear_wgrad -- dW = dY^T X on FP8 operands, using both transposes.
 *
 *   dw[n, k] = out( (sum_m dec(dy_t[n,m]) dec(x_t[k,m])) * dy_sinv * x_sinv )
 *
 * dy->data_t [N, M] (dy->rows = M, dy->cols = N), x->data_t [K, M]
 * (x->rows = M, x->cols = K), dw device [N, K] in out_dtype (FP8_DTYPE_FP32
 * for fp32 master weights, as in the FP8 run of the reproduction script of
 * "CPU Overhead of te.Linear FP8 Layers", or FP8_DTYPE_BF16).  Constraints as
 * fp8_linear_fwd with the contraction M a multiple of 16 and K a multiple of 8.
 */
int fp8_linear_wgrad(const fp8_tensor_t *dy, const fp8_tensor_t *x, void *dw, int32_t out_dtype,
                     fp8_stream_t stream);

/*
 * The same three products with a caller-owned workspace, for products whose
 * few output tiles would leave compute units idle over a long contraction:
 * the weight gradient of a 2048 x 2048 linear over 16384 or more tokens, of a
 * 2048 x 1024 one over 32768.
 *
 * Each is the product of the entry point without "_ws" (same arguments,
 * constraints, errors and rounding of the result), computed in K parts when
 * the workspace allows: every part's fp32 sum of products goes to the
 * workspace, then a second pass adds the parts in part order (fp32) and
 * applies the scale-inverses, the bias and the output rounding.  The sum
 * over K is thus grouped differently from the unsplit product (the result
 * differs from it within fp32 accumulation error); repeated calls with the
 * same workspace size give identical bits.  The part count P is the largest
 * (at most 16) whose (tile, part) units of 256 x 256 outputs fill between
 * three quarters of the compute units and all of them, with K a multiple of
 * 128 P and at least 4096 contraction bytes per part (the parts' sums cost
 * 8 P M N bytes of memory traffic, repaid only by long parts).  Products with
 * more than one 128 x 128 tile or three quarters of a 256 x 256 tile per
 * compute unit are never split: the unsplit kernels keep the chip busy.
 *
 * fp8_gemm_workspace_bytes(M, N, K): the workspace bytes the split form of a
 * product with output [M, N] and contraction K uses on the current device
 * (M, N, K: fwd (tokens, out features, in features), dgrad (tokens, in, out),
 * wgrad (out, in, tokens)); 0 when the product fills the device unsplit.  A
 * negative value is a status code (FP8_ERR_SHAPE for negative sizes, or the
 * device query's error).
 *
 * workspace        device, 16-byte aligned, owned by the caller; NULL (any
 *                  size) computes unsplit.  A workspace smaller than
 *                  fp8_gemm_workspace_bytes gives fewer parts or none, never
 *                  an error.  Its contents on entry do not matter and on
 *                  return are unspecified; calls that overlap on one
 *                  workspace race.
 * workspace_bytes  its size; negative with a non-NULL workspace is FP8_ERR_ARG.
 * Errors: those of the unsplit entry point, FP8_ERR_ALIGN (workspace),
 * FP8_ERR_ARG.
 */
int64_t fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int fp8_linear_fwd_ws(const fp8_tensor_t *x, const fp8_tensor_t *w, const uint16_t *bias,
                      uint16_t *y, void *workspace, int64_t workspace_bytes,
                      fp8_stream_t stream);
int fp8_linear_dgrad_ws(const fp8_tensor_t *dy, const fp8_tensor_t *w, uint16_t *dx,
                        void *workspace, int64_t workspace_bytes, fp8_stream_t stream);
int fp8_linear_wgrad_ws(const fp8_tensor_t *dy, const fp8_tensor_t *x, void *dw,
                        int32_t out_dtype, void *workspace, int64_t workspace_bytes,
                        fp8_stream_t stream);

/* Human-readable name of a status code (static storage). */
const char *fp8_status_string(int status);

/* FP8DSL_ABI_VERSION of the built library. */
int fp8_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8DSL_H */
