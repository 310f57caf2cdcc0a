// Internal declarations shared by the kernels and the C-ABI layer of the
// delayed-scaling FP8 linear library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fp8dsl.h"

namespace fp8dsl {

// Number of compute units of the current device.  Cached per device after the
// first query (an immutable fact of the device; concurrent first calls store
// the same value), so launchers can size persistent grids without a runtime
// query per call.
hipError_t current_cu_count(int *cu_count);

// Enables `lds_bytes` of dynamic LDS for `kernel` on the current device once
// (the runtime call is idempotent, so a race repeats it harmlessly).  `done`
// is one bit per device owned by the calling launcher.
hipError_t enable_dynamic_lds(const void *kernel, int lds_bytes, std::atomic<uint64_t> &done);

// K parts for the split form of the product C [M, N] (contraction K) on a
// device with `cus` compute units and `ws_bytes` of workspace.  The parts'
// fp32 sums go out to memory and are read back (8 P M N bytes, at about the
// HBM rate), so a split only pays where the unsplit kernels leave most CUs
// idle for a long time: products with at most one 128 x 128 tile per CU and
// fewer than three quarters of a 256 x 256 tile per CU, split into P parts
// of at least SPLIT_MIN_K contraction bytes that occupy at least three
// quarters of the CUs (tiles * P between 3/4 cus and cus, K a multiple of
// 128 P, the P * M * N fp32 sums within ws_bytes); else 1 (no split).
// Measured on MI355X against the direct-to-LDS small kernel: 2048 x 2048
// and 4096 x 2048 over K = 8192 run faster unsplit (48-51 / 65-70 us
// against 52 / 77 us in 4 / 2 parts), while K = 16384 and beyond split.
constexpr int64_t SPLIT_MIN_K = 4096;
inline int gemm_split_parts(int64_t M, int64_t N, int64_t K, int cus, int64_t ws_bytes) {
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    if (M <= 0 || N <= 0 || tiles == 0) return 1;
    if (M * N >= (int64_t)256 * 256 * 256 || 4 * tiles >= 3 * (int64_t)cus) return 1;
    if (((M + 127) / 128) * ((N + 127) / 128) > cus) return 1;
    if (K % 128 != 0) return 1;
    int best = 1;
    for (int p = 2; p <= 16; ++p) {
        if (K / p < SPLIT_MIN_K || tiles * p > cus || (int64_t)p * M * N * 4 > ws_bytes) break;
        if (K % (128 * p) == 0 && 4 * tiles * p >= 3 * (int64_t)cus) best = p;
    }
    return best;
}

// Launchers: each validates nothing (the C-ABI layer has done that), enqueues
// one kernel on `stream` and returns the launch status.
hipError_t launch_scale_update(float *hist, float *amax_cur, float *scale, float *scale_inv,
                               const uint8_t *fmt, int T, int H, int margin,
                               hipStream_t stream);

// dbias_ws: nullptr, or the bias-gradient workspace [tiles_r, ws_ld] fp32
// (ws_ld = 128 * tiles_c) that receives each tile's column sums.
hipError_t launch_cast_transpose_amax(const void *x, int src, int64_t rows, int64_t cols,
                                      int64_t ld, const float *scale, int fmt, uint8_t *q,
                                      uint8_t *qt, float *amax_cur, float *scale_inv_out,
                                      const int32_t *noop, float *dbias_ws, int64_t ws_ld,
                                      hipStream_t stream, bool cached = false);

// A grouped cast: up to kCastGroupMax tensors (one source type, one format,
// the same outputs wanted) in one launch of cast_tile_group_kernel.  first[i]
// is the first tile of tensor i in the launch (first[n] = all tiles), each
// tensor's tiles row-major over tiles_c tile columns.
constexpr int kCastGroupMax = FP8DSL_CAST_GROUP_MAX;
struct CastGroupItem {
    const void *x;
    int64_t rows, cols, ld, tiles_c;
    const float *scale;
    uint8_t *q, *qt;
    float *amax_cur, *scale_inv;
};
struct CastGroupArgs {
    int n;
    int64_t first[kCastGroupMax + 1];
    CastGroupItem item[kCastGroupMax];
};
hipError_t launch_cast_group(const CastGroupArgs &args, int src, int fmt, bool want_q,
                             bool want_qt, const int32_t *noop, bool cached,
                             hipStream_t stream);

// Measurement reference: copy `bytes` (a multiple of 16) from src to dst with
// 16-byte loads and stores, `blocks` workgroups of 256 threads, loads
// non-temporal or not.
hipError_t launch_reference_copy(const void *src, void *dst, int64_t bytes, int blocks,
                                 bool nontemporal, hipStream_t stream);

// y = op(x, a, b) in bf16 (row-major [rows, cols]), then the cast of y.
hipError_t launch_produce_cast(int op, const uint16_t *x, int64_t ldx, const uint16_t *a,
                               int64_t lda, const uint16_t *b, int64_t ldb, uint16_t *y,
                               int64_t rows, int64_t cols, const float *scale, int fmt,
                               uint8_t *q, uint8_t *qt, float *amax_cur, float *scale_inv_out,
                               const int32_t *noop, hipStream_t stream);

// Gradient of y = a * x / b: dx, da, db (bf16 [rows, cols], cols % 8 == 0,
// row strides multiples of 8 elements, 16-byte aligned).
hipError_t launch_modulate_backward(bool finite, const uint16_t *dy, int64_t lddy,
                                    const uint16_t *x, int64_t ldx, const uint16_t *a,
                                    int64_t lda, const uint16_t *b, int64_t ldb, uint16_t *dx,
                                    int64_t lddx, uint16_t *da, int64_t ldda, uint16_t *db,
                                    int64_t lddb, int64_t rows, int64_t cols,
                                    hipStream_t stream);

// Dynamic scaling: *amax = max |x| (cleared first), then *scale = fp8_max /
// (amax * 2^margin) unless zero / non-finite (the scale update's guard).
hipError_t launch_dynamic_scale(const void *x, int src, int64_t rows, int64_t cols, int64_t ld,
                                int fmt, int margin, float *amax, float *scale,
                                const int32_t *noop, hipStream_t stream);

// dbias[c] = sum over tr < tiles_r of ws[tr * ws_ld + c] (tile-row order).
hipError_t launch_dbias_reduce(const float *ws, int64_t tiles_r, int64_t ws_ld, int64_t cols,
                               float *dbias, const int32_t *noop, hipStream_t stream);

hipError_t launch_scale_inv_only(const float *scale, float *scale_inv_out, const int32_t *noop,
                                 hipStream_t stream);

// C[i, j] = out( sum_k dec(A[i, k]) dec(B[j, k]) * (*sinv_a) * (*sinv_b) + bias[j] )
// A [M, K], B [N, K] row-major FP8; C [M, N] row-major, bf16 (out_dtype 0) or
// fp32 (1).  bias is bf16 [N] or nullptr.
// ws (may be nullptr): the split form's workspace of ws_bytes bytes (16-byte
// aligned), used when gemm_split_parts(M, N, K, CUs, ws_bytes) > 1.
hipError_t launch_gemm_nt(const uint8_t *A, int fa, const uint8_t *B, int fb, int64_t M,
                          int64_t N, int64_t K, const float *sinv_a, const float *sinv_b,
                          const uint16_t *bias, int out_dtype, void *C, hipStream_t stream,
                          void *ws = nullptr, int64_t ws_bytes = 0);

// The same product with an FP8 output (format fo): C [M, N] codes = the cast
// of v = acc * (*sinv_a) * (*sinv_b) + bias[j] (fp32) with *scale_out;
// *amax (non-negative or NaN; may be null) folds in max |v| of the unscaled
// output; *scale_inv (may be null) = 1 / *scale_out.  N % 16 == 0.
hipError_t launch_gemm_nt_fp8out(const uint8_t *A, int fa, const uint8_t *B, int fb, int64_t M,
                                 int64_t N, int64_t K, const float *sinv_a, const float *sinv_b,
                                 const uint16_t *bias, int fo, const float *scale_out,
                                 uint8_t *C, float *amax, float *scale_inv, hipStream_t stream);

}  // namespace fp8dsl
