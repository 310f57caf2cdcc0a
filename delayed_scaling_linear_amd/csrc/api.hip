// C-ABI entry points of the delayed-scaling FP8 linear library.
//
// This layer only validates arguments and picks a launcher; every step of
// the computation runs in the HIP kernels.  It allocates nothing, never
// synchronises and never reads device memory, so every call is capturable in
// a HIP graph (the class of bug "[PyTorch] Refactor FP8 workspaces in linear
// modules" describes for transpose caches filled outside the captured region
// cannot arise: the cast always writes the transpose it is asked for).
#include <string.h>

#include "fp8dsl_internal.h"

using namespace fp8dsl;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool valid_fmt(int32_t f) { return f == FP8_E4M3 || f == FP8_E5M2; }

// A launch on a device this library has no code object for (anything but a
// gfx950) fails in the runtime; that is reported as FP8_ERR_DEVICE.
int status_of(hipError_t e) {
    if (e == hipSuccess) return FP8_OK;
    if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction ||
        e == hipErrorInvalidImage || e == hipErrorInvalidDevice || e == hipErrorNoDevice)
        return FP8_ERR_DEVICE;
    return FP8_ERR_LAUNCH;
}

// Shared checks of one GEMM: A [M, K], B [N, K], C [M, N].
int check_gemm(const uint8_t *A, const uint8_t *B, int64_t M, int64_t N, int64_t K,
               const float *sa, const float *sb, const void *C, int64_t out_align_elems) {
    if (M < 0 || N < 0 || K < 0 || (K % 16) != 0 || (N % out_align_elems) != 0)
        return FP8_ERR_SHAPE;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return FP8_ERR_SHAPE;
    if (M == 0 || N == 0) return FP8_OK;
    if (C == nullptr || sa == nullptr || sb == nullptr) return FP8_ERR_NULL;
    if (K > 0 && (A == nullptr || B == nullptr)) return FP8_ERR_NULL;
    if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B)))) return FP8_ERR_ALIGN;
    return FP8_OK;
}

// Shared checks of the two cast entry points (shape, format, alignment).
int check_cast(const void *x, int32_t src, int64_t rows, int64_t cols, int64_t ld,
               const float *scale, const fp8_tensor_t *out) {
    if (out == nullptr) return FP8_ERR_NULL;
    if (src != FP8_DTYPE_BF16 && src != FP8_DTYPE_FP32) return FP8_ERR_ARG;
    if (!valid_fmt(out->fmt)) return FP8_ERR_FORMAT;
    if (out->reserved != 0) return FP8_ERR_ARG;
    if (rows < 0 || cols < 0 || (rows % 16) != 0 || (cols % 16) != 0 || ld < cols ||
        (ld % (src == FP8_DTYPE_BF16 ? 8 : 4)) != 0 || out->rows != rows || out->cols != cols)
        return FP8_ERR_SHAPE;
    const int64_t tiles = ((rows + 127) / 128) * ((cols + 127) / 128);
    if (tiles > INT32_MAX) return FP8_ERR_SHAPE;
    // A 128-row tile of the source is addressed with 32-bit byte offsets.
    if (128 * ld * (src == FP8_DTYPE_BF16 ? 2 : 4) >= ((int64_t)1 << 31)) return FP8_ERR_SHAPE;
    if (scale == nullptr) return FP8_ERR_NULL;
    const bool empty = (rows == 0 || cols == 0);
    if (!empty && (x == nullptr || (out->data == nullptr && out->data_t == nullptr)))
        return FP8_ERR_NULL;
    if ((x && !aligned16(x)) || (out->data && !aligned16(out->data)) ||
        (out->data_t && !aligned16(out->data_t)))
        return FP8_ERR_ALIGN;
    return FP8_OK;
}

// Scratch of fp8_cast_transpose_amax_dbias_noalloc: each GPU holds its own
// copy of this array.  In host code its name is only a stand-in for the
// device symbol, so host code never passes it to a kernel: the device
// address is looked up once per device (with that device current) and kept
// in noalloc_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[FP8DSL_NOALLOC_SCRATCH_BYTES];
std::atomic<void *> noalloc_scratch_ptr[64];

// Device address of `scratch` on the current device (looked up on the first
// call per device; concurrent first calls store the same address).
hipError_t noalloc_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void *p = noalloc_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        noalloc_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace

namespace fp8dsl {

hipError_t current_cu_count(int *cu_count) {
    static std::atomic<int> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (n <= 0) return hipErrorInvalidDevice;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    *cu_count = n;
    return hipSuccess;
}

hipError_t enable_dynamic_lds(const void *kernel, int lds_bytes, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    const uint64_t bit = uint64_t(1) << dev;
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    done.fetch_or(bit, std::memory_order_release);
    return hipSuccess;
}

}  // namespace fp8dsl

extern "C" {

int fp8_abi_version(void) { return FP8DSL_ABI_VERSION; }

const char *fp8_status_string(int status) {
    switch (status) {
        case FP8_OK: return "FP8_OK";
        case FP8_ERR_NULL: return "FP8_ERR_NULL: a required pointer is NULL";
        case FP8_ERR_SHAPE: return "FP8_ERR_SHAPE: size out of range or not a required multiple";
        case FP8_ERR_ALIGN: return "FP8_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
        case FP8_ERR_FORMAT: return "FP8_ERR_FORMAT: FP8 format not accepted here";
        case FP8_ERR_ARG: return "FP8_ERR_ARG: argument out of range";
        case FP8_ERR_LAUNCH: return "FP8_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
        case FP8_ERR_DEVICE: return "FP8_ERR_DEVICE: no gfx950 code object for the current device";
        case FP8_ERR_SCRATCH:
            return "FP8_ERR_SCRATCH: the call needs more scratch than the no-allocation entry "
                   "point holds (FP8DSL_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown fp8dsl status";
    }
}

int fp8_scale_update(float *amax_history, float *amax_cur, float *scale, float *scale_inv,
                     const uint8_t *fmt, int32_t T, int32_t H, int32_t margin, int32_t algo,
                     fp8_stream_t stream) {
    if (T < 0 || H < 1 || H > 1024 || margin < -126 || margin > 126 ||
        algo != FP8_AMAX_ALGO_MAX)
        return FP8_ERR_ARG;
    if (T == 0) return FP8_OK;
    if (!amax_history || !amax_cur || !scale || !scale_inv || !fmt) return FP8_ERR_NULL;
    return status_of(launch_scale_update(amax_history, amax_cur, scale, scale_inv, fmt, T, H,
                                         margin, static_cast<hipStream_t>(stream)));
}

int fp8_cast_transpose_amax(const void *x, int32_t src, int64_t rows, int64_t cols, int64_t ld,
                            const float *scale, const fp8_tensor_t *out, float *amax_cur,
                            const int32_t *noop_flag, fp8_stream_t stream) {
    if (int e = check_cast(x, src, rows, cols, ld, scale, out)) return e;
    const bool empty = (rows == 0 || cols == 0);
    // Nothing to cast in an empty tensor; the scale-inverse snapshot is still taken.
    if (empty && out->scale_inv == nullptr) return FP8_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (empty) return status_of(launch_scale_inv_only(scale, out->scale_inv, noop_flag, s));
    return status_of(launch_cast_transpose_amax(x, src, rows, cols, ld, scale, out->fmt,
                                                out->data, out->data_t, amax_cur, out->scale_inv,
                                                noop_flag, nullptr, 0, s));
}

int fp8_cast_transpose_amax_group(int32_t src, const fp8_cast_group_item_t *items, int32_t count,
                                  const int32_t *noop_flag, fp8_stream_t stream) {
    if (items == nullptr) return FP8_ERR_NULL;
    if (count < 1 || count > FP8DSL_CAST_GROUP_MAX) return FP8_ERR_ARG;
    // Every check first: nothing is enqueued on an error.
    CastGroupArgs args{};
    args.n = 0;
    int64_t tiles = 0;
    // One format for all; the same outputs asked of every non-empty item (an
    // empty item writes no codes, whatever its pointers).
    const fp8_tensor_t *first_out = nullptr;
    for (int i = 0; i < count; ++i) {
        const fp8_cast_group_item_t &it = items[i];
        if (int e = check_cast(it.x, src, it.rows, it.cols, it.ld, it.scale, it.out)) return e;
        if (it.out->fmt != items[0].out->fmt) return FP8_ERR_ARG;
        if (it.rows == 0 || it.cols == 0) continue;
        if (first_out == nullptr) {
            first_out = it.out;
        } else if ((it.out->data == nullptr) != (first_out->data == nullptr) ||
                   (it.out->data_t == nullptr) != (first_out->data_t == nullptr)) {
            return FP8_ERR_ARG;
        }
    }
    int64_t all_tiles = 0;
    for (int i = 0; i < count; ++i) {
        for (int j = 0; j < i; ++j) {
            const fp8_tensor_t *a = items[i].out, *b = items[j].out;
            if ((a->data && a->data == b->data) || (a->data_t && a->data_t == b->data_t))
                return FP8_ERR_ARG;
        }
        all_tiles += ((items[i].rows + 127) / 128) * ((items[i].cols + 127) / 128);
    }
    if (all_tiles > INT32_MAX) return FP8_ERR_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int i = 0; i < count; ++i) {
        const fp8_cast_group_item_t &it = items[i];
        if (it.rows == 0 || it.cols == 0) {
            // Nothing to cast; the snapshot is still taken.
            if (it.out->scale_inv) {
                if (int e = status_of(launch_scale_inv_only(it.scale, it.out->scale_inv,
                                                            noop_flag, s)))
                    return e;
            }
            continue;
        }
        CastGroupItem &g = args.item[args.n];
        g.x = it.x;
        g.rows = it.rows;
        g.cols = it.cols;
        g.ld = it.ld;
        g.tiles_c = (it.cols + 127) / 128;
        g.scale = it.scale;
        g.q = it.out->data;
        g.qt = it.out->data_t;
        g.amax_cur = it.amax_cur;
        g.scale_inv = it.out->scale_inv;
        args.first[args.n] = tiles;
        tiles += ((it.rows + 127) / 128) * g.tiles_c;
        ++args.n;
    }
    for (int i = args.n; i <= FP8DSL_CAST_GROUP_MAX; ++i) args.first[i] = tiles;
    if (args.n == 0) return FP8_OK;   // only empty items: their snapshots are taken
    return status_of(launch_cast_group(args, src, first_out->fmt, first_out->data != nullptr,
                                       first_out->data_t != nullptr, noop_flag, false, s));
}

int fp8_cast_transpose_amax_cached(const void *x, int32_t src, int64_t rows, int64_t cols,
                                   int64_t ld, const float *scale, const fp8_tensor_t *out,
                                   float *amax_cur, const int32_t *noop_flag,
                                   fp8_stream_t stream) {
    if (int e = check_cast(x, src, rows, cols, ld, scale, out)) return e;
    const bool empty = (rows == 0 || cols == 0);
    if (empty && out->scale_inv == nullptr) return FP8_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (empty) return status_of(launch_scale_inv_only(scale, out->scale_inv, noop_flag, s));
    return status_of(launch_cast_transpose_amax(x, src, rows, cols, ld, scale, out->fmt,
                                                out->data, out->data_t, amax_cur, out->scale_inv,
                                                noop_flag, nullptr, 0, s, /*cached=*/true));
}

int fp8_reference_copy(const void *src, void *dst, int64_t bytes, int32_t workgroups,
                       int32_t nontemporal, fp8_stream_t stream) {
    if (bytes < 0 || (bytes % 16) != 0 || workgroups < 1 || workgroups > 65536 ||
        (nontemporal != 0 && nontemporal != 1))
        return FP8_ERR_ARG;
    if (bytes == 0) return FP8_OK;
    if (src == nullptr || dst == nullptr) return FP8_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst)) return FP8_ERR_ALIGN;
    return status_of(launch_reference_copy(src, dst, bytes, workgroups, nontemporal != 0,
                                           static_cast<hipStream_t>(stream)));
}

int64_t fp8_cast_dbias_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0 || rows > INT32_MAX || cols > INT32_MAX) return FP8_ERR_SHAPE;
    return ((rows + 127) / 128) * ((cols + 127) / 128) * 128 * (int64_t)sizeof(float);
}

int fp8_cast_transpose_amax_dbias_noalloc(const void *x, int32_t src, int64_t rows, int64_t cols,
                                          int64_t ld, const float *scale, const fp8_tensor_t *out,
                                          float *amax_cur, float *dbias,
                                          const int32_t *noop_flag, fp8_stream_t stream) {
    // Size and argument checks first: nothing is enqueued on an error.
    if (int e = check_cast(x, src, rows, cols, ld, scale, out)) return e;
    if (cols > 0 && dbias == nullptr) return FP8_ERR_NULL;
    if (dbias && (reinterpret_cast<uintptr_t>(dbias) & 3) != 0) return FP8_ERR_ALIGN;
    const int64_t need = fp8_cast_dbias_workspace_bytes(rows, cols);
    if (need < 0) return (int)need;
    if (need > FP8DSL_NOALLOC_SCRATCH_BYTES) return FP8_ERR_SCRATCH;
    void *ws = nullptr;
    if (hipError_t e = noalloc_scratch(&ws)) return status_of(e);
    return fp8_cast_transpose_amax_dbias(x, src, rows, cols, ld, scale, out, amax_cur, dbias, ws,
                                         FP8DSL_NOALLOC_SCRATCH_BYTES, noop_flag, stream);
}

int fp8_cast_transpose_amax_dbias(const void *x, int32_t src, int64_t rows, int64_t cols,
                                  int64_t ld, const float *scale, const fp8_tensor_t *out,
                                  float *amax_cur, float *dbias, void *workspace,
                                  int64_t workspace_bytes, const int32_t *noop_flag,
                                  fp8_stream_t stream) {
    if (int e = check_cast(x, src, rows, cols, ld, scale, out)) return e;
    if (cols > 0 && dbias == nullptr) return FP8_ERR_NULL;
    if (dbias && (reinterpret_cast<uintptr_t>(dbias) & 3) != 0) return FP8_ERR_ALIGN;
    const bool empty = (rows == 0 || cols == 0);
    const int64_t tiles_r = (rows + 127) / 128, tiles_c = (cols + 127) / 128;
    if (!empty) {
        if (workspace == nullptr) return FP8_ERR_NULL;
        if (workspace_bytes < fp8_cast_dbias_workspace_bytes(rows, cols)) return FP8_ERR_SHAPE;
        if (!aligned16(workspace)) return FP8_ERR_ALIGN;
    }
    if (cols == 0 && out->scale_inv == nullptr) return FP8_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (empty) {
        // No rows: the bias gradient is zero; the scale-inverse snapshot is still taken.
        if (out->scale_inv) {
            if (int e = status_of(launch_scale_inv_only(scale, out->scale_inv, noop_flag, s)))
                return e;
        }
        return status_of(launch_dbias_reduce(nullptr, 0, 0, cols, dbias, noop_flag, s));
    }
    float *ws = static_cast<float *>(workspace);
    if (int e = status_of(launch_cast_transpose_amax(x, src, rows, cols, ld, scale, out->fmt,
                                                     out->data, out->data_t, amax_cur,
                                                     out->scale_inv, noop_flag, ws,
                                                     128 * tiles_c, s)))
        return e;
    return status_of(launch_dbias_reduce(ws, tiles_r, 128 * tiles_c, cols, dbias, noop_flag, s));
}

int fp8_produce_cast_transpose_amax(int32_t op, const uint16_t *x, int64_t ldx,
                                    const uint16_t *a, int64_t lda, const uint16_t *b,
                                    int64_t ldb, uint16_t *y, int64_t rows, int64_t cols,
                                    const float *scale, const fp8_tensor_t *out, float *amax_cur,
                                    const int32_t *noop_flag, fp8_stream_t stream) {
    if (op != FP8_PRODUCE_MODULATE && op != FP8_PRODUCE_ADD && op != FP8_PRODUCE_ADD2 &&
        op != FP8_PRODUCE_MODULATE_FINITE)
        return FP8_ERR_ARG;
    // The cast of y: same rules as a bf16 cast of a contiguous [rows, cols].
    if (int e = check_cast(y, FP8_DTYPE_BF16, rows, cols, cols, scale, out)) return e;
    const bool reads_b = (op != FP8_PRODUCE_ADD);
    if (ldx < cols || lda < cols || (ldx % 8) != 0 || (lda % 8) != 0 ||
        (reads_b && (ldb < cols || (ldb % 8) != 0)))
        return FP8_ERR_SHAPE;
    const bool empty = (rows == 0 || cols == 0);
    if (!empty && (x == nullptr || a == nullptr || y == nullptr || (reads_b && b == nullptr)))
        return FP8_ERR_NULL;
    if ((x && !aligned16(x)) || (a && !aligned16(a)) || (reads_b && b && !aligned16(b)))
        return FP8_ERR_ALIGN;
    if (empty && out->scale_inv == nullptr) return FP8_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (empty) return status_of(launch_scale_inv_only(scale, out->scale_inv, noop_flag, s));
    return status_of(launch_produce_cast(op, x, ldx, a, lda, reads_b ? b : nullptr, ldb, y, rows,
                                         cols, scale, out->fmt, out->data, out->data_t, amax_cur,
                                         out->scale_inv, noop_flag, s));
}

int fp8_produce_modulate_backward(int32_t op, const uint16_t *dy, int64_t lddy,
                                  const uint16_t *x, int64_t ldx, const uint16_t *a, int64_t lda,
                                  const uint16_t *b, int64_t ldb, uint16_t *dx, int64_t lddx,
                                  uint16_t *da, int64_t ldda, uint16_t *db, int64_t lddb,
                                  int64_t rows, int64_t cols, fp8_stream_t stream) {
    if (op != FP8_PRODUCE_MODULATE && op != FP8_PRODUCE_MODULATE_FINITE) return FP8_ERR_ARG;
    if (rows < 0 || cols < 0 || (cols % 8) != 0) return FP8_ERR_SHAPE;
    for (int64_t ld : {lddy, ldx, lda, ldb, lddx, ldda, lddb})
        if (ld < cols || (ld % 8) != 0) return FP8_ERR_SHAPE;
    if (rows == 0 || cols == 0) return FP8_OK;
    if (rows > INT64_MAX / ldx) return FP8_ERR_SHAPE;
    if ((rows * (cols / 8) + 255) / 256 > (int64_t)UINT32_MAX) return FP8_ERR_SHAPE;
    for (const void *p : {(const void *)dy, (const void *)x, (const void *)a, (const void *)b,
                          (const void *)dx, (const void *)da, (const void *)db}) {
        if (p == nullptr) return FP8_ERR_NULL;
        if (!aligned16(p)) return FP8_ERR_ALIGN;
    }
    return status_of(launch_modulate_backward(op == FP8_PRODUCE_MODULATE_FINITE, dy, lddy, x, ldx,
                                              a, lda, b, ldb, dx, lddx, da, ldda, db, lddb, rows,
                                              cols, static_cast<hipStream_t>(stream)));
}

int fp8_cast_transpose_dynamic(const void *x, int32_t src, int64_t rows, int64_t cols,
                               int64_t ld, int32_t margin, float *scale, const fp8_tensor_t *out,
                               float *amax, const int32_t *noop_flag, fp8_stream_t stream) {
    if (int e = check_cast(x, src, rows, cols, ld, scale, out)) return e;
    if (margin < -126 || margin > 126) return FP8_ERR_ARG;
    if (amax == nullptr) return FP8_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // amax of x and the scale derived from it, then the ordinary cast with
    // that scale (no amax accumulation: the amax is already known).
    if (int e = status_of(launch_dynamic_scale(x, src, rows, cols, ld, out->fmt, margin, amax,
                                               scale, noop_flag, s)))
        return e;
    if (rows == 0 || cols == 0) {
        if (out->scale_inv == nullptr) return FP8_OK;
        return status_of(launch_scale_inv_only(scale, out->scale_inv, noop_flag, s));
    }
    return status_of(launch_cast_transpose_amax(x, src, rows, cols, ld, scale, out->fmt,
                                                out->data, out->data_t, nullptr, out->scale_inv,
                                                noop_flag, nullptr, 0, s));
}

// The split-product workspace of the *_ws entry points: a NULL workspace (any
// size) is no workspace; a non-NULL one must be 16-byte aligned, with a
// non-negative size.
static int check_gemm_ws(const void *ws, int64_t ws_bytes) {
    if (ws == nullptr) return FP8_OK;
    if (ws_bytes < 0) return FP8_ERR_ARG;
    return aligned16(ws) ? FP8_OK : FP8_ERR_ALIGN;
}

int64_t fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return FP8_ERR_SHAPE;
    int cus = 0;
    if (hipError_t e = current_cu_count(&cus)) return status_of(e);
    const int parts = gemm_split_parts(M, N, K, cus, INT64_MAX);
    return parts > 1 ? (int64_t)parts * M * N * (int64_t)sizeof(float) : 0;
}

static int linear_fwd(const fp8_tensor_t *x, const fp8_tensor_t *w, const uint16_t *bias,
                      uint16_t *y, void *ws, int64_t ws_bytes, fp8_stream_t stream) {
    if (!x || !w) return FP8_ERR_NULL;
    if (!valid_fmt(x->fmt) || !valid_fmt(w->fmt)) return FP8_ERR_FORMAT;
    const int64_t M = x->rows, K = x->cols, N = w->rows;
    if (w->cols != K) return FP8_ERR_SHAPE;
    if (int e = check_gemm(x->data, w->data, M, N, K, x->scale_inv, w->scale_inv, y, 8)) return e;
    if (M == 0 || N == 0) return FP8_OK;
    if (bias && !aligned16(bias)) return FP8_ERR_ALIGN;
    if (int e = check_gemm_ws(ws, ws_bytes)) return e;
    return status_of(launch_gemm_nt(x->data, x->fmt, w->data, w->fmt, M, N, K, x->scale_inv,
                                    w->scale_inv, bias, FP8_DTYPE_BF16, y,
                                    static_cast<hipStream_t>(stream), ws, ws_bytes));
}

int fp8_linear_fwd(const fp8_tensor_t *x, const fp8_tensor_t *w, const uint16_t *bias,
                   uint16_t *y, fp8_stream_t stream) {
    return linear_fwd(x, w, bias, y, nullptr, 0, stream);
}

int fp8_linear_fwd_ws(const fp8_tensor_t *x, const fp8_tensor_t *w, const uint16_t *bias,
                      uint16_t *y, void *workspace, int64_t workspace_bytes,
                      fp8_stream_t stream) {
    return linear_fwd(x, w, bias, y, workspace, workspace_bytes, stream);
}

int fp8_linear_fwd_fp8out(const fp8_tensor_t *x, const fp8_tensor_t *w, const uint16_t *bias,
                          const float *scale_y, const fp8_tensor_t *y, float *amax_y,
                          fp8_stream_t stream) {
    if (!x || !w || !y || !scale_y) return FP8_ERR_NULL;
    if (!valid_fmt(x->fmt) || !valid_fmt(w->fmt) || !valid_fmt(y->fmt)) return FP8_ERR_FORMAT;
    if (y->reserved != 0 || y->data_t != nullptr) return FP8_ERR_ARG;
    const int64_t M = x->rows, K = x->cols, N = w->rows;
    if (w->cols != K || y->rows != M || y->cols != N) return FP8_ERR_SHAPE;
    if (int e = check_gemm(x->data, w->data, M, N, K, x->scale_inv, w->scale_inv, y->data, 16))
        return e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (M == 0 || N == 0) {
        // No output: the amax is untouched; the snapshot is still taken.
        if (y->scale_inv == nullptr) return FP8_OK;
        return status_of(launch_scale_inv_only(scale_y, y->scale_inv, nullptr, s));
    }
    if (bias && !aligned16(bias)) return FP8_ERR_ALIGN;
    return status_of(launch_gemm_nt_fp8out(x->data, x->fmt, w->data, w->fmt, M, N, K,
                                           x->scale_inv, w->scale_inv, bias, y->fmt, scale_y,
                                           y->data, amax_y, y->scale_inv, s));
}

static int linear_dgrad(const fp8_tensor_t *dy, const fp8_tensor_t *w, uint16_t *dx, void *ws,
                        int64_t ws_bytes, fp8_stream_t stream) {
    if (!dy || !w) return FP8_ERR_NULL;
    if (!valid_fmt(dy->fmt) || !valid_fmt(w->fmt)) return FP8_ERR_FORMAT;
    // dx [M, K] = dy [M, N] . (w_t [K, N])^T
    const int64_t M = dy->rows, N = dy->cols, K = w->cols;
    if (w->rows != N) return FP8_ERR_SHAPE;
    if (int e = check_gemm(dy->data, w->data_t, M, K, N, dy->scale_inv, w->scale_inv, dx, 8))
        return e;
    if (M == 0 || K == 0) return FP8_OK;
    if (int e = check_gemm_ws(ws, ws_bytes)) return e;
    return status_of(launch_gemm_nt(dy->data, dy->fmt, w->data_t, w->fmt, M, K, N, dy->scale_inv,
                                    w->scale_inv, nullptr, FP8_DTYPE_BF16, dx,
                                    static_cast<hipStream_t>(stream), ws, ws_bytes));
}

int fp8_linear_dgrad(const fp8_tensor_t *dy, const fp8_tensor_t *w, uint16_t *dx,
                     fp8_stream_t stream) {
    return linear_dgrad(dy, w, dx, nullptr, 0, stream);
}

int fp8_linear_dgrad_ws(const fp8_tensor_t *dy, const fp8_tensor_t *w, uint16_t *dx,
                        void *workspace, int64_t workspace_bytes, fp8_stream_t stream) {
    return linear_dgrad(dy, w, dx, workspace, workspace_bytes, stream);
}

static int linear_wgrad(const fp8_tensor_t *dy, const fp8_tensor_t *x, void *dw,
                        int32_t out_dtype, void *ws, int64_t ws_bytes, fp8_stream_t stream) {
    if (!dy || !x) return FP8_ERR_NULL;
    if (!valid_fmt(dy->fmt) || !valid_fmt(x->fmt)) return FP8_ERR_FORMAT;
    if (out_dtype != FP8_DTYPE_BF16 && out_dtype != FP8_DTYPE_FP32) return FP8_ERR_ARG;
    // dw [N, K] = dy_t [N, M] . (x_t [K, M])^T
    const int64_t M = dy->rows, N = dy->cols, K = x->cols;
    if (x->rows != M) return FP8_ERR_SHAPE;
    if (int e = check_gemm(dy->data_t, x->data_t, N, K, M, dy->scale_inv, x->scale_inv, dw,
                           out_dtype == FP8_DTYPE_BF16 ? 8 : 4))
        return e;
    if (N == 0 || K == 0) return FP8_OK;
    if (int e = check_gemm_ws(ws, ws_bytes)) return e;
    return status_of(launch_gemm_nt(dy->data_t, dy->fmt, x->data_t, x->fmt, N, K, M,
                                    dy->scale_inv, x->scale_inv, nullptr, out_dtype, dw,
                                    static_cast<hipStream_t>(stream), ws, ws_bytes));
}

int fp8_linear_wgrad(const fp8_tensor_t *dy, const fp8_tensor_t *x, void *dw, int32_t out_dtype,
                     fp8_stream_t stream) {
    return linear_wgrad(dy, x, dw, out_dtype, nullptr, 0, stream);
}

int fp8_linear_wgrad_ws(const fp8_tensor_t *dy, const fp8_tensor_t *x, void *dw,
                        int32_t out_dtype, void *workspace, int64_t workspace_bytes,
                        fp8_stream_t stream) {
    return linear_wgrad(dy, x, dw, out_dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"
