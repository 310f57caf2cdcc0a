// Per-tensor-scaled FP8 GEMM, "NT" layout, on CDNA4 FP8 matrix cores.
//
//   C[i, j] = out( (sum_k dec(A[i, k]) * dec(B[j, k])) * sinv_a * sinv_b + bias[j] )
//
// out is bf16 or fp32 rounding, or (OUT_E4M3 / OUT_E5M2) the FP8 cast of the
// fp32 value with the output's own scale, together with the amax of the
// unscaled output: torch._scaled_mm called with an FP8 out_dtype returns that
// amax beside the FP8 output.
//
// This is torch._scaled_mm of "Accelerating PyTorch Training Workloads with
// FP8 -- Part 2" (row-major first operand, transposed second operand,
// per-tensor scales held on the device, optional bf16 bias), used for the
// forward, dgrad and wgrad products of te.Linear ("CPU Overhead of te.Linear
// FP8 Layers").  Every FP8 x FP8 product is exact; the matrix core adds them
// in groups of eight consecutive K positions aligned to the group's largest
// product, dropping bits more than 13 binades below it (measured on gfx950:
// a group loses less than 2^-10 of its largest product), and accumulates the
// group sums in fp32.
//
// Design (gfx950, wave64).  Four kernels; launch_fmt picks one per call:
//
//   * gemm_nt_dma_kernel -- every large product (256^3 outputs or more, or
//     at least three quarters of a 256 x 256 tile per CU) with K % 128 == 0
//     (all the toy-block shapes at 8192 tokens).  Persistent: one 256-thread workgroup per CU walks
//     256 x 256 output tiles in an XCD-aware order (workgroup b runs on XCD
//     b % 8, and each XCD gets a contiguous, row-grouped range of tiles).
//     Four waves own 128 x 128 each as 4 x 4 v_mfma_f32_32x32x64_f8f6f4
//     blocks (256 fp32 accumulators per lane).  Operand stages of 128
//     K-bytes are written straight into two 64 KiB LDS buffers by buffer
//     loads with the LDS flag (no staging registers), and stages stream on
//     across tile boundaries.  The bf16 / fp32 epilogue writes the raw fp32
//     accumulators straight from the accumulator registers into the drained
//     stage buffer in half-blocks (32 rows x 64 columns), reads them back as
//     row segments, applies sinv_a * sinv_b and the bias and stores whole
//     row segments; it starts inside the last stage, between its MFMAs, and
//     runs while the next tile's first stages are in flight.
//   * gemm_nt_big_kernel -- the same tiling for large products whose K is a
//     multiple of 16 only: 64-byte stages in three LDS buffers, loaded
//     through registers, K tails read as zero through the buffer range check.
//   * gemm_nt_sdma_kernel -- small products with K % 128 == 0 and 32-bit
//     operand offsets: 128 x 128 tiles (64 x 128 when there would be no
//     more tiles than CUs), one workgroup per tile, v_mfma_f32_16x16x128_f8f6f4,
//     operand stages written into LDS by buffer loads with the LDS flag, two
//     or three stages in flight.
//   * gemm_nt_kernel -- the other small products (K tails, K = 128, 64-bit
//     offsets): the same tiles with loads staged through registers,
//     double-buffered LDS.
//   * The split form: gemm_nt_dma_kernel over (tile, K part) units writing
//     raw fp32 sums to a caller workspace, then splitk_reduce_kernel, for
//     products with few tiles and a long contraction (gemm_split_parts).
//
// Shared by all four: LDS rows are 128 bytes with the 16-byte chunk c of row
// r stored at a row-dependent XOR of c (conflict-free fragment reads); the B
// fragment is the matrix core's first operand, so each lane holds four
// consecutive output columns of one output row; out-of-range operand rows
// are clamped for loading (or read as zero through a buffer range) and
// never stored.
//
// The kernels and their launch templates live in this header; the library's
// sources instantiate them per output kind (bf16 / fp32, FP8 codes) so that
// the two sets compile in parallel.
#pragma once

#include <algorithm>
#include <type_traits>

#include "fp8_codec.h"
#include "fp8dsl_internal.h"

namespace fp8dsl {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 128;

// Output kinds beyond FP8_DTYPE_BF16 / FP8_DTYPE_FP32: FP8 codes.
constexpr int OUT_E4M3 = 2;
constexpr int OUT_E5M2 = 3;
template <int OUT>
constexpr bool is_q_out() { return OUT == OUT_E4M3 || OUT == OUT_E5M2; }
template <int OUT>
constexpr int q_fmt() { return OUT == OUT_E5M2 ? FP8_E5M2 : FP8_E4M3; }

// FP8 output of the product: codes = cast(v, *scale) with v = acc * s + bias
// in fp32; *amax folds in max |v| of the UNSCALED output (one atomic per
// workgroup); workgroup 0 writes *scale_inv = 1 / *scale.  amax and
// scale_inv may be null.  Unused for bf16 / fp32 output.
struct QOut {
    const float *scale;
    float *amax;
    float *scale_inv;
};

// IEEE 754-2019 maximum: NaN if either input is NaN (v_maximum3_f32 on
// gfx950, which takes |x| as a source modifier).
__device__ __forceinline__ float nan_max(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}

// Codes of four consecutive outputs (byte i = y_i); their amax key (the
// bits of max |y|, a NaN above inf's) is folded into `key`.
template <int OUT>
__device__ __forceinline__ uint32_t encode_out4(float y0, float y1, float y2, float y3, float so,
                                                bool so_special, uint32_t &key) {
    const uint32_t k = __float_as_uint(
        nan_max(nan_max(nan_max(fabsf(y0), fabsf(y1)), fabsf(y2)), fabsf(y3)));
    key = max(key, k);
    uint32_t w = encode4<q_fmt<OUT>()>(y0, y1, y2, y3, so);
    if (so_special || k > 0x7F800000u) {
        const float x[4] = {y0, y1, y2, y3};
        w = patch_nan4(w, x, so);
    }
    return w;
}

// True when the output scale is 0, inf or NaN: every product may be NaN.
__device__ __forceinline__ bool scale_is_special(float so) {
    return !(fabsf(so) > 0.0f && fabsf(so) <= 3.402823466e38f);
}

// An output scale that can be folded into the epilogue's multiply-add
// (v * so computed as acc * (s * so) + bias * so) without leaving fp32's
// comfortable range; any other scale takes the cast's own order.
__device__ __forceinline__ bool scale_is_foldable(float so) {
    return fabsf(so) >= 0x1p-60f && fabsf(so) <= 0x1p60f;
}

// End of a 256-thread workgroup with an FP8 output: one atomic max of the
// lanes' amax keys into *amax (which holds a non-negative value or NaN), and
// the scale-inverse snapshot from workgroup 0.  With `scaled_key` the keys
// are of |v * so| and the amax is recovered as max |v * so| / |so|.  `red`
// is 16 bytes of LDS that no wave reads any more; every thread calls this.
__device__ __forceinline__ void finish_q_out(uint32_t key, const QOut &qo, float so,
                                             uint32_t *red, bool scaled_key = false) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) key = max(key, (uint32_t)__shfl_xor((int)key, off, 64));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t k = max(max(red[0], red[1]), max(red[2], red[3]));
        if (scaled_key && k <= 0x7F800000u) k = __float_as_uint(__uint_as_float(k) / fabsf(so));
        if (qo.amax != nullptr) {
            unsigned int *a = reinterpret_cast<unsigned int *>(qo.amax);
            if (k > __atomic_load_n(a, __ATOMIC_RELAXED)) atomicMax(a, k);
        }
        if (blockIdx.x == 0 && qo.scale_inv != nullptr) *qo.scale_inv = 1.0f / so;
    }
}

// Tile index of workgroup b.  Workgroups are dealt round-robin to the eight
// XCDs (b % 8); when the tile count allows, each XCD gets a contiguous range
// of tiles, walked in groups of GROUP_M tile rows, so that the workgroups
// sharing an XCD's L2 also share A and B slabs.
__device__ __forceinline__ void tile_of_block(int b, int tiles_m, int tiles_n, int &tm, int &tn) {
    constexpr int XCDS = 8;
    constexpr int GROUP_M = 4;
    const int T = tiles_m * tiles_n;
    int t = b;
    if (T % XCDS == 0) t = (b % XCDS) * (T / XCDS) + b / XCDS;
    const int per_group = GROUP_M * tiles_n;
    const int g = t / per_group;
    const int first_m = g * GROUP_M;
    const int rows_here = min(GROUP_M, tiles_m - first_m);
    const int r = t - g * per_group;
    tm = first_m + r % rows_here;
    tn = r / rows_here;
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, bool HAS_BIAS>
__global__ __launch_bounds__(WM *WN * 64) void gemm_nt_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, int M, int N, int K,
    const float *__restrict__ sinv_a, const float *__restrict__ sinv_b,
    const uint16_t *__restrict__ bias, void *__restrict__ Cv, int tiles_m, int tiles_n, QOut qo) {
    static_assert(!is_q_out<OUT>() || WM * WN == 4, "the FP8 output reduces over four waves");
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM;            // wave tile rows
    constexpr int WTN = BN / WN;            // wave tile cols
    constexpr int FM = WTM / 16;
    constexpr int FN = WTN / 16;
    constexpr int A_CHUNKS = BM * BK / 16;  // 16-byte chunks per stage
    constexpr int B_CHUNKS = BN * BK / 16;
    constexpr int LA = A_CHUNKS / NT;
    constexpr int LB = B_CHUNKS / NT;
    static_assert(A_CHUNKS % NT == 0 && B_CHUNKS % NT == 0, "loader shape");
    constexpr int STAGE = (BM + BN) * BK;

    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;

    int tile_m, tile_n;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN;

    // Loader bookkeeping: chunk id = tid + i*NT -> (row = id / 8, kc = id % 8).
    // Rows past M (N) are clamped to the last row: loaded, never stored.
    const uint8_t *a_src[LA];
    const uint8_t *b_src[LB];
    int a_lds[LA], b_lds[LB];
    const int kc16 = (tid & 7) * 16;        // same K chunk for every i (NT % 8 == 0)
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int id = tid + i * NT;
        const int row = id >> 3, kc = id & 7;
        const int grow = min(m0 + row, M - 1);
        a_src[i] = A + (int64_t)grow * K + kc * 16;
        a_lds[i] = row * BK + ((kc ^ (row & 7)) << 4);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int id = tid + i * NT;
        const int row = id >> 3, kc = id & 7;
        const int grow = min(n0 + row, N - 1);
        b_src[i] = B + (int64_t)grow * K + kc * 16;
        b_lds[i] = BM * BK + row * BK + ((kc ^ (row & 7)) << 4);
    }

    u32x4 ra[LA], rb[LB];
    // Full K step: unconditional 16-byte loads.
    auto load_full = [&](int k0) {
#pragma unroll
        for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4 *>(a_src[i] + k0);
#pragma unroll
        for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4 *>(b_src[i] + k0);
    };
    // Last, partial K step: chunks at or past K read as zero (the address is
    // pulled back in range and the value discarded).
    auto load_tail = [&](int k0) {
        const bool in = k0 + kc16 < K;
        const int k = in ? k0 : 0;
#pragma unroll
        for (int i = 0; i < LA; ++i) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(a_src[i] + k);
            ra[i] = in ? v : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(b_src[i] + k);
            rb[i] = in ? v : u32x4{0, 0, 0, 0};
        }
    };
    auto store_lds = [&](int stage) {
        uint8_t *base = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4 *>(base + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < LB; ++i) *reinterpret_cast<u32x4 *>(base + b_lds[i]) = rb[i];
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Fragment addressing: lane holds row (lane % 16) of a 16-row fragment and
    // the 32 K-bytes of chunks 2*(lane/16) and 2*(lane/16)+1.
    const int frow = lane & 15;
    const int fc0 = (lane >> 4) * 2;
    const int sw = frow & 7;   // fragment bases are multiples of 16 rows
    const int off0 = ((fc0 ^ sw) << 4);
    const int off1 = (((fc0 + 1) ^ sw) << 4);

    const int nk = (K + BK - 1) / BK;
    const int nfull = K / BK;               // steps with no K tail
    if (nk > 0) {
        if (nfull > 0) load_full(0); else load_tail(0);
        store_lds(0);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int stage = kt & 1;
        if (kt + 1 < nfull) load_full((kt + 1) * BK);
        else if (kt + 1 < nk) load_tail((kt + 1) * BK);

        const uint8_t *As = lds + stage * STAGE + (wm * WTM + frow) * BK;
        const uint8_t *Bs = lds + stage * STAGE + BM * BK + (wn * WTN + frow) * BK;
        v8i bf[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(Bs + j * 16 * BK + off0);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(Bs + j * 16 * BK + off1);
            bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(As + i * 16 * BK + off0);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(As + i * 16 * BK + off1);
            const v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
            for (int j = 0; j < FN; ++j)
                // B fragment first: lane (l%16, l/16) receives output row
                // (l%16) of the A fragment, columns 4*(l/16) .. +3.
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bf[j], af, acc[i][j], FB, FA, 0, 0, 0, 0);
        }

        if (kt + 1 < nk) store_lds(stage ^ 1);
        __syncthreads();
    }

    // Epilogue.
    const float s = (*sinv_a) * (*sinv_b);
    float so = 0.f;
    bool so_special = false;
    if constexpr (is_q_out<OUT>()) {
        so = *qo.scale;
        so_special = scale_is_special(so);
    }
    uint32_t key = 0;
    const int orow = lane & 15;
    const int ocol = (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int gc = n0 + wn * WTN + j * 16 + ocol;
        if (gc >= N) continue;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (HAS_BIAS) {
            const u32x2 b2 = *reinterpret_cast<const u32x2 *>(bias + gc);
            bv[0] = __uint_as_float(b2.x << 16);
            bv[1] = __uint_as_float(b2.x & 0xFFFF0000u);
            bv[2] = __uint_as_float(b2.y << 16);
            bv[3] = __uint_as_float(b2.y & 0xFFFF0000u);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int gr = m0 + wm * WTM + i * 16 + orow;
            if (gr >= M) continue;
            const v4f a = acc[i][j];
            const float y0 = a.x * s + bv[0];
            const float y1 = a.y * s + bv[1];
            const float y2 = a.z * s + bv[2];
            const float y3 = a.w * s + bv[3];
            if constexpr (OUT == FP8_DTYPE_BF16) {
                uint16_t *C = static_cast<uint16_t *>(Cv);
                const bf16x4 o = {(__bf16)y0, (__bf16)y1, (__bf16)y2, (__bf16)y3};
                *reinterpret_cast<bf16x4 *>(C + (int64_t)gr * N + gc) = o;
            } else if constexpr (is_q_out<OUT>()) {
                uint8_t *C = static_cast<uint8_t *>(Cv);
                *reinterpret_cast<uint32_t *>(C + (int64_t)gr * N + gc) =
                    encode_out4<OUT>(y0, y1, y2, y3, so, so_special, key);
            } else {
                float *C = static_cast<float *>(Cv);
                *reinterpret_cast<v4f *>(C + (int64_t)gr * N + gc) = v4f{y0, y1, y2, y3};
            }
        }
    }
    if constexpr (is_q_out<OUT>()) finish_q_out(key, qo, so, reinterpret_cast<uint32_t *>(lds));
}

// Epilogue of one wave's 128 x 128 accumulator tile, 4 x 4 fragments of
// v_mfma_f32_32x32x64 with the B fragment passed first: lane l holds output
// row r0 + 32 i + l % 32 of fragment row block i and, for register group g
// (registers 4g .. 4g+3) of fragment column block j, the four consecutive
// columns c0 + 32 j + 8 g + 4 (l / 32) .. +3.  Writes out(acc * s + bias) for
// the in-range elements as one 8-byte (bf16), 16-byte (fp32) or 4-byte (FP8
// codes, scale so, amax key folded into `key`) vector per row and group
// (N % 8 == 0 keeps every vector inside the row), then clears the
// accumulators for the next tile.
template <int OUT, bool HAS_BIAS>
__device__ __forceinline__ void store_wave_tile(v16f (&acc)[4][4], void *__restrict__ Cv,
                                                const uint16_t *__restrict__ bias, int M, int N,
                                                int r0, int c0, int lane, float s, float so,
                                                bool so_special, uint32_t &key) {
    const int frow = lane & 31;
    const int half = lane >> 5;
    // All bias loads first (one latency, not sixteen); columns past N read
    // as zero through the descriptor's range check.
    u32x2 bq[4][4];
    if constexpr (HAS_BIAS) {
        const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(bias), (short)0, 2 * N, 0x00020000);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                bq[j][g] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                    brs, 2 * (c0 + j * 32 + 8 * g + 4 * half), 0, 0));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int gc = c0 + j * 32 + 8 * g + 4 * half;
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (HAS_BIAS) {
                const u32x2 b2 = bq[j][g];
                bv[0] = __uint_as_float(b2.x << 16);
                bv[1] = __uint_as_float(b2.x & 0xFFFF0000u);
                bv[2] = __uint_as_float(b2.y << 16);
                bv[3] = __uint_as_float(b2.y & 0xFFFF0000u);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int gr = r0 + i * 32 + frow;
                const float y0 = acc[i][j][4 * g + 0] * s + bv[0];
                const float y1 = acc[i][j][4 * g + 1] * s + bv[1];
                const float y2 = acc[i][j][4 * g + 2] * s + bv[2];
                const float y3 = acc[i][j][4 * g + 3] * s + bv[3];
                if (gr < M && gc < N) {
                    if constexpr (OUT == FP8_DTYPE_BF16) {
                        uint16_t *C = static_cast<uint16_t *>(Cv);
                        const bf16x4 o = {(__bf16)y0, (__bf16)y1, (__bf16)y2, (__bf16)y3};
                        *reinterpret_cast<bf16x4 *>(C + (int64_t)gr * N + gc) = o;
                    } else if constexpr (is_q_out<OUT>()) {
                        uint8_t *C = static_cast<uint8_t *>(Cv);
                        *reinterpret_cast<uint32_t *>(C + (int64_t)gr * N + gc) =
                            encode_out4<OUT>(y0, y1, y2, y3, so, so_special, key);
                    } else {
                        float *C = static_cast<float *>(Cv);
                        *reinterpret_cast<v4f *>(C + (int64_t)gr * N + gc) = v4f{y0, y1, y2, y3};
                    }
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
}

// Large-problem kernel: persistent, one 256-thread workgroup per CU.
//
//   * Each workgroup walks the 256 x 256 output tiles blockIdx.x,
//     blockIdx.x + gridDim.x, ... as one continuous stream of 64-byte K
//     stages, so the loads of the next tile's first stages are already in
//     flight while the current tile's epilogue runs.
//   * Four waves (one per SIMD) of 128 x 128, each a 4 x 4 grid of
//     v_mfma_f32_32x32x64_f8f6f4 tiles (this instruction runs measurably
//     faster per FLOP on gfx950 than 16x16x128); 256 fp32 accumulators per
//     lane in AGPRs.
//   * Stages live in three LDS buffers.  With one wave per SIMD nothing else
//     can issue matrix-core work while a wave sits in a memory instruction,
//     so every memory instruction of a stage is threaded between its 16
//     matrix-core instructions:
//        slots 0-7  : MFMA, then one LDS write committing stage k+2 and one
//                     buffer load fetching stage k+3 into registers;
//        barrier    : stage k+2 is in LDS for everyone;
//        slots 8-15 : MFMA, then two LDS reads of stage k+1's fragments
//                     (double-buffered fragment registers).
//     Three buffers make one barrier per stage enough: stage k+2 overwrites
//     the buffer of stage k-1, whose fragments were read before the previous
//     barrier.  The loop has no data-dependent branches, so the compiler's
//     wait counters stay exact (a conditional memory instruction makes it
//     fall back to waiting for everything).
//   * Operands come in with buffer loads (an SGPR descriptor per operand, a
//     32-bit offset per lane); rows past M or N, K past the end and stages
//     past the last tile fall outside the descriptor and read as zero.
//   * LDS rows are 64 bytes; 16-byte chunk c of row r sits at chunk
//     c ^ ((r >> 1) & 3) ^ (3 * ((r >> 3) & 1)): fragment reads (lanes on
//     consecutive rows) and staging writes (4 lanes per row) are free of bank
//     conflicts with 32 or with 64 banks.
//
// Fragment layout of v_mfma_f32_32x32x64_f8f6f4: lane l holds row l % 32 and
// 32 K-bytes of half (l / 32) of the 64-byte K slice; A and B use the same
// K assignment, so any consistent choice of bytes gives the same sum.  With
// the B fragment passed first, lane l ends up with output row l % 32 and, for
// register r, output column 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ int big_swz(int r) { return ((r >> 1) & 3) ^ (3 * ((r >> 3) & 1)); }

template <int FA, int FB, int OUT, bool HAS_BIAS>
__global__ __launch_bounds__(256) void gemm_nt_big_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, int M, int N, int K,
    const float *__restrict__ sinv_a, const float *__restrict__ sinv_b,
    const uint16_t *__restrict__ bias, void *__restrict__ Cv, int tiles_m, int tiles_n, QOut qo) {
    constexpr int BM = 256, BN = 256;
    constexpr int KS = 64;                  // K bytes per stage
    constexpr int WT = 128;                 // wave tile (square)
    constexpr int F = WT / 32;              // 4 x 4 fragments of 32 x 32
    constexpr int LPT = BM * KS / 16 / 256; // 4 chunk loads per thread per operand
    constexpr int STAGE = (BM + BN) * KS;   // 32 KiB
    constexpr int OOB = 0x7FFFFFF0;         // an offset outside every descriptor
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int T = tiles_m * tiles_n;
    if ((int)blockIdx.x >= T) return;
    const int my_tiles = (T - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    const __amdgpu_buffer_rsrc_t ra_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(A), (short)0, M * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(B), (short)0, N * K, 0x00020000);

    // Loader: thread -> (row = tid/4 + 64 i, chunk kc = tid % 4) of a stage;
    // the 8 chunk loads of a stage alternate A, B, A, B, ...
    const int kc = tid & 3;
    const int lrow = tid >> 2;
    const int rowstep = 64 * K;
    const int st_off = lrow * KS + ((kc ^ big_swz(lrow)) << 4);   // + 4096 i (swizzle repeats)
    // Per-lane operand offsets of tile number r of this workgroup (OOB when
    // r is past its last tile).
    auto tile_offsets = [&](int r, int &oa, int &ob) {
        if (r < my_tiles) {
            int tm, tn;
            tile_of_block((int)blockIdx.x + r * (int)gridDim.x, tiles_m, tiles_n, tm, tn);
            oa = (tm * BM + lrow) * K + kc * 16;
            ob = (tn * BN + lrow) * K + kc * 16;
        } else {
            oa = OOB;
            ob = OOB;
        }
    };

    u32x4 reg[2][2 * LPT];                  // two staging sets of one stage
    // Load chunk q of a stage whose per-lane base offsets are (oa, ob), K
    // byte offset k0, into staging set `set`.
    auto load_one = [&](int set, int q, int oa, int ob, int k0) {
        const bool in = k0 + kc * 16 < K;
        const int i = q >> 1;
        if (q & 1) {
            const int o = (in && ob != OOB) ? ob + i * rowstep + k0 : OOB;
            reg[set][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb_rsrc, o, 0, 0));
        } else {
            const int o = (in && oa != OOB) ? oa + i * rowstep + k0 : OOB;
            reg[set][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, o, 0, 0));
        }
    };
    auto store_one = [&](int set, int q, int buf_off) {
        const int i = q >> 1;
        uint8_t *dst = lds + buf_off + st_off + 4096 * i + ((q & 1) ? BM * KS : 0);
        *reinterpret_cast<u32x4 *>(dst) = reg[set][q];
    };

    // Fragment reads: row (lane % 32) of each 32-row fragment, chunks
    // 2*(lane/32) and +1.
    const int frow = lane & 31;
    const int fsw = big_swz(frow);
    const int c0 = 2 * (lane >> 5);
    const int fo0 = frow * KS + ((c0 ^ fsw) << 4);
    const int fo1 = frow * KS + (((c0 + 1) ^ fsw) << 4);
    const int a_fbase = wm * WT * KS;
    const int b_fbase = BM * KS + wn * WT * KS;

    v8i af[2][F], bf[2][F];
    auto read_half = [&](v8i &dst, int off, int h) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + off + (h ? fo1 : fo0));
        if (h == 0) { dst[0] = (int)v.x; dst[1] = (int)v.y; dst[2] = (int)v.z; dst[3] = (int)v.w; }
        else        { dst[4] = (int)v.x; dst[5] = (int)v.y; dst[6] = (int)v.z; dst[7] = (int)v.w; }
    };

    v16f acc[F][F];
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Stages per tile, padded to even (a padded stage lies past K and adds
    // nothing); the caller guarantees nk >= 4, so stage k+3 is in this tile
    // or the next one.
    const int nk = ((K + KS - 1) / KS + 1) & ~1;

    int cur_a, cur_b, nxt_a, nxt_b;         // tile offsets: this tile, next tile
    tile_offsets(0, cur_a, cur_b);
    tile_offsets(1, nxt_a, nxt_b);

    // Prologue: stages 0 and 1 committed, stage 2 in flight (set 0), the
    // fragments of stage 0 in registers.
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int q = 0; q < 2 * LPT; ++q) load_one(p, q, cur_a, cur_b, p * KS);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int q = 0; q < 2 * LPT; ++q) store_one(p, q, p * STAGE);
#pragma unroll
    for (int q = 0; q < 2 * LPT; ++q) load_one(0, q, cur_a, cur_b, 2 * KS);
    __syncthreads();
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            read_half(af[0][f], a_fbase + f * 32 * KS, h);
            read_half(bf[0][f], b_fbase + f * 32 * KS, h);
        }

    const float s = (*sinv_a) * (*sinv_b);
    float so = 0.f;
    bool so_special = false;
    if constexpr (is_q_out<OUT>()) {
        so = *qo.scale;
        so_special = scale_is_special(so);
    }
    uint32_t key = 0;
    int buf_next = STAGE;            // buffer of stage k+1
    int buf_commit = 2 * STAGE;      // buffer of stage k+2

    for (int r = 0; r < my_tiles; ++r) {
        for (int kt = 0; kt < nk; kt += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int k = kt + u;
                const int cur = u, nxt = u ^ 1;
                // Stage k+3: this tile, or the next tile's stage k+3-nk.
                const bool same = k + 3 < nk;
                const int ia = same ? cur_a : nxt_a;
                const int ib = same ? cur_b : nxt_b;
                const int ik = (same ? k + 3 : k + 3 - nk) * KS;
#pragma unroll
                for (int slot = 0; slot < 16; ++slot) {
                    const int i = slot >> 2, j = slot & 3;
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bf[cur][j], af[cur][i], acc[i][j], FB, FA, 0, 0, 0, 0);
                    if (slot < 8) {
                        store_one(cur, slot, buf_commit);        // stage k+2: set k%2
                        load_one(nxt, slot, ia, ib, ik);         // stage k+3 -> set (k+1)%2
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // LDS write
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
                        if (slot == 7) __syncthreads();
                    } else {
                        // Stage k+1's fragments, in the order the next stage's
                        // first MFMAs need them: A0, B0..B3, A1..A3.
                        const int f = slot - 8;
                        if (f >= 1 && f <= 4) {
                            read_half(bf[nxt][f - 1], buf_next + b_fbase + (f - 1) * 32 * KS, 0);
                            read_half(bf[nxt][f - 1], buf_next + b_fbase + (f - 1) * 32 * KS, 1);
                        } else {
                            const int a = (f == 0) ? 0 : f - 4;
                            read_half(af[nxt][a], buf_next + a_fbase + a * 32 * KS, 0);
                            read_half(af[nxt][a], buf_next + a_fbase + a * 32 * KS, 1);
                        }
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 LDS reads
                    }
                }
                // Rotate the three buffers: next <- commit, commit <- current.
                const int buf_cur = (buf_next == 0) ? 2 * STAGE : buf_next - STAGE;
                buf_next = buf_commit;
                buf_commit = buf_cur;
            }
        }

        int tm, tn;
        tile_of_block((int)blockIdx.x + r * (int)gridDim.x, tiles_m, tiles_n, tm, tn);
        store_wave_tile<OUT, HAS_BIAS>(acc, Cv, bias, M, N, tm * BM + wm * WT, tn * BN + wn * WT,
                                       lane, s, so, so_special, key);
        // The next tile becomes current; look one further ahead.
        cur_a = nxt_a;
        cur_b = nxt_b;
        tile_offsets(r + 2, nxt_a, nxt_b);
    }
    if constexpr (is_q_out<OUT>()) finish_q_out(key, qo, so, reinterpret_cast<uint32_t *>(lds));
}

// One 16-byte-per-lane load from global memory straight into LDS: lane l's
// 16 bytes at byte offset `voff` of the buffer land at LDS address
// m0 + 16 l, so one instruction fills 1 KiB of LDS in lane order.  Offsets
// at or past the descriptor's record count read as zero and move no data.
// Issued from inline assembly so that the compiler neither waits for it
// before unrelated LDS reads nor tracks it at all: the kernel that uses it
// places every vmcnt wait itself (nothing else in that kernel touches M0;
// gfx9 LDS instructions do not read it).  An SALU write of M0 needs one wait
// state before an LDS-DMA load reads it, hence the s_nop.
__device__ __forceinline__ void dma_b128(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voff), "s"(rsrc) : "memory");
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 128-byte-row LDS swizzle: chunk c (16 bytes) of row r sits at chunk
// c ^ dma_swz(r).  Fragment reads touch 16 consecutive rows at one logical
// chunk per 256-byte LDS cycle (or 8 rows per 128 bytes): the rows' (r & 1,
// chunk) pairs are all distinct, so neither layout has bank conflicts.
__device__ __forceinline__ int dma_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Output stores of the LDS-DMA kernel go through a buffer resource over the
// wave's 128 output rows r0 .. r0 + 127 (those below M): a store at an
// offset at or past the resource's size is dropped by the hardware.  So
// every store instruction is issued whatever the tails, and the kernel can
// count them in its vmcnt waits.  Column groups past N take OUT_OOB.  The
// host guarantees 128 * N * EB < 2^31.
constexpr uint32_t OUT_OOB = 0x80000000u;
// They are non-temporal (the nt cache-policy bit).  With normal
// stores a product's output stays dirty in the last-level cache and is
// written back while the next memory-bound kernel streams its own bytes
// (measured on MI355X: the E5M2 cast of an [8192, 8192] gradient takes 62 us
// after a forward product of [8192, 8192] bf16 outputs and 49 us with
// non-temporal output stores).  The product, compute-bound, pays for its own
// writes instead, but less: one linear's forward + backward step is 4%
// faster and a 32-block forward 3%.
constexpr int OUT_POLICY = 2;
template <int EB>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rows_rsrc(void *C, int M, int N, int r0) {
    // Every input is wave-uniform, but the clamp compiles to a vector
    // instruction; without readfirstlane the resource would sit in vector
    // registers and the compiler would loop over its values at every store.
    const int rows = min(128, max(0, M - r0));
    const int nrec = __builtin_amdgcn_readfirstlane(rows * N * EB);
    return __builtin_amdgcn_make_buffer_rsrc(static_cast<uint8_t *>(C) + (int64_t)r0 * N * EB,
                                             (short)0, nrec, 0x00020000);
}

// bf16 / fp32 epilogue of the LDS-DMA kernel, in half-blocks.  A wave's
// 128 x 128 tile is eight half-blocks h = 2 i + p: fragment row block i
// (tile rows 32 i .. 32 i + 31) and fragment columns 2 p, 2 p + 1 (tile
// columns 64 p .. 64 p + 63).  A half-block is staged as the raw fp32
// accumulators, 32 rows of 256 bytes (8 KiB), 16-byte chunk c of row q at
// chunk c ^ (q & 15); the wave's 16 KiB staging quarter holds two (regions
// h % 2).  The swizzle makes both the matrix-core-layout writes and the row
// reads conflict-free (16 lanes per LDS cycle touch 16 distinct chunks).
//
// stage_hb writes half-block h straight from the accumulator registers (the
// LDS store reads them; no register reads, no arithmetic): lane l holds row
// l % 32 and, per register group g of fragment column j, the four columns
// 32 j + 8 g + 4 (l / 32) .. +3, i.e. chunk 8 (j - 2 p) + 2 g + l / 32.
__device__ __forceinline__ void stage_hb(const v16f (&acc)[4][4], uint8_t *reg, int lane, int h) {
    const int i = h >> 1, p = h & 1;
    const int q = lane & 31;
    const int sw = (q & 15) ^ (lane >> 5);
    uint8_t *const row = reg + q * 256;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int j = 2 * p + jj;
            const v4f o = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                           acc[i][j][4 * g + 3]};
            *reinterpret_cast<v4f *>(row + (((8 * jj + 2 * g) ^ sw) << 4)) = o;
        }
}

// Read a staged half-block back as row segments.
// bf16 output: v[2 it + k] is row 8 it + l / 8, logical chunk 2 (l % 8) + k,
//   so lane l holds columns 8 (l % 8) .. +7 of its row (one 16-byte store).
// fp32 output: v[it] is row 4 it + l / 16, chunk l % 16 (columns 4 (l % 16)
//   .. +3, one 16-byte store).
template <int OUT>
__device__ __forceinline__ void read_hb(const uint8_t *reg, int lane, u32x4 (&v)[8]) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        int q, c;
        if constexpr (OUT == FP8_DTYPE_BF16) {
            q = 8 * (n >> 1) + (lane >> 3);
            c = 2 * (lane & 7) + (n & 1);
        } else {
            q = 4 * n + (lane >> 4);
            c = lane & 15;
        }
        v[n] = *reinterpret_cast<const u32x4 *>(reg + q * 256 + ((c ^ (q & 15)) << 4));
    }
}

// This lane's bias columns of the tile as fp32: bf16 output, columns
// 64 p + 8 (l % 8) .. +7 at b[8 p + k]; fp32 output, columns 64 p + 4 (l % 16)
// .. +3 at b[4 p + k].  `bl` is the tile's bf16 bias in LDS (the wave's 128
// columns).
template <int OUT, bool HAS_BIAS>
__device__ __forceinline__ void load_hb_bias(const uint8_t *bl, int lane, float (&b)[16]) {
#pragma unroll
    for (int k = 0; k < 16; ++k) b[k] = 0.f;
    if constexpr (HAS_BIAS) {
        if constexpr (OUT == FP8_DTYPE_BF16) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(bl + 2 * (64 * p + 8 * (lane & 7)));
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    b[8 * p + 2 * k] = __uint_as_float(ws[k] << 16);
                    b[8 * p + 2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const u32x2 w = *reinterpret_cast<const u32x2 *>(bl + 2 * (64 * p + 4 * (lane & 15)));
                b[4 * p + 0] = __uint_as_float(w.x << 16);
                b[4 * p + 1] = __uint_as_float(w.x & 0xFFFF0000u);
                b[4 * p + 2] = __uint_as_float(w.y << 16);
                b[4 * p + 3] = __uint_as_float(w.y & 0xFFFF0000u);
            }
        }
    }
}

// out(acc * s + bias) of half-block h from read_hb's registers, rows
// n0 .. n1 - 1 of its loop (bf16: row groups of 8 rows, 0..3; fp32: of 4
// rows, 0..7), stored as whole row segments (bf16: 128 bytes per row, eight
// rows per instruction; fp32: 256 bytes, four rows) through the resource
// over the wave's 128 output rows.  Columns past N take OUT_OOB (N is a
// multiple of 8 for bf16 and of 4 for fp32, so a lane's columns are all in
// or all out).
template <int OUT, bool HAS_BIAS, int POL>
__device__ __forceinline__ void out_hb(const u32x4 (&v)[8], const float (&b)[16],
                                       __amdgpu_buffer_rsrc_t rs, int N, int c0, int lane, float s,
                                       int h, int n0, int n1) {
    const int i = h >> 1, p = h & 1;
    if constexpr (OUT == FP8_DTYPE_BF16) {
        const int gc = c0 + 64 * p + 8 * (lane & 7);
        const uint32_t cb = gc < N ? (uint32_t)gc * 2u : OUT_OOB;   // + row offset < 2^31
        const uint32_t voff = cb + (uint32_t)((32 * i + (lane >> 3)) * N) * 2u;
#pragma unroll
        for (int it = n0; it < n1; ++it) {
            const u32x4 lo = v[2 * it], hi = v[2 * it + 1];
            const float x[8] = {__uint_as_float(lo.x), __uint_as_float(lo.y), __uint_as_float(lo.z),
                                __uint_as_float(lo.w), __uint_as_float(hi.x), __uint_as_float(hi.y),
                                __uint_as_float(hi.z), __uint_as_float(hi.w)};
            float y[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = HAS_BIAS ? x[k] * s + b[8 * p + k] : x[k] * s;
            const bf16x2 o0 = {(__bf16)y[0], (__bf16)y[1]}, o1 = {(__bf16)y[2], (__bf16)y[3]},
                         o2 = {(__bf16)y[4], (__bf16)y[5]}, o3 = {(__bf16)y[6], (__bf16)y[7]};
            const u32x4 o = {__builtin_bit_cast(uint32_t, o0), __builtin_bit_cast(uint32_t, o1),
                             __builtin_bit_cast(uint32_t, o2), __builtin_bit_cast(uint32_t, o3)};
            // the whole offset in the vector operand: the range check that
            // drops rows past M and columns past N does not see the scalar one
            __builtin_amdgcn_raw_buffer_store_b128(o, rs, (int)(voff + (uint32_t)(8 * it * N) * 2u),
                                                   0, POL);
        }
    } else {
        const int gc = c0 + 64 * p + 4 * (lane & 15);
        const uint32_t cb = gc < N ? (uint32_t)gc * 4u : OUT_OOB;   // + row offset < 2^31
        const uint32_t voff = cb + (uint32_t)((32 * i + (lane >> 4)) * N) * 4u;
#pragma unroll
        for (int it = n0; it < n1; ++it) {
            const u32x4 x = v[it];
            const v4f y = {__uint_as_float(x.x) * s + b[4 * p + 0], __uint_as_float(x.y) * s + b[4 * p + 1],
                           __uint_as_float(x.z) * s + b[4 * p + 2], __uint_as_float(x.w) * s + b[4 * p + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), rs,
                                                   (int)(voff + (uint32_t)(4 * it * N) * 4u), 0, POL);
        }
    }
}

// FP8-code epilogue of one wave's tile through LDS (16 KiB at `stg`): 128
// staging rows of 128 bytes, 16-byte chunk c of row q at chunk c ^ (q & 7).
// Lane l holds row (l % 32) of fragment row block i and, per register group
// g of fragment column block j, the four columns 32 j + 8 g + 4 (l / 32) ..
// +3: one code word at byte 16 (2 j + g / 2) + 8 (g % 2) + 4 (l / 32) of its
// row.  The bias is read from the tile's LDS bias slot.  The accumulators are left as they are
// (the next tile's first MFMAs start from zero).
//   fold: t = acc * (s * so) + bias * so, the scaled value itself, is clamped
//     and converted, and the amax keys are of |t| (the caller divides by
//     |so| once at the end).  Otherwise t = v = acc * s + bias and the encode
//     multiplies by so, exactly as the cast does (the only order in which a
//     0, inf or NaN scale gives the cast's results); that encode happens
//     only in the second pass below, which unfolded tiles always take.
//     `fold` is wave-uniform.
// Returns this lane's amax key of the tile's in-range outputs: the bits of
// max |t|, taken per fragment row block with the NaN-propagating maximum
// (one three-input instruction per two values), so a NaN t gives a key
// above inf's bits.  Columns past N hold t = 0
// (operand rows and bias read as zero there), so only rows past M (t =
// bias) are masked, once per block.  The words are first encoded without
// the NaN rule; when a key shows a NaN t in any lane of the wave (or the
// scale is not folded: the scale itself may make NaN products), the wave
// encodes the tile again with it, a NaN t getting 0x7F | sign.  One
// wave-uniform branch per tile, taken only on NaN data, instead of the rule
// evaluated and selected for every value.
template <int OUT, bool HAS_BIAS>
__device__ __forceinline__ uint32_t stage_wave_tile_q(v16f (&acc)[4][4], uint8_t *stg,
                                                      const uint8_t *bias_lds, int lane, float s,
                                                      float so, bool fold, int M, int r0) {
    constexpr int FMT = q_fmt<OUT>();
    const int frow = lane & 31;
    const int half = lane >> 5;
    const float sm = fold ? s * so : s;       // multiplier of the accumulator
    const float se = fold ? 1.0f : so;        // the encode's own scale
    const float sb = fold ? so : 1.0f;        // multiplier of the bias
    auto bias4 = [&](int j, int g, float mul, float (&bv)[4]) {
        bv[0] = bv[1] = bv[2] = bv[3] = 0.f;
        if constexpr (HAS_BIAS) {
            const u32x2 b2 = *reinterpret_cast<const u32x2 *>(
                bias_lds + 2 * (j * 32 + 8 * g + 4 * half));
            bv[0] = __uint_as_float(b2.x << 16) * mul;
            bv[1] = __uint_as_float(b2.x & 0xFFFF0000u) * mul;
            bv[2] = __uint_as_float(b2.y << 16) * mul;
            bv[3] = __uint_as_float(b2.y & 0xFFFF0000u) * mul;
        }
    };
    auto word_addr = [&](int i, int j, int g) {
        const int q = i * 32 + frow;
        return stg + q * 128 + (((2 * j + (g >> 1)) ^ (q & 7)) << 4) + 8 * (g & 1) + 4 * half;
    };
    // Per block i, max |t| by the NaN-propagating maximum (a NaN t makes the
    // key NaN, whose bits exceed those of inf).
    float kabs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float bv[4];
            bias4(j, g, sb, bv);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float t[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) t[q] = acc[i][j][4 * g + q] * sm + bv[q];
                // Folded, the encode's own scale is 1; unfolded, the second
                // pass below rewrites every word with it.
                const uint32_t w = encode4<FMT>(t[0], t[1], t[2], t[3], 1.0f);
                *reinterpret_cast<uint32_t *>(word_addr(i, j, g)) = w;
                kabs[i] = nan_max(nan_max(kabs[i], fabsf(t[0])), fabsf(t[1]));
                kabs[i] = nan_max(nan_max(kabs[i], fabsf(t[2])), fabsf(t[3]));
            }
        }
    }
    bool nan_seen = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) nan_seen |= __float_as_uint(kabs[i]) > 0x7F800000u;
    if (!fold || __builtin_amdgcn_ballot_w64(nan_seen) != 0) {
        // The same values again, read afresh from the accumulator registers:
        // the empty asm hides that they are unchanged, so the compiler does
        // not keep the first loop's copies of all 256 alive across the branch.
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float bv[4];
                bias4(j, g, sb, bv);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float t[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) t[q] = acc[i][j][4 * g + q] * sm + bv[q];
                    const uint32_t w = encode4<FMT>(t[0], t[1], t[2], t[3], se);
                    *reinterpret_cast<uint32_t *>(word_addr(i, j, g)) = patch_nan4(w, t, se);
                }
            }
        }
    }
    uint32_t key = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (r0 + i * 32 + frow < M) key = max(key, __float_as_uint(kabs[i]));
    return key;
}

// Largest key of the wave, as a wave-uniform value (held in a scalar
// register, so that it takes no vector register across the main loop).
__device__ __forceinline__ uint32_t wave_max_key(uint32_t k) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) k = max(k, (uint32_t)__shfl_xor((int)k, off, 64));
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)k);
}

// Read the staged codes back, 8 lanes per 128-byte row: v[it] is row
// 8 it + lane / 8, columns 16 (lane % 8) .. +15.
__device__ __forceinline__ void read_staged_rows_q(const uint8_t *stg, int lane, u32x4 (&v)[16]) {
    const int c = lane & 7;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int q = 8 * it + (lane >> 3);
        v[it] = *reinterpret_cast<const u32x4 *>(stg + q * 128 + ((c ^ (q & 7)) << 4));
    }
}

// Store the rows of read_staged_rows_q: 16 instructions, each writing eight
// 128-byte row segments (N % 16 == 0 keeps every 16-column group inside
// the row).
__device__ __forceinline__ void store_rows_q(__amdgpu_buffer_rsrc_t rs, const u32x4 (&v)[16],
                                             int N, int c0, int lane) {
    const int gc = c0 + 16 * (lane & 7);
    const uint32_t cb = gc < N ? (uint32_t)gc : OUT_OOB;        // + row offset < 2^31
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int row = 8 * it + (lane >> 3);
        const uint32_t off = cb + (uint32_t)(row * N);
        __builtin_amdgcn_raw_buffer_store_b128(v[it], rs, (int)off, 0, OUT_POLICY);
    }
}

// vmcnt wait that leaves the last N vector memory instructions in flight.
// Vector memory instructions of a wave complete in issue order (loads and
// stores alike on gfx9), so this waits for everything issued before them.
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
    static_assert(N == 4 || N == 8 || N == 16 || N == 20 || N == 24 || N == 32,
                  "wait_vmem_but: unsupported count");
    if constexpr (N == 4)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (N == 20)
        asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
    else if constexpr (N == 8)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if constexpr (N == 16)
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if constexpr (N == 24)
        asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
}

// Wait until this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Lane index from an instruction the compiler cannot merge with others, so
// that values derived from it are recomputed where they are used instead of
// being kept live (or spilled) across the kernel.
__device__ __forceinline__ int fresh_lane_id() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// vmcnt wait with any count (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and
// 15:14; expcnt (6:4) and lgkmcnt (11:8) at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
    static_assert(N >= 0 && N < 64, "vmcnt has six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// A direct-to-LDS 16-byte-per-lane load whose K offset is the scalar offset.
__device__ __forceinline__ void dma_b128_k(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                           uint32_t soff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m0), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// Small products with K % 128 == 0 and 32-bit operand offsets: the small
// kernel's tiles (BM x 128, four waves of BM/2 x 64 outputs with
// v_mfma_f32_16x16x128_f8f6f4, the same LDS layout and epilogue), with the
// operand stages written into LDS by the load unit (buffer loads with the
// LDS flag) instead of through registers: NS stages of 128 K-bytes, NS - 1
// of them in flight while the matrix cores work on one, one barrier per
// stage and no LDS write instructions.
//   * A stage is BM + 128 rows of 128 bytes, fetched by (BM + 128) / 8
//     instructions of 8 rows; wave w issues instructions w, w + 4, ...  Lane l
//     loads row 8q + l / 8 of instruction q, logical chunk (l % 8) ^ (l / 8),
//     which lands at chunk position l % 8: row r keeps chunk c at c ^ (r & 7).
//     Operand rows past M (N) read as zero through the descriptor range.
//   * In step k: wait for this wave's loads of stage k (the loads of the
//     later stages already requested stay in flight), barrier (every wave's loads of stage k
//     have landed and every wave has finished reading stage k - 1), request
//     stage k + NS - 1 into the buffer stage k - 1 used, read and multiply.
template <int BM, int NS, int FA, int FB, int OUT, bool HAS_BIAS>
__global__ __launch_bounds__(256) void gemm_nt_sdma_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, int M, int N, int K,
    const float *__restrict__ sinv_a, const float *__restrict__ sinv_b,
    const uint16_t *__restrict__ bias, void *__restrict__ Cv, int tiles_m, int tiles_n,
    const QOut qo) {
    static_assert(NS >= 2 && NS <= 4, "stages");
    constexpr int BN = 128, WN = 2;
    constexpr int WTM = BM / 2, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr uint32_t STAGE = (BM + BN) * BK;
    constexpr int LPW = (BM + BN) / 32;     // load instructions per wave per stage
    constexpr int LA = BM / 32;             // of them, on A rows

    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN;
    const int wn = wave % WN;

    int tile_m, tile_n;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN;

    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(A), (short)0, M * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(B), (short)0, N * K, 0x00020000);
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    uint32_t voff[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int q = wave + 4 * i;         // instruction: rows 8q .. 8q + 7 of the stage
        const int r = 8 * q + (lane >> 3);
        const int kc = (lane & 7) ^ (lane >> 3);
        const int grow = i < LA ? m0 + r : n0 + (r - BM);
        voff[i] = (uint32_t)grow * (uint32_t)K + (uint32_t)(16 * kc);
    }
    auto issue = [&](int st, int buf) {
        const uint32_t k0 = (uint32_t)__builtin_amdgcn_readfirstlane(st * BK);
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            dma_b128_k(i < LA ? ra : rb, voff[i], k0,
                       lds0 + (uint32_t)buf * STAGE + (uint32_t)(wave + 4 * i) * 1024u);
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;
    const int fc0 = (lane >> 4) * 2;
    const int sw = frow & 7;
    const int off0 = ((fc0 ^ sw) << 4);
    const int off1 = (((fc0 + 1) ^ sw) << 4);

    const int nk = K / BK;                  // >= 2 (the launcher guarantees)
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
        if (st < nk) issue(st, st);
    for (int k = 0; k < nk; ++k) {
        // stages issued after stage k: k + 1 .. min(k + NS - 2, nk - 1)
        const int ahead = min(NS - 2, nk - 1 - k);
        if (ahead <= 0)
            wait_vmem_le<0>();
        else if (NS >= 3 && ahead == 1)
            wait_vmem_le<LPW>();
        else
            wait_vmem_le<(NS >= 4 ? 2 : 1) * LPW>();
        __syncthreads();
        if (k + NS - 1 < nk) issue(k + NS - 1, (k + NS - 1) % NS);

        const uint8_t *stg = lds + (uint32_t)(k % NS) * STAGE;
        const uint8_t *As = stg + (wm * WTM + frow) * BK;
        const uint8_t *Bs = stg + BM * BK + (wn * WTN + frow) * BK;
        v8i bf[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(Bs + j * 16 * BK + off0);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(Bs + j * 16 * BK + off1);
            bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(As + i * 16 * BK + off0);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(As + i * 16 * BK + off1);
            const v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bf[j], af, acc[i][j], FB, FA, 0, 0, 0, 0);
        }
    }

    // Epilogue (the small kernel's): lane (l % 16, l / 16) holds output row
    // l % 16 of each 16-row fragment, columns 4 (l / 16) .. +3.
    const float s = (*sinv_a) * (*sinv_b);
    float so = 0.f;
    bool so_special = false;
    if constexpr (is_q_out<OUT>()) {
        so = *qo.scale;
        so_special = scale_is_special(so);
    }
    uint32_t key = 0;
    const int orow = lane & 15;
    const int ocol = (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int gc = n0 + wn * WTN + j * 16 + ocol;
        if (gc >= N) continue;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (HAS_BIAS) {
            const u32x2 b2 = *reinterpret_cast<const u32x2 *>(bias + gc);
            bv[0] = __uint_as_float(b2.x << 16);
            bv[1] = __uint_as_float(b2.x & 0xFFFF0000u);
            bv[2] = __uint_as_float(b2.y << 16);
            bv[3] = __uint_as_float(b2.y & 0xFFFF0000u);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int gr = m0 + wm * WTM + i * 16 + orow;
            if (gr >= M) continue;
            const v4f a = acc[i][j];
            const float y0 = a.x * s + bv[0];
            const float y1 = a.y * s + bv[1];
            const float y2 = a.z * s + bv[2];
            const float y3 = a.w * s + bv[3];
            if constexpr (OUT == FP8_DTYPE_BF16) {
                uint16_t *C = static_cast<uint16_t *>(Cv);
                const bf16x4 o = {(__bf16)y0, (__bf16)y1, (__bf16)y2, (__bf16)y3};
                *reinterpret_cast<bf16x4 *>(C + (int64_t)gr * N + gc) = o;
            } else if constexpr (is_q_out<OUT>()) {
                uint8_t *C = static_cast<uint8_t *>(Cv);
                *reinterpret_cast<uint32_t *>(C + (int64_t)gr * N + gc) =
                    encode_out4<OUT>(y0, y1, y2, y3, so, so_special, key);
            } else {
                float *C = static_cast<float *>(Cv);
                *reinterpret_cast<v4f *>(C + (int64_t)gr * N + gc) = v4f{y0, y1, y2, y3};
            }
        }
    }
    // All waves are past their last stage reads at the reduction's barrier.
    if constexpr (is_q_out<OUT>()) finish_q_out(key, qo, so, reinterpret_cast<uint32_t *>(lds));
}

// Large-problem kernel for K % 128 == 0: persistent 256 x 256 tiles (one
// 256-thread workgroup per CU, four waves of 128 x 128 with
// v_mfma_f32_32x32x64_f8f6f4) whose operand stages are written into LDS by
// the load unit itself (buffer loads with the LDS flag), not through
// registers.
//   * Stages are 128 K-bytes (64 KiB for A and B), so every operand row
//     segment is one whole 128-byte line, double-buffered in 128 KiB of LDS;
//     no staging registers and no LDS write instructions in the main loop.
//   * Wave w fetches rows 128 w .. 128 w + 127 of the 512-row stage (A rows
//     for waves 0-1, B rows for 2-3): 16 instructions of 8 rows, lane l
//     taking row l / 8 of the eight and the logical chunk that lands at
//     chunk position l % 8 under the swizzle.
//   * One barrier per stage, in its middle.  Stage k runs 16 MFMAs on the
//     fragments of its first 64 K-bytes (read earlier) while reading those
//     of its second 64; then every wave waits for its own loads of stage k+1
//     and meets the others at the barrier, after which stage k's buffer is
//     free (all its fragments are in registers) and stage k+1's is complete.
//     The second 16 MFMAs then carry the loads of stage k+2 into the freed
//     buffer (one per MFMA, which paces them at the load unit's rate) and
//     the reads of stage k+1's first fragments.
//   * Stages stream on across tile boundaries.  A tile's stage nk-2
//     requests the next tile's stage 0 and bias (two 1 KiB bias slots past
//     the stages); the epilogue stages each wave's output in its own 16 KiB
//     quarter of the buffer freed by stage nk-1 and reads it back as whole
//     row segments: bf16 and fp32 as raw accumulators in eight half-blocks
//     through two 8 KiB regions (see stage_hb; the first ones between the
//     last stage's MFMAs), FP8 codes in one pass (128-byte segments).  Each
//     half-block's stores go out as soon as it is read back, so they drain
//     while the next one is converted.  That
//     quarter is exactly what the wave's own stage loads fill, so once its
//     staging reads have returned the wave requests the next tile's stage 1
//     there, with no barrier, and issues its last block's stores after it.
//     The stores are buffer stores that are always issued (the hardware
//     drops the out-of-range ones).  Vector memory instructions of a wave
//     complete in order, so the next tile waits with exact counts: for its
//     stage 0 with stage 1 and the last stores in flight, then at stage 0's
//     middle for stage 1 with those stores in flight.
//   * The per-lane load offsets and epilogue addresses are recomputed where
//     they are used, from a lane index the compiler cannot hoist: kept live
//     across the loop they spill, and a spill reload waits for every load
//     in flight.
template <int FA, int FB, int OUT, bool HAS_BIAS, bool PART>
__global__ __launch_bounds__(256) void gemm_nt_dma_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, int M, int N, int K,
    const float *__restrict__ sinv_a, const float *__restrict__ sinv_b,
    const uint16_t *__restrict__ bias, void *__restrict__ Cv, int tiles_m, int tiles_n, QOut qo,
    int parts) {
    static_assert(!PART || (OUT == FP8_DTYPE_FP32 && !HAS_BIAS), "parts are raw fp32 sums");
    constexpr int BM = 256, BN = 256;
    constexpr int KS = 128;                     // K bytes per stage
    constexpr int WT = 128;                     // wave tile (square)
    constexpr int F = WT / 32;                  // 4 x 4 fragments of 32 x 32
    constexpr uint32_t STAGE = (BM + BN) * KS;  // 64 KiB
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int T = tiles_m * tiles_n;
    // Work units: unit r is tile r % T over K part r / T (PART), else tile r.
    const int NU = PART ? T * parts : T;
    if ((int)blockIdx.x >= NU) return;
    const int KP = PART ? K / parts : K;        // K bytes of one unit

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1;
    const int wn = wave & 1;

    const __amdgpu_buffer_rsrc_t ra_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(A), (short)0, M * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(B), (short)0, N * K, 0x00020000);
    const bool loads_b = wave >= 2;
    const __amdgpu_buffer_rsrc_t ld_rsrc = loads_b ? rb_rsrc : ra_rsrc;
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    const uint32_t ld_lds = lds0 + (uint32_t)wave * (128 * KS);   // this wave's 128 rows
    // Two 1 KiB bias slots past the two stages: a tile's 256 bias values
    // (512 bytes; one load instruction moves 1 KiB) in slot t % 2 for the
    // t-th tile of this workgroup, so the next tile's bias can land while
    // the current tile's epilogue reads its own.
    uint8_t *const bias_lds = lds + 2 * STAGE;

    // Per-lane part of the load offsets: row l / 8 of an 8-row group, the
    // logical chunk stored at position l % 8 (the swizzle of rows 8i..8i+7
    // is (l / 8) ^ (i & 1)).  Recomputed at the top of every tile and before
    // every request of a tile's first stages, so that they are never kept
    // live (or spilled) across the epilogue: a spill reload there would wait
    // for every load in flight.
    uint32_t voff_e, voff_o;
    auto set_voff = [&]() {
        const int l = fresh_lane_id();
        const int lr = l >> 3;
        voff_e = (uint32_t)(lr * K + 16 * ((l & 7) ^ lr));
        voff_o = (uint32_t)(lr * K + 16 * ((l & 7) ^ lr ^ 1));
    };
    // Load instruction i (0..15) of a stage: rows 8i..8i+7 of this wave's
    // 128, starting at operand byte offset `base` (+ k0 along K).
    auto load_one = [&](int i, uint32_t base, uint32_t k0, uint32_t buf) {
        const uint32_t so = base + (uint32_t)(8 * i) * (uint32_t)K + k0;
        dma_b128(ld_rsrc, so + ((i & 1) ? voff_o : voff_e), ld_lds + buf + (uint32_t)i * 1024u);
    };

    // Fragment reads: row (lane % 32) of a 32-row fragment, 16-byte chunks
    // 4 s + 2 (lane / 32) and + 1 for K half s of the stage.
    const int frow = lane & 31;
    const int fsw = dma_swz(frow);
    const int c0 = 2 * (lane >> 5);
    uint32_t fo[2][2];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh)
#pragma unroll
        for (int h = 0; h < 2; ++h) fo[sh][h] = frow * KS + (((4 * sh + c0 + h) ^ fsw) << 4);
    const uint32_t a_fbase = (uint32_t)(wm * WT * KS);
    const uint32_t b_fbase = (uint32_t)(BM * KS + wn * WT * KS);

    v8i af[2][F], bf[2][F];                     // [K half][fragment]
    auto read_half = [&](v8i &dst, uint32_t off, int h) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + off);
        dst[4 * h + 0] = (int)v.x; dst[4 * h + 1] = (int)v.y;
        dst[4 * h + 2] = (int)v.z; dst[4 * h + 3] = (int)v.w;
    };
    // Fragment n (0..7) of a K half in read order A0, B0..B3, A1..A3, half h.
    auto read_frag = [&](int sh, int n, int h, uint32_t buf) {
        if (n >= 1 && n <= 4)
            read_half(bf[sh][n - 1], buf + b_fbase + (n - 1) * 32 * KS + fo[sh][h], h);
        else {
            const int a = (n == 0) ? 0 : n - 4;
            read_half(af[sh][a], buf + a_fbase + a * 32 * KS + fo[sh][h], h);
        }
    };

    v16f acc[F][F];
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Output stores a tile leaves in flight past its last load request.
    constexpr int NST = OUT == FP8_DTYPE_BF16 ? 4 : (OUT == FP8_DTYPE_FP32 ? 8 : 16);
    // One stage: MFMAs on both K halves around the barrier.  DMA: issue the
    // loads of stage k+2 (or of the next tile's stage 0, at `base` and
    // `ld_k0`) into this stage's buffer; RD: read the next stage's first
    // fragments.  WAIT, before the barrier: 0 = every load of this wave has
    // landed (stage k+1 was requested last); 1 = the same, but the previous
    // tile's NST output stores, the only memory instructions issued after
    // stage k+1's loads, stay in flight; 2 = no wait (a tile's last stage:
    // nothing of the tile is loading, only the next tile's first stage).
    // FIRST: the tile's first stage (see first_half).
    // First half of a stage: 16 MFMAs on the first K half's fragments, with
    // the reads of the second half's.  ZERO (a tile's first stage): the
    // MFMAs start from zero instead of the accumulators, so the epilogue
    // never clears them.
    auto first_half = [&](uint32_t buf, auto zero) {
#pragma unroll
        for (int slot = 0; slot < 16; ++slot) {
            const int i = slot >> 2, j = slot & 3;
            if constexpr (decltype(zero)::value)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    bf[0][j], af[0][i], v16f{}, FB, FA, 0, 0, 0, 0);
            else
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    bf[0][j], af[0][i], acc[i][j], FB, FA, 0, 0, 0, 0);
            if (slot < 8) {
                read_frag(1, slot, 0, buf);
                read_frag(1, slot, 1, buf);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto stage = [&](uint32_t buf, bool dma, bool rd, uint32_t base, uint32_t ld_k0, int wait,
                     bool first) {
        const uint32_t nbuf = buf ^ STAGE;
        if (first)
            first_half(buf, std::true_type{});
        else
            first_half(buf, std::false_type{});
        // Stage k+1 has landed (own loads) and is visible (barrier); nobody
        // reads this stage's buffer any more.
        if (wait == 0)
            wait_vmem_all();
        else if (wait == 1)
            wait_vmem_but<NST>();
        __syncthreads();
#pragma unroll
        for (int slot = 0; slot < 16; ++slot) {
            const int i = slot >> 2, j = slot & 3;
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[1][j], af[1][i], acc[i][j], FB, FA, 0, 0, 0, 0);
            if (dma) load_one(slot, base, ld_k0, buf);
            if (rd) read_frag(0, slot >> 1, slot & 1, nbuf);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int nk = KP / KS;                     // >= 2 (caller guarantees)
    // A part is the raw sum: the reduction applies the scales and the bias.
    const float s = PART ? 1.0f : (*sinv_a) * (*sinv_b);
    // Parts are read back at once by the reduction: cached stores.
    constexpr int OPOL = PART ? 0 : OUT_POLICY;
    // bf16 / fp32 output: a tile's last stage, with the epilogue's first
    // half-blocks (see stage_hb) staged, read back and stored between the
    // MFMAs of its second half.  The wave's staging quarter `stg` (regions
    // stg and stg + 8 KiB) is free once every wave has passed the stage's
    // barrier.  Fragment (i, j) is final after the MFMA of slot 4 i + j, so
    // half-block h = 2 i + p can be staged one slot after slot 4 i + 2 p + 1.
    // A wave's LDS instructions execute in issue order, so a region is
    // rewritten right after the read of its previous half-block is issued,
    // and read right after it is written.  The arithmetic of a half-block is
    // spread one quarter (U store loops, about a dozen vector instructions)
    // per MFMA, which the matrix core's 64 cycles per instruction cover.
    // Half-blocks 0, 1 and the first quarter of 2 are stored here; va holds
    // half-block 2 on return.
    constexpr int U = OUT == FP8_DTYPE_BF16 ? 1 : 2;   // store loops per quarter
    auto last_stage_hb = [&](uint32_t buf, uint8_t *stg, u32x4 (&va)[8], u32x4 (&vb)[8],
                             const float (&bb)[16], __amdgpu_buffer_rsrc_t ors, int cc0, int el) {
        first_half(buf, std::false_type{});   // stage nk-1 >= 1 is never a tile's first
        __syncthreads();
        auto quarter = [&](const u32x4 (&v)[8], int h, int qn) {
            out_hb<OUT, HAS_BIAS, OPOL>(v, bb, ors, N, cc0, el, s, h, qn * U, qn * U + U);
        };
#pragma unroll
        for (int sl = 0; sl < 16; ++sl) {
            const int i = sl >> 2, j = sl & 3;
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[1][j], af[1][i], acc[i][j], FB, FA, 0, 0, 0, 0);
            if (sl == 2) stage_hb(acc, stg, el, 0);
            if (sl == 4) stage_hb(acc, stg + 8192, el, 1);
            if (sl == 5) read_hb<OUT>(stg, el, va);
            if (sl == 6) stage_hb(acc, stg, el, 2);
            if (sl >= 7 && sl <= 10) quarter(va, 0, sl - 7);
            if (sl == 9) read_hb<OUT>(stg + 8192, el, vb);
            if (sl == 10) stage_hb(acc, stg + 8192, el, 3);
            if (sl >= 11 && sl <= 14) quarter(vb, 1, sl - 11);
            if (sl == 13) read_hb<OUT>(stg, el, va);
            if (sl == 14) stage_hb(acc, stg, el, 4);
            if (sl == 15) quarter(va, 2, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    float so = 0.f;
    bool so_fold = false;
    if constexpr (is_q_out<OUT>()) {
        so = *qo.scale;
        so_fold = scale_is_foldable(so);
    }
    uint32_t wkey = 0;                          // FP8 output: the wave's amax key
    // Operand byte offset of this wave's 128 rows of unit r's tile, at the
    // start of its K part.  (T % 8 == 0 keeps tile r % T on unit r's XCD.)
    auto unit_tile = [&](int r, int &tm, int &tn) {
        tile_of_block(PART ? r % T : r, tiles_m, tiles_n, tm, tn);
    };
    auto tile_base = [&](int r) {
        int tm, tn;
        unit_tile(r, tm, tn);
        const uint32_t k0 = PART ? (uint32_t)((r / T) * KP) : 0u;
        return (uint32_t)(((loads_b ? tn * BN : tm * BM) + (wave & 1) * 128) * K) + k0;
    };
    // Tile r's bias into bias slot `slot` (wave 0).
    auto load_bias = [&](int r, int slot) {
        if constexpr (HAS_BIAS) {
            if (wave == 0) {
                int tm, tn;
                tile_of_block(r, tiles_m, tiles_n, tm, tn);
                const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<uint16_t *>(bias), (short)0, 2 * N, 0x00020000);
                dma_b128(brs, (uint32_t)(2 * tn * BN + 16 * fresh_lane_id()),
                         lds0 + 2 * STAGE + 1024u * (uint32_t)slot);
            }
        }
    };
    auto issue_stage = [&](uint32_t base, uint32_t k0, uint32_t buf) {
        set_voff();
#pragma unroll
        for (int i = 0; i < 16; ++i) load_one(i, base, k0, buf);
    };
    // Stage 0's first fragments of the buffer `buf` into registers.
    auto read_first = [&](uint32_t buf) {
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int h = 0; h < 2; ++h) read_frag(0, n, h, buf);
    };

    // The first tile: its bias and stages 0 and 1, waited for.
    load_bias((int)blockIdx.x, 0);
    issue_stage(tile_base((int)blockIdx.x), 0, 0);
    issue_stage(tile_base((int)blockIdx.x), KS, STAGE);
    wait_vmem_all();
    __syncthreads();
    read_first(0);

    // Stages stream on across tiles: the buffer of a stage alternates with
    // no reset at tile boundaries.  At the end of a tile, stage nk-2 requests
    // the next tile's stage 0 (and its bias) into its freed buffer; stage
    // nk-1's buffer, free after its barrier, stages the epilogue; once every
    // wave has read the staging back, it receives the next tile's stage 1,
    // and only then are the output stores issued.  The next tile waits for
    // its stages with the NST stores still in flight; the first wait that
    // needs a later load (stage 1's) also waits for them.
    uint32_t buf = 0;
    int slot = 0;
    bool pend = false;                          // the previous tile's stores are in flight
    for (int r = (int)blockIdx.x; r < NU; r += (int)gridDim.x) {
        int tm, tn;
        set_voff();
        unit_tile(r, tm, tn);
        const uint32_t base =
            (uint32_t)(((loads_b ? tn * BN : tm * BM) + (wave & 1) * 128) * K) +
            (PART ? (uint32_t)((r / T) * KP) : 0u);
        const int rn = r + (int)gridDim.x;
        const bool more = rn < NU;
        const uint32_t nbase = more ? tile_base(rn) : 0u;
        for (int k = 0; k + 2 < nk; ++k) {
            stage(buf, true, true, base, (uint32_t)((k + 2) * KS), (k == 0 && pend) ? 1 : 0, k == 0);
            buf ^= STAGE;
        }
        stage(buf, more, true, nbase, 0, (nk == 2 && pend) ? 1 : 0, nk == 2);   // stage nk-2
        if (more) load_bias(rn, slot ^ 1);
        buf ^= STAGE;
        const uint32_t sbuf = buf;              // staging; then the next tile's stage 1
        // The epilogue's per-lane addresses derive from a lane index read
        // here, so the compiler cannot hoist them out of the tile loop (where
        // they would be spilled and reloaded with a wait for every load).
        const int el = fresh_lane_id();
        uint8_t *stg = lds + sbuf + wave * 16384;
        const uint8_t *bl = bias_lds + 1024 * slot + 2 * wn * WT;
        const int r0 = tm * BM + wm * WT, cc0 = tn * BN + wn * WT;
        if constexpr (!is_q_out<OUT>()) {
            constexpr int EB = OUT == FP8_DTYPE_BF16 ? 2 : 4;
            // A part goes to its own [M, N] fp32 slice of the workspace.
            void *const Cu = PART ? static_cast<void *>(static_cast<float *>(Cv) +
                                                        (int64_t)(r / T) * M * N)
                                  : Cv;
            const __amdgpu_buffer_rsrc_t ors = out_rows_rsrc<EB>(Cu, M, N, r0);
            float bb[16];
            load_hb_bias<OUT, HAS_BIAS>(bl, el, bb);
            u32x4 va[8], vb[8];
            last_stage_hb(buf, stg, va, vb, bb, ors, cc0, el);   // stage nk-1, half-blocks 0-2
            buf ^= STAGE;                                     // the next tile's stage 0
            uint8_t *const reg1 = stg + 8192;
            // The rest of the tile, each read issued before the previous
            // half-block's arithmetic so that its latency is covered.
            read_hb<OUT>(reg1, el, vb);                        // 3
            stage_hb(acc, reg1, el, 5);
            out_hb<OUT, HAS_BIAS, OPOL>(va, bb, ors, N, cc0, el, s, 2, U, 4 * U);
            read_hb<OUT>(stg, el, va);                         // 4
            stage_hb(acc, stg, el, 6);
            out_hb<OUT, HAS_BIAS, OPOL>(vb, bb, ors, N, cc0, el, s, 3, 0, 4 * U);
            read_hb<OUT>(reg1, el, vb);                        // 5
            stage_hb(acc, reg1, el, 7);
            out_hb<OUT, HAS_BIAS, OPOL>(va, bb, ors, N, cc0, el, s, 4, 0, 4 * U);
            read_hb<OUT>(stg, el, va);                         // 6
            out_hb<OUT, HAS_BIAS, OPOL>(vb, bb, ors, N, cc0, el, s, 5, 0, 4 * U);
            read_hb<OUT>(reg1, el, vb);                        // 7
            out_hb<OUT, HAS_BIAS, OPOL>(va, bb, ors, N, cc0, el, s, 6, 0, 4 * U);
            // The staging quarter is the one this wave's own stage loads
            // fill and no other wave reads it: once this wave's staging
            // reads have returned, the next tile's stage 1 is requested into
            // it (no barrier), and the last half-block's NST stores follow.
            wait_lds_reads();
            if (more) issue_stage(nbase, KS, sbuf);
            out_hb<OUT, HAS_BIAS, OPOL>(vb, bb, ors, N, cc0, el, s, 7, 0, 4 * U);
        } else {
            stage(buf, false, false, 0, 0, 2, false);   // stage nk-1: its buffer is free after the barrier
            buf ^= STAGE;                           // the next tile's stage 0
            // The staging quarter of the buffer is the one this wave's own
            // stage loads fill, and no other wave reads it after stage nk-1's
            // barrier: so the next tile's stage 1 is requested as soon as this
            // wave's own staging reads have returned, with no barrier.
            const uint32_t tk = stage_wave_tile_q<OUT, HAS_BIAS>(acc, stg, bl, el, s, so,
                                                                 so_fold, M, r0);
            wkey = max(wkey, wave_max_key(tk));
            u32x4 rows_out[16];
            read_staged_rows_q(stg, el, rows_out);
            wait_lds_reads();
            if (more) issue_stage(nbase, KS, sbuf);
            store_rows_q(out_rows_rsrc<1>(Cv, M, N, r0), rows_out, N, cc0, el);
        }
        if (more) {
            // The next tile's bias and stage 0 have landed (its stage 1, 16
            // loads, and the NST stores may still be in flight; stage 0's
            // middle waits for stage 1); its first fragments into registers.
            wait_vmem_but<NST + 16>();
            __syncthreads();
            read_first(buf);
        }
        slot ^= 1;
        pend = true;
    }
    if constexpr (is_q_out<OUT>())
        finish_q_out(wkey, qo, so, reinterpret_cast<uint32_t *>(lds), so_fold);
}

template <int FA, int FB, int OUT, bool HAS_BIAS>
hipError_t launch_big(const uint8_t *A, const uint8_t *B, int M, int N, int K, const float *sa,
                      const float *sb, const uint16_t *bias, void *C, const QOut &qo,
                      hipStream_t stream) {
    auto kern = gemm_nt_big_kernel<FA, FB, OUT, HAS_BIAS>;
    constexpr int lds_bytes = 3 * (256 + 256) * 64;   // three 32 KiB stages
    static std::atomic<uint64_t> lds_enabled{0};
    if (hipError_t e = enable_dynamic_lds(reinterpret_cast<const void *>(kern), lds_bytes,
                                          lds_enabled))
        return e;
    int cus = 0;
    if (hipError_t e = current_cu_count(&cus)) return e;
    const int tiles_m = (M + 255) / 256;
    const int tiles_n = (N + 255) / 256;
    const int grid = std::min(tiles_m * tiles_n, cus);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds_bytes, stream, A, B, M, N, K, sa, sb, bias,
                       C, tiles_m, tiles_n, qo);
    return hipGetLastError();
}

// PART: `parts` K parts per tile, raw fp32 sums into C = the [parts, M, N]
// workspace (then splitk_reduce_kernel); one unit per workgroup when
// tiles * parts <= CUs.
template <int FA, int FB, int OUT, bool HAS_BIAS, bool PART = false>
hipError_t launch_dma(const uint8_t *A, const uint8_t *B, int M, int N, int K, const float *sa,
                      const float *sb, const uint16_t *bias, void *C, const QOut &qo,
                      hipStream_t stream, int parts = 1) {
    auto kern = gemm_nt_dma_kernel<FA, FB, OUT, HAS_BIAS, PART>;
    constexpr int lds_bytes = 2 * (256 + 256) * 128 + 2048;   // two 64 KiB stages, 2 bias slots
    static std::atomic<uint64_t> lds_enabled{0};
    if (hipError_t e = enable_dynamic_lds(reinterpret_cast<const void *>(kern), lds_bytes,
                                          lds_enabled))
        return e;
    int cus = 0;
    if (hipError_t e = current_cu_count(&cus)) return e;
    const int tiles_m = (M + 255) / 256;
    const int tiles_n = (N + 255) / 256;
    const int grid = std::min(tiles_m * tiles_n * (PART ? parts : 1), cus);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds_bytes, stream, A, B, M, N, K, sa, sb, bias,
                       C, tiles_m, tiles_n, qo, PART ? parts : 1);
    return hipGetLastError();
}

// The second pass of a split product: C[i, j] = out(sum over p of
// part[p][i, j] (in part order, fp32) * (*sinv_a) * (*sinv_b) + bias[j]),
// the unsplit kernels' epilogue arithmetic.  One lane per V consecutive
// outputs of a row (V = 8 for bf16, 4 for fp32; N is a multiple of V).
template <int OUT, bool HAS_BIAS>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const float *__restrict__ part, int parts, int64_t MN, int N, const float *__restrict__ sinv_a,
    const float *__restrict__ sinv_b, const uint16_t *__restrict__ bias, void *__restrict__ Cv) {
    constexpr int V = OUT == FP8_DTYPE_BF16 ? 8 : 4;
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
    if (i >= MN) return;
    const float s = (*sinv_a) * (*sinv_b);
    float acc[V];
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
        const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(part + i) + h);
        acc[4 * h + 0] = v[0]; acc[4 * h + 1] = v[1]; acc[4 * h + 2] = v[2]; acc[4 * h + 3] = v[3];
    }
    for (int p = 1; p < parts; ++p) {
        const float *q = part + (int64_t)p * MN + i;
#pragma unroll
        for (int h = 0; h < V / 4; ++h) {
            const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(q) + h);
            acc[4 * h + 0] += v[0]; acc[4 * h + 1] += v[1];
            acc[4 * h + 2] += v[2]; acc[4 * h + 3] += v[3];
        }
    }
    const int c = (int)(i % N);
    float b[V];
#pragma unroll
    for (int k = 0; k < V; ++k)
        b[k] = HAS_BIAS ? __uint_as_float((uint32_t)bias[c + k] << 16) : 0.f;
    if constexpr (OUT == FP8_DTYPE_BF16) {
        float y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = HAS_BIAS ? acc[k] * s + b[k] : acc[k] * s;
        const bf16x2 o0 = {(__bf16)y[0], (__bf16)y[1]}, o1 = {(__bf16)y[2], (__bf16)y[3]},
                     o2 = {(__bf16)y[4], (__bf16)y[5]}, o3 = {(__bf16)y[6], (__bf16)y[7]};
        const u32x4 o = {__builtin_bit_cast(uint32_t, o0), __builtin_bit_cast(uint32_t, o1),
                         __builtin_bit_cast(uint32_t, o2), __builtin_bit_cast(uint32_t, o3)};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(Cv) + i));
    } else {
        const v4f y = {acc[0] * s + b[0], acc[1] * s + b[1], acc[2] * s + b[2], acc[3] * s + b[3]};
        __builtin_nontemporal_store(y, reinterpret_cast<v4f *>(static_cast<float *>(Cv) + i));
    }
}

template <int OUT, bool HAS_BIAS>
hipError_t launch_splitk_reduce(const float *part, int parts, int64_t M, int64_t N,
                                const float *sa, const float *sb, const uint16_t *bias, void *C,
                                hipStream_t stream) {
    constexpr int V = OUT == FP8_DTYPE_BF16 ? 8 : 4;
    const int64_t lanes = M * N / V;
    hipLaunchKernelGGL((splitk_reduce_kernel<OUT, HAS_BIAS>), dim3((unsigned)((lanes + 255) / 256)),
                       dim3(256), 0, stream, part, parts, M * N, (int)N, sa, sb, bias, C);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, bool HAS_BIAS>
hipError_t launch_cfg(const uint8_t *A, const uint8_t *B, int M, int N, int K, const float *sa,
                      const float *sb, const uint16_t *bias, void *C, const QOut &qo,
                      hipStream_t stream) {
    auto kern = gemm_nt_kernel<BM, BN, WM, WN, FA, FB, OUT, HAS_BIAS>;
    constexpr int lds_bytes = 2 * (BM + BN) * BK;
    // Dynamic LDS above 64 KiB must be enabled once per device and kernel.
    static std::atomic<uint64_t> lds_enabled{0};
    if (hipError_t e = enable_dynamic_lds(reinterpret_cast<const void *>(kern), lds_bytes,
                                          lds_enabled))
        return e;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(WM * WN * 64), lds_bytes, stream, A, B,
                       M, N, K, sa, sb, bias, C, tiles_m, tiles_n, qo);
    return hipGetLastError();
}

// LDS stages of the direct-to-LDS small kernel per tile height: 72 KiB and
// 64 KiB, so two workgroups share a CU (measured on MI355X: two 128-row
// stages of 32 KiB beat three, which leave one workgroup per CU, by 10-40%;
// two, three or four 64-row stages are within a few percent).
constexpr int SDMA_STAGES_64 = 3;
constexpr int SDMA_STAGES_128 = 2;

template <int BM, int FA, int FB, int OUT, bool HAS_BIAS>
hipError_t launch_sdma(const uint8_t *A, const uint8_t *B, int M, int N, int K, const float *sa,
                       const float *sb, const uint16_t *bias, void *C, const QOut &qo,
                       hipStream_t stream) {
    constexpr int NS = BM == 64 ? SDMA_STAGES_64 : SDMA_STAGES_128;
    auto kern = gemm_nt_sdma_kernel<BM, NS, FA, FB, OUT, HAS_BIAS>;
    constexpr int lds_bytes = NS * (BM + 128) * BK;
    static std::atomic<uint64_t> lds_enabled{0};
    if (hipError_t e = enable_dynamic_lds(reinterpret_cast<const void *>(kern), lds_bytes,
                                          lds_enabled))
        return e;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + 127) / 128;
    hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(256), lds_bytes, stream, A, B, M, N,
                       K, sa, sb, bias, C, tiles_m, tiles_n, qo);
    return hipGetLastError();
}

template <int FA, int FB, int OUT, bool HAS_BIAS>
hipError_t launch_fmt(const uint8_t *A, const uint8_t *B, int64_t M, int64_t N, int64_t K,
                      const float *sa, const float *sb, const uint16_t *bias, void *C,
                      const QOut &qo, hipStream_t stream, void *ws = nullptr,
                      int64_t ws_bytes = 0) {
    // Large problems: 256 x 256 tiles, four waves of 128 x 128 (32x32x64
    // instructions); small ones: 128 x 128 or 64 x 128 tiles (16x16x128
    // instructions).
    // The large kernel addresses operands with 32-bit buffer offsets.
    // It also needs at least four 64-byte K stages.
    const bool fits32 = (M + 256) * K < ((int64_t)1 << 31) && (N + 256) * K < ((int64_t)1 << 31);
    // The LDS-DMA kernel also addresses 128 output rows with 32-bit offsets.
    constexpr int64_t out_bytes = OUT == FP8_DTYPE_BF16 ? 2 : (OUT == FP8_DTYPE_FP32 ? 4 : 1);
    const bool out32 = 128 * N * out_bytes < ((int64_t)1 << 31);
    int cus = 0;
    if (hipError_t e = current_cu_count(&cus)) return e;
    // Products that leave CUs idle, given a workspace: K parts on the LDS-DMA
    // kernel, then the part sum (gemm_split_parts picks the count).
    if constexpr (!is_q_out<OUT>()) {
        const bool part32 = 128 * N * 4 < ((int64_t)1 << 31);
        const int parts = (ws != nullptr && fits32 && part32)
                              ? gemm_split_parts(M, N, K, cus, ws_bytes)
                              : 1;
        if (parts > 1) {
            if (hipError_t e = launch_dma<FA, FB, FP8_DTYPE_FP32, false, true>(
                    A, B, (int)M, (int)N, (int)K, sa, sb, nullptr, ws, qo, stream, parts))
                return e;
            return launch_splitk_reduce<OUT, HAS_BIAS>(static_cast<const float *>(ws), parts, M,
                                                       N, sa, sb, bias, C, stream);
        }
    }
    // The large kernels run at about twice the small kernel's rate per CU, so
    // they take every product with at least three quarters of a 256 x 256
    // tile per CU (e.g. 1024 x 12288: 192 tiles).
    const int64_t tiles256 = ((M + 255) / 256) * ((N + 255) / 256);
    const bool large = M * N >= (int64_t)256 * 256 * 256 || 4 * tiles256 >= 3 * (int64_t)cus;
    if (large && fits32 && out32 && K >= 256 && K % 128 == 0)
        return launch_dma<FA, FB, OUT, HAS_BIAS>(A, B, (int)M, (int)N, (int)K, sa, sb, bias, C,
                                                 qo, stream);
    if (large && fits32 && K >= 256)
        return launch_big<FA, FB, OUT, HAS_BIAS>(A, B, (int)M, (int)N, (int)K, sa, sb, bias, C,
                                                 qo, stream);
    // Small problems with fewer 128 x 128 tiles than CUs (few tokens, narrow
    // outputs: e.g. 1024 x 2048 with K = 8192 has 128) take 64 x 128 tiles,
    // twice as many, so that more CUs share the K loop.
    const int64_t tiles128 = ((M + 127) / 128) * ((N + 127) / 128);
    const bool half = tiles128 < cus;
    // Whole 128-byte K stages and 32-bit operand offsets: the operand stages
    // go straight into LDS.  Exactly one 128 x 128 tile per CU also takes
    // 64-row tiles there, two per CU (1024 x 4096 x 2048: 15.9 -> 14.7 us,
    // 2048 x 2048 x 2048: 16.0 -> 14.7); at 1.5 or 2 tiles per CU the
    // 128-row tiles stay faster (1024 x 6144 x 2048: 20.5 against 23.7).
    if (fits32 && K >= 256 && K % 128 == 0) {
        if (tiles128 <= cus)
            return launch_sdma<64, FA, FB, OUT, HAS_BIAS>(A, B, (int)M, (int)N, (int)K, sa, sb,
                                                          bias, C, qo, stream);
        return launch_sdma<128, FA, FB, OUT, HAS_BIAS>(A, B, (int)M, (int)N, (int)K, sa, sb, bias,
                                                       C, qo, stream);
    }
    if (half)
        return launch_cfg<64, 128, 2, 2, FA, FB, OUT, HAS_BIAS>(A, B, (int)M, (int)N, (int)K, sa,
                                                                sb, bias, C, qo, stream);
    return launch_cfg<128, 128, 2, 2, FA, FB, OUT, HAS_BIAS>(A, B, (int)M, (int)N, (int)K, sa, sb,
                                                             bias, C, qo, stream);
}

}  // namespace
}  // namespace fp8dsl
