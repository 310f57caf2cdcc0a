// Per-tensor-scaled FP8 GEMM, "NT" layout, on CDNA4 FP8 matrix cores.
//
//   C[i, j] = out( (sum_k dec(A[i, k]) * dec(B[j, k])) * sinv_a * sinv_b + bias[j] )
//
// This is torch._scaled_mm of "Accelerating PyTorch Training Workloads with
// FP8 -- Part 2" (row-major first operand, transposed second operand,
// per-tensor scales held on the device, optional bf16 bias), used for the
// forward, dgrad and wgrad products of te.Linear ("CPU Overhead of te.Linear
// FP8 Layers").  Every FP8 x FP8 product is exact in fp32; accumulation is
// fp32 in the matrix cores.
//
// Design (gfx950, wave64):
//   * v_mfma_f32_16x16x128_f8f6f4 with per-operand format select (E4M3 /
//     E5M2), 8192 FLOP per instruction;
//   * block tile BM x BN, K step 128 bytes, waves arranged WM x WN, each wave
//     owning a (BM/WM) x (BN/WN) accumulator tile in AGPRs/VGPRs;
//   * A and B K-slabs staged through LDS, double-buffered: the global loads
//     of step k+1 are in flight while the matrix cores work on step k;
//   * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk
//     c ^ (r & 7), so both the row-wise stores and the fragment reads (8 lanes
//     on 8 consecutive rows) touch 8 distinct chunks: no bank conflicts;
//   * the B fragment is fed as the matrix core's first operand, so each lane
//     ends up holding four consecutive output columns of one output row: the
//     epilogue applies sinv_a * sinv_b and the bias in fp32 and writes 8-byte
//     (bf16) or 16-byte (fp32) vectors;
//   * M and N tails: out-of-range operand rows are clamped to the last valid
//     row for loading and never stored; a K tail (K % 128 != 0) is zero-filled.
#include "fp8dsl_internal.h"

namespace fp8dsl {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 128;

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;   // NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, bool HAS_BIAS>
__global__ __launch_bounds__(WM *WN * 64) void gemm_nt_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, int M, int N, int K,
    const float *__restrict__ sinv_a, const float *__restrict__ sinv_b,
    const uint16_t *__restrict__ bias, void *__restrict__ Cv, int tiles_n) {
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

    const int tile_m = blockIdx.x / tiles_n;
    const int tile_n = blockIdx.x - tile_m * tiles_n;
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN;

    // Loader bookkeeping: chunk id = tid + i*NT -> (row = id / 8, kc = id % 8).
    const uint8_t *a_src[LA];
    const uint8_t *b_src[LB];
    int a_lds[LA], b_lds[LB], a_kc[LA], b_kc[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int id = tid + i * NT;
        const int row = id >> 3, kc = id & 7;
        const int grow = min(m0 + row, M - 1);
        a_src[i] = A + (int64_t)grow * K + kc * 16;
        a_lds[i] = row * BK + ((kc ^ (row & 7)) << 4);
        a_kc[i] = kc * 16;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int id = tid + i * NT;
        const int row = id >> 3, kc = id & 7;
        const int grow = min(n0 + row, N - 1);
        b_src[i] = B + (int64_t)grow * K + kc * 16;
        b_lds[i] = BM * BK + row * BK + ((kc ^ (row & 7)) << 4);
        b_kc[i] = kc * 16;
    }

    u32x4 ra[LA], rb[LB];
    auto load_global = [&](int k0) {
        const bool full = (k0 + BK) <= K;
#pragma unroll
        for (int i = 0; i < LA; ++i) {
            if (full || k0 + a_kc[i] < K)
                ra[i] = *reinterpret_cast<const u32x4 *>(a_src[i] + k0);
            else
                ra[i] = u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            if (full || k0 + b_kc[i] < K)
                rb[i] = *reinterpret_cast<const u32x4 *>(b_src[i] + k0);
            else
                rb[i] = u32x4{0, 0, 0, 0};
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
    if (nk > 0) {
        load_global(0);
        store_lds(0);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int stage = kt & 1;
        if (kt + 1 < nk) load_global((kt + 1) * BK);

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
                const u32x2 o = u32x2{f32_to_bf16_rne(y0) | (f32_to_bf16_rne(y1) << 16),
                                      f32_to_bf16_rne(y2) | (f32_to_bf16_rne(y3) << 16)};
                *reinterpret_cast<u32x2 *>(C + (int64_t)gr * N + gc) = o;
            } else {
                float *C = static_cast<float *>(Cv);
                *reinterpret_cast<v4f *>(C + (int64_t)gr * N + gc) = v4f{y0, y1, y2, y3};
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int OUT, bool HAS_BIAS>
hipError_t launch_cfg(const uint8_t *A, const uint8_t *B, int M, int N, int K, const float *sa,
                      const float *sb, const uint16_t *bias, void *C, hipStream_t stream) {
    auto kern = gemm_nt_kernel<BM, BN, WM, WN, FA, FB, OUT, HAS_BIAS>;
    constexpr int lds_bytes = 2 * (BM + BN) * BK;
    // Dynamic LDS above 64 KiB must be enabled once per device and kernel.
    static bool attr_set[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!attr_set[dev]) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
        if (e != hipSuccess) return e;
        attr_set[dev] = true;
    }
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(WM * WN * 64), lds_bytes, stream, A, B,
                       M, N, K, sa, sb, bias, C, tiles_n);
    return hipGetLastError();
}

template <int FA, int FB, int OUT, bool HAS_BIAS>
hipError_t launch_fmt(const uint8_t *A, const uint8_t *B, int64_t M, int64_t N, int64_t K,
                      const float *sa, const float *sb, const uint16_t *bias, void *C,
                      hipStream_t stream) {
    // Large problems: 256 x 256 tiles (128 x 128 per wave); small ones: 128 x 128.
    if (M * N >= (int64_t)256 * 256 * 256)
        return launch_cfg<256, 256, 2, 2, FA, FB, OUT, HAS_BIAS>(A, B, (int)M, (int)N, (int)K, sa,
                                                                 sb, bias, C, stream);
    return launch_cfg<128, 128, 2, 2, FA, FB, OUT, HAS_BIAS>(A, B, (int)M, (int)N, (int)K, sa, sb,
                                                             bias, C, stream);
}

template <int FA, int FB>
hipError_t launch_out(const uint8_t *A, const uint8_t *B, int64_t M, int64_t N, int64_t K,
                      const float *sa, const float *sb, const uint16_t *bias, int out, void *C,
                      hipStream_t stream) {
    if (out == FP8_DTYPE_BF16) {
        if (bias) return launch_fmt<FA, FB, FP8_DTYPE_BF16, true>(A, B, M, N, K, sa, sb, bias, C, stream);
        return launch_fmt<FA, FB, FP8_DTYPE_BF16, false>(A, B, M, N, K, sa, sb, bias, C, stream);
    }
    if (bias) return launch_fmt<FA, FB, FP8_DTYPE_FP32, true>(A, B, M, N, K, sa, sb, bias, C, stream);
    return launch_fmt<FA, FB, FP8_DTYPE_FP32, false>(A, B, M, N, K, sa, sb, bias, C, stream);
}

}  // namespace

hipError_t launch_gemm_nt(const uint8_t *A, int fa, const uint8_t *B, int fb, int64_t M,
                          int64_t N, int64_t K, const float *sinv_a, const float *sinv_b,
                          const uint16_t *bias, int out_dtype, void *C, hipStream_t stream) {
    if (fa == FP8_E4M3 && fb == FP8_E4M3)
        return launch_out<FP8_E4M3, FP8_E4M3>(A, B, M, N, K, sinv_a, sinv_b, bias, out_dtype, C, stream);
    if (fa == FP8_E5M2 && fb == FP8_E4M3)
        return launch_out<FP8_E5M2, FP8_E4M3>(A, B, M, N, K, sinv_a, sinv_b, bias, out_dtype, C, stream);
    if (fa == FP8_E4M3 && fb == FP8_E5M2)
        return launch_out<FP8_E4M3, FP8_E5M2>(A, B, M, N, K, sinv_a, sinv_b, bias, out_dtype, C, stream);
    return launch_out<FP8_E5M2, FP8_E5M2>(A, B, M, N, K, sinv_a, sinv_b, bias, out_dtype, C, stream);
}

}  // namespace fp8dsl
