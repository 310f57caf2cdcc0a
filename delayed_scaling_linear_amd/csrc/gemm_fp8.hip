// The bf16 / fp32-output instantiations of the per-tensor-scaled FP8 matrix
// product (the kernels are in gemm_fp8_kernels.h): the forward, dgrad and
// wgrad products of te.Linear ("CPU Overhead of te.Linear FP8 Layers") as
// torch._scaled_mm computes them ("Accelerating PyTorch Training Workloads
// with FP8 -- Part 2").
#include "gemm_fp8_kernels.h"

namespace fp8dsl {
namespace {

template <int FA, int FB>
hipError_t launch_out(const uint8_t *A, const uint8_t *B, int64_t M, int64_t N, int64_t K,
                      const float *sa, const float *sb, const uint16_t *bias, int out, void *C,
                      hipStream_t stream, void *ws, int64_t wsb) {
    const QOut none{nullptr, nullptr, nullptr};
    if (out == FP8_DTYPE_BF16) {
        if (bias)
            return launch_fmt<FA, FB, FP8_DTYPE_BF16, true>(A, B, M, N, K, sa, sb, bias, C, none,
                                                            stream, ws, wsb);
        return launch_fmt<FA, FB, FP8_DTYPE_BF16, false>(A, B, M, N, K, sa, sb, bias, C, none,
                                                         stream, ws, wsb);
    }
    if (bias)
        return launch_fmt<FA, FB, FP8_DTYPE_FP32, true>(A, B, M, N, K, sa, sb, bias, C, none,
                                                        stream, ws, wsb);
    return launch_fmt<FA, FB, FP8_DTYPE_FP32, false>(A, B, M, N, K, sa, sb, bias, C, none, stream,
                                                     ws, wsb);
}

}  // namespace

hipError_t launch_gemm_nt(const uint8_t *A, int fa, const uint8_t *B, int fb, int64_t M,
                          int64_t N, int64_t K, const float *sinv_a, const float *sinv_b,
                          const uint16_t *bias, int out_dtype, void *C, hipStream_t stream,
                          void *ws, int64_t wsb) {
    if (fa == FP8_E4M3 && fb == FP8_E4M3)
        return launch_out<FP8_E4M3, FP8_E4M3>(A, B, M, N, K, sinv_a, sinv_b, bias, out_dtype, C, stream, ws, wsb);
    if (fa == FP8_E5M2 && fb == FP8_E4M3)
        return launch_out<FP8_E5M2, FP8_E4M3>(A, B, M, N, K, sinv_a, sinv_b, bias, out_dtype, C, stream, ws, wsb);
    if (fa == FP8_E4M3 && fb == FP8_E5M2)
        return launch_out<FP8_E4M3, FP8_E5M2>(A, B, M, N, K, sinv_a, sinv_b, bias, out_dtype, C, stream, ws, wsb);
    return launch_out<FP8_E5M2, FP8_E5M2>(A, B, M, N, K, sinv_a, sinv_b, bias, out_dtype, C, stream, ws, wsb);
}

}  // namespace fp8dsl
