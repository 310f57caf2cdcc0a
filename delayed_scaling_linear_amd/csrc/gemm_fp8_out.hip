// The FP8-output instantiations of the per-tensor-scaled FP8 matrix product
// (the kernels are in gemm_fp8_kernels.h).
//
// torch._scaled_mm called with an FP8 out_dtype ("Accelerating PyTorch
// Training Workloads with FP8 -- Part 2", the torch._scaled_mm example)
// returns the FP8 output and its amax.  Here the epilogue casts the fp32
// value v = acc * sinv_a * sinv_b + bias with the output's own (delayed)
// scale, exactly as the cast kernel encodes, and takes the amax of the
// unscaled v in the same pass: no bf16 round trip through HBM and no second
// read for the amax.
#include "gemm_fp8_kernels.h"

namespace fp8dsl {
namespace {

template <int FA, int FB, int OUT>
hipError_t launch_q_bias(const uint8_t *A, const uint8_t *B, int64_t M, int64_t N, int64_t K,
                         const float *sa, const float *sb, const uint16_t *bias, void *C,
                         const QOut &qo, hipStream_t stream) {
    if (bias) return launch_fmt<FA, FB, OUT, true>(A, B, M, N, K, sa, sb, bias, C, qo, stream);
    return launch_fmt<FA, FB, OUT, false>(A, B, M, N, K, sa, sb, bias, C, qo, stream);
}

template <int FA, int FB>
hipError_t launch_q(const uint8_t *A, const uint8_t *B, int64_t M, int64_t N, int64_t K,
                    const float *sa, const float *sb, const uint16_t *bias, int fo, void *C,
                    const QOut &qo, hipStream_t stream) {
    if (fo == FP8_E4M3)
        return launch_q_bias<FA, FB, OUT_E4M3>(A, B, M, N, K, sa, sb, bias, C, qo, stream);
    return launch_q_bias<FA, FB, OUT_E5M2>(A, B, M, N, K, sa, sb, bias, C, qo, stream);
}

}  // namespace

hipError_t launch_gemm_nt_fp8out(const uint8_t *A, int fa, const uint8_t *B, int fb, int64_t M,
                                 int64_t N, int64_t K, const float *sinv_a, const float *sinv_b,
                                 const uint16_t *bias, int fo, const float *scale_out,
                                 uint8_t *C, float *amax, float *scale_inv, hipStream_t stream) {
    const QOut qo{scale_out, amax, scale_inv};
    if (fa == FP8_E4M3 && fb == FP8_E4M3)
        return launch_q<FP8_E4M3, FP8_E4M3>(A, B, M, N, K, sinv_a, sinv_b, bias, fo, C, qo, stream);
    if (fa == FP8_E5M2 && fb == FP8_E4M3)
        return launch_q<FP8_E5M2, FP8_E4M3>(A, B, M, N, K, sinv_a, sinv_b, bias, fo, C, qo, stream);
    if (fa == FP8_E4M3 && fb == FP8_E5M2)
        return launch_q<FP8_E4M3, FP8_E5M2>(A, B, M, N, K, sinv_a, sinv_b, bias, fo, C, qo, stream);
    return launch_q<FP8_E5M2, FP8_E5M2>(A, B, M, N, K, sinv_a, sinv_b, bias, fo, C, qo, stream);
}

}  // namespace fp8dsl
