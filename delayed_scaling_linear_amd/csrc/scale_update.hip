// Delayed-scaling update of every scaled tensor of a model in one launch.
//
// The recipe is the DelayedScaling one of "CPU Overhead of te.Linear FP8
// Layers" (amax history of length 16, reduced with "max"); TE runs its scale
// update for every FP8 tensor each forward pass ("[PyTorch] Refactor FP8
// workspaces in linear modules"), and float8_experimental packs all amaxes
// into one tensor and syncs them once per step ("support delayed scaling of
// weight in float8 all-gather").  Here one thread owns one tensor record, so
// a model's 384 records take one small launch instead of one per tensor.
//
// The pages do not print the scale formula.  The conventional reading is
// used: scale = fp8_max / (max(history) * 2^margin), kept when the history
// maximum is zero or not finite, or when the quotient is not a finite
// positive fp32.  Division and reciprocal are IEEE correctly rounded (the
// library is built without fast-math and with correctly rounded fp32
// division), so the result is bit-identical to any IEEE implementation.
#include "fp8dsl_internal.h"

namespace fp8dsl {
namespace {

__device__ __forceinline__ uint32_t abs_key(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

__device__ __forceinline__ void finish_record(uint32_t best, uint8_t f, int margin, float *scale,
                                              float *scale_inv, float *amax_cur, int t) {
    float m = __uint_as_float(best);
    float s = scale[t];
    if (m > 0.0f && m <= 3.402823466e38f) {           // finite and positive (NaN fails)
        const float fp8_max = (f == FP8_E4M3) ? 448.0f : 57344.0f;
        float q = fp8_max / ldexpf(m, margin);
        if (q > 0.0f && q <= 3.402823466e38f) s = q;
    }
    scale[t] = s;
    scale_inv[t] = 1.0f / s;
    amax_cur[t] = 0.0f;
}

// H == 16 with a 16-byte aligned history: the row moves as four float4s.
__global__ __launch_bounds__(256) void scale_update_h16(float *__restrict__ hist,
                                                        float *__restrict__ amax_cur,
                                                        float *__restrict__ scale,
                                                        float *__restrict__ scale_inv,
                                                        const uint8_t *__restrict__ fmt, int T,
                                                        int margin) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const uint8_t f = fmt[t];
    if (f > FP8_E5M2) return;
    float4 *row = reinterpret_cast<float4 *>(hist + (int64_t)t * 16);
    float4 r0 = row[0], r1 = row[1], r2 = row[2], r3 = row[3];
    const float cur = amax_cur[t];
    // New window: cur, old[0..14]; old[15] drops out.
    float4 n0 = make_float4(cur, r0.x, r0.y, r0.z);
    float4 n1 = make_float4(r0.w, r1.x, r1.y, r1.z);
    float4 n2 = make_float4(r1.w, r2.x, r2.y, r2.z);
    float4 n3 = make_float4(r2.w, r3.x, r3.y, r3.z);
    row[0] = n0; row[1] = n1; row[2] = n2; row[3] = n3;
    uint32_t best = abs_key(n0.x);
    best = max(best, abs_key(n0.y)); best = max(best, abs_key(n0.z)); best = max(best, abs_key(n0.w));
    best = max(best, abs_key(n1.x)); best = max(best, abs_key(n1.y)); best = max(best, abs_key(n1.z));
    best = max(best, abs_key(n1.w)); best = max(best, abs_key(n2.x)); best = max(best, abs_key(n2.y));
    best = max(best, abs_key(n2.z)); best = max(best, abs_key(n2.w)); best = max(best, abs_key(n3.x));
    best = max(best, abs_key(n3.y)); best = max(best, abs_key(n3.z)); best = max(best, abs_key(n3.w));
    finish_record(best, f, margin, scale, scale_inv, amax_cur, t);
}

// Any history length.
__global__ __launch_bounds__(256) void scale_update_generic(float *__restrict__ hist,
                                                            float *__restrict__ amax_cur,
                                                            float *__restrict__ scale,
                                                            float *__restrict__ scale_inv,
                                                            const uint8_t *__restrict__ fmt,
                                                            int T, int H, int margin) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const uint8_t f = fmt[t];
    if (f > FP8_E5M2) return;
    float *row = hist + (int64_t)t * H;
    float carry = amax_cur[t];
    uint32_t best = 0;
    for (int i = 0; i < H; ++i) {
        const float old = row[i];
        row[i] = carry;
        best = max(best, abs_key(carry));
        carry = old;
    }
    finish_record(best, f, margin, scale, scale_inv, amax_cur, t);
}

}  // namespace

hipError_t launch_scale_update(float *hist, float *amax_cur, float *scale, float *scale_inv,
                               const uint8_t *fmt, int T, int H, int margin,
                               hipStream_t stream) {
    const int threads = 256;
    const int blocks = (T + threads - 1) / threads;
    if (H == 16 && (reinterpret_cast<uintptr_t>(hist) & 15) == 0) {
        hipLaunchKernelGGL(scale_update_h16, dim3(blocks), dim3(threads), 0, stream, hist,
                           amax_cur, scale, scale_inv, fmt, T, margin);
    } else {
        hipLaunchKernelGGL(scale_update_generic, dim3(blocks), dim3(threads), 0, stream, hist,
                           amax_cur, scale, scale_inv, fmt, T, H, margin);
    }
    return hipGetLastError();
}

}  // namespace fp8dsl
