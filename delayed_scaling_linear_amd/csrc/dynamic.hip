// Dynamic scaling, the comparator of delayed scaling.
//
// "support delayed scaling of weight in float8 all-gather" contrasts the two
// recipes: dynamic scaling derives a tensor's scale from that tensor's own
// amax, which takes a read of the tensor before the cast can start, while
// delayed scaling casts with a scale from earlier amaxes and takes the new
// amax in the cast's own read.  This file supplies the extra pieces dynamic
// scaling needs -- an amax-only pass and the scale derived from it -- so the
// two can be run and timed side by side; the cast is the library's ordinary
// cast kernel.
#include <algorithm>

#include "fp8dsl_internal.h"

namespace fp8dsl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// *p = v (a capturable way to clear a scalar: no memset node).
__global__ void set_scalar_kernel(float *__restrict__ p, float v, const int32_t *__restrict__ noop) {
    if (noop != nullptr && *noop != 0) return;
    *p = v;
}

// max |x| over a [rows, cols] tensor with row stride ld, as the sign-cleared
// fp32 bit pattern (so a NaN dominates), folded into *amax with atomicMax.
// Workgroups stride over groups of four rows (rows is a multiple of 16),
// threads over the rows' 16-byte chunks: four independent loads in flight
// per thread and step.
template <int SRC>
__global__ __launch_bounds__(256) void amax_kernel(const void *__restrict__ xv, int64_t rows,
                                                   int64_t cols, int64_t ld,
                                                   float *__restrict__ amax,
                                                   const int32_t *__restrict__ noop) {
    if (noop != nullptr && *noop != 0) return;
    constexpr int EB = (SRC == FP8_DTYPE_BF16) ? 2 : 4;
    const uint8_t *x = static_cast<const uint8_t *>(xv);
    const int64_t chunks = cols * EB / 16;
    uint32_t key = 0;
    for (int64_t r0 = (int64_t)blockIdx.x * 4; r0 < rows; r0 += (int64_t)gridDim.x * 4) {
        const uint8_t *row = x + r0 * ld * EB;
        for (int64_t ch = threadIdx.x; ch < chunks; ch += 256) {
            u32x4 v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = *reinterpret_cast<const u32x4 *>(row + (int64_t)i * ld * EB + ch * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if constexpr (SRC == FP8_DTYPE_BF16) {
                        const uint32_t m = d[k] & 0x7FFF7FFFu;
                        key = max(key, max(m << 16, m & 0xFFFF0000u));
                    } else {
                        key = max(key, d[k] & 0x7FFFFFFFu);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) key = max(key, (uint32_t)__shfl_xor((int)key, off, 64));
    __shared__ uint32_t lds[4];
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t k = max(max(lds[0], lds[1]), max(lds[2], lds[3]));
        unsigned int *a = reinterpret_cast<unsigned int *>(amax);
        if (k > __atomic_load_n(a, __ATOMIC_RELAXED)) atomicMax(a, k);
    }
}

// scale = fp8_max / (amax * 2^margin), the guard of the scale update: the
// scale is kept when amax is zero or not finite or the quotient is not a
// finite positive number.
__global__ void dynamic_scale_kernel(const float *__restrict__ amax, float *__restrict__ scale,
                                     int fmt, int margin, const int32_t *__restrict__ noop) {
    if (noop != nullptr && *noop != 0) return;
    const float m = *amax;
    if (m > 0.0f && m <= 3.402823466e38f) {
        const float fp8_max = (fmt == FP8_E4M3) ? 448.0f : 57344.0f;
        const float q = fp8_max / ldexpf(m, margin);
        if (q > 0.0f && q <= 3.402823466e38f) *scale = q;
    }
}

}  // namespace

hipError_t launch_dynamic_scale(const void *x, int src, int64_t rows, int64_t cols, int64_t ld,
                                int fmt, int margin, float *amax, float *scale,
                                const int32_t *noop, hipStream_t stream) {
    int cus = 0;
    if (hipError_t e = current_cu_count(&cus)) return e;
    hipLaunchKernelGGL(set_scalar_kernel, dim3(1), dim3(1), 0, stream, amax, 0.0f, noop);
    if (rows > 0 && cols > 0) {
        // Two workgroups per CU, each striding over many row groups: few
        // atomics on the one amax word.
        const dim3 grid((unsigned)std::min<int64_t>(rows / 4, (int64_t)cus * 2));
        if (src == FP8_DTYPE_BF16)
            hipLaunchKernelGGL(amax_kernel<FP8_DTYPE_BF16>, grid, dim3(256), 0, stream, x, rows,
                               cols, ld, amax, noop);
        else
            hipLaunchKernelGGL(amax_kernel<FP8_DTYPE_FP32>, grid, dim3(256), 0, stream, x, rows,
                               cols, ld, amax, noop);
    }
    hipLaunchKernelGGL(dynamic_scale_kernel, dim3(1), dim3(1), 0, stream, amax, scale, fmt, margin,
                       noop);
    return hipGetLastError();
}

}  // namespace fp8dsl
