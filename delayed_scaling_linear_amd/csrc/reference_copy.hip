// Measurement reference, not part of the method: a plain device-to-device
// copy with 16-byte accesses.  The cast-transpose-amax moves the same bytes
// as a copy (one read of the source, one write of the codes and of their
// transpose), so a copy of that volume is the ceiling the cast is measured
// against on the same device.
#include "fp8dsl_internal.h"

namespace fp8dsl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup b copies 16 KiB slabs b, b + gridDim.x, ...: each thread loads
// four 16-byte chunks 4 KiB apart, then stores them (all loads of a slab in
// flight before its stores).
template <bool NT>
__global__ __launch_bounds__(256) void reference_copy_kernel(const u32x4 *__restrict__ src,
                                                             u32x4 *__restrict__ dst, int64_t n) {
    constexpr int64_t SLAB = 4 * 256;   // 16-byte chunks per slab
    for (int64_t base = (int64_t)blockIdx.x * SLAB; base < n; base += (int64_t)gridDim.x * SLAB) {
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = base + k * 256 + threadIdx.x;
            if (i < n) v[k] = NT ? __builtin_nontemporal_load(src + i) : src[i];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = base + k * 256 + threadIdx.x;
            if (i < n) dst[i] = v[k];
        }
    }
}

}  // namespace

hipError_t launch_reference_copy(const void *src, void *dst, int64_t bytes, int blocks,
                                 bool nontemporal, hipStream_t stream) {
    const int64_t n = bytes / 16;
    const auto *s = static_cast<const u32x4 *>(src);
    auto *d = static_cast<u32x4 *>(dst);
    if (nontemporal)
        hipLaunchKernelGGL(reference_copy_kernel<true>, dim3(blocks), dim3(256), 0, stream, s, d, n);
    else
        hipLaunchKernelGGL(reference_copy_kernel<false>, dim3(blocks), dim3(256), 0, stream, s, d, n);
    return hipGetLastError();
}

}  // namespace fp8dsl
