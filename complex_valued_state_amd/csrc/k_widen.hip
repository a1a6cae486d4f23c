// bf16 -> fp32 widening of an input plane.  The backward takes bf16 x, B, C by
// widening each plane once into its workspace and running the fp32 kernels on the
// values exactly as rounded (the widening is exact: a bf16 value is the top half
// of the fp32 with the same value).
#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

// thread i widens elements 8 i .. 8 i + 7 (16-byte load, two 16-byte stores);
// the last thread of a length that is not a multiple of 8 takes the rest singly
__global__ __launch_bounds__(256) void k_widen(const uint16_t* __restrict__ src,
                                               float* __restrict__ dst, int64_t n) {
    const int64_t i8 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i8 + 8 <= n) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + i8);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = __uint_as_float(u[k] << 16);
            f[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
        }
        *reinterpret_cast<float4*>(dst + i8) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4*>(dst + i8 + 4) = make_float4(f[4], f[5], f[6], f[7]);
    } else {
        for (int64_t i = i8; i < n; ++i) dst[i] = __uint_as_float((uint32_t)src[i] << 16);
    }
}

hipError_t launch_widen(const uint16_t* src, float* dst, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = ((n + 7) / 8 + 255) / 256;
    hipLaunchKernelGGL(k_widen, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace cssd
