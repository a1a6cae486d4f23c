// Micro-kernels that measure what the kernels' design assumes about gfx950:
// the achievable fp32 matrix-core rate (v_mfma_f32_16x16x4_f32) and whether
// vector-ALU work of one wave overlaps its own matrix-core work.  Test
// infrastructure only: built beside the tests, never part of libcssd.so.
//
// Each kernel runs `iters` iterations of a fixed instruction mix on every wave
// and writes one value per lane so that nothing is optimised away.
#include <hip/hip_runtime.h>

typedef float floatx4 __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// four independent accumulator chains of 16x16x4 fp32 MFMAs
__global__ __launch_bounds__(256) void k_probe_mfma(float* out, int iters) {
    const float x = 1e-3f * (float)(threadIdx.x & 63), y = 1e-3f;
    floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, a3 = a0;
    for (int i = 0; i < iters; ++i) {
        a0 = mfma4(x, y, a0);
        a1 = mfma4(y, x, a1);
        a2 = mfma4(x, x, a2);
        a3 = mfma4(y, y, a3);
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = a0[0] + a1[1] + a2[2] + a3[3];
}

// 16 dependent fp32 FMAs per iteration over four independent chains
__global__ __launch_bounds__(256) void k_probe_valu(float* out, int iters) {
    float v0 = 1e-3f * (float)(threadIdx.x & 63), v1 = v0 + 1.f, v2 = v0 + 2.f, v3 = v0 + 3.f;
    const float m = 0.999f, d = 1e-4f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v0 = __builtin_fmaf(v0, m, d);
            v1 = __builtin_fmaf(v1, m, d);
            v2 = __builtin_fmaf(v2, m, d);
            v3 = __builtin_fmaf(v3, m, d);
        }
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = v0 + v1 + v2 + v3;
}

// both mixes in the same wave: every iteration issues the four MFMAs and the
// sixteen FMAs of the two kernels above
__global__ __launch_bounds__(256) void k_probe_mixed(float* out, int iters) {
    const float x = 1e-3f * (float)(threadIdx.x & 63), y = 1e-3f;
    floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, a3 = a0;
    float v0 = x, v1 = v0 + 1.f, v2 = v0 + 2.f, v3 = v0 + 3.f;
    const float m = 0.999f, d = 1e-4f;
    for (int i = 0; i < iters; ++i) {
        a0 = mfma4(x, y, a0);
        a1 = mfma4(y, x, a1);
        a2 = mfma4(x, x, a2);
        a3 = mfma4(y, y, a3);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v0 = __builtin_fmaf(v0, m, d);
            v1 = __builtin_fmaf(v1, m, d);
            v2 = __builtin_fmaf(v2, m, d);
            v3 = __builtin_fmaf(v3, m, d);
        }
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = a0[0] + a1[1] + a2[2] + a3[3] + v0 + v1 + v2 + v3;
}

// workgroups of eight waves: waves 0-3 run the MFMA mix, waves 4-7 the VALU
// mix; the waves of a workgroup are dealt to the CU's four SIMDs in turn, so
// every SIMD holds one wave of each
__global__ __launch_bounds__(512) void k_probe_split(float* out, int iters) {
    if ((threadIdx.x >> 6) < 4) {
        const float x = 1e-3f * (float)(threadIdx.x & 63), y = 1e-3f;
        floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, a3 = a0;
        for (int i = 0; i < iters; ++i) {
            a0 = mfma4(x, y, a0);
            a1 = mfma4(y, x, a1);
            a2 = mfma4(x, x, a2);
            a3 = mfma4(y, y, a3);
        }
        out[blockIdx.x * blockDim.x + threadIdx.x] = a0[0] + a1[1] + a2[2] + a3[3];
    } else {
        float v0 = 1e-3f * (float)(threadIdx.x & 63), v1 = v0 + 1.f, v2 = v0 + 2.f, v3 = v0 + 3.f;
        const float m = 0.999f, d = 1e-4f;
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v0 = __builtin_fmaf(v0, m, d);
                v1 = __builtin_fmaf(v1, m, d);
                v2 = __builtin_fmaf(v2, m, d);
                v3 = __builtin_fmaf(v3, m, d);
            }
        }
        out[blockIdx.x * blockDim.x + threadIdx.x] = v0 + v1 + v2 + v3;
    }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void bf16_mix(float* out, int iters) {
    bf16x8 x, y;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[j] = (__bf16)(1e-3f * (float)((threadIdx.x + j) & 63));
        y[j] = (__bf16)1e-3f;
    }
    floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, a3 = a0;
    for (int i = 0; i < iters; ++i) {
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(y, x, a1, 0, 0, 0);
        a2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, x, a2, 0, 0, 0);
        a3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(y, y, a3, 0, 0, 0);
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = a0[0] + a1[1] + a2[2] + a3[3];
}

// four independent chains of 16x16x32 bf16 MFMAs
__global__ __launch_bounds__(256) void k_probe_bf16(float* out, int iters) { bf16_mix(out, iters); }

// waves 0-3 the bf16 MFMA mix, waves 4-7 the VALU mix (one of each per SIMD)
__global__ __launch_bounds__(512) void k_probe_split_bf16(float* out, int iters) {
    if ((threadIdx.x >> 6) < 4) {
        bf16_mix(out, iters);
    } else {
        float v0 = 1e-3f * (float)(threadIdx.x & 63), v1 = v0 + 1.f, v2 = v0 + 2.f, v3 = v0 + 3.f;
        const float m = 0.999f, d = 1e-4f;
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v0 = __builtin_fmaf(v0, m, d);
                v1 = __builtin_fmaf(v1, m, d);
                v2 = __builtin_fmaf(v2, m, d);
                v3 = __builtin_fmaf(v3, m, d);
            }
        }
        out[blockIdx.x * blockDim.x + threadIdx.x] = v0 + v1 + v2 + v3;
    }
}

}  // namespace

// kind 0: fp32 MFMA only, 1: VALU only, 2: both in one wave, 3: the two mixes in
// separate waves of one SIMD, 4: bf16 MFMA only, 5: bf16 MFMA and VALU in
// separate waves.  `blocks` workgroups of `threads` threads (a multiple of 64,
// at most 256, or 512 for kinds 3 and 5); `out` holds blocks x threads
// floats.  Returns the launch's hipError_t.
extern "C" int probe_launch(int kind, int blocks, int threads, int iters, float* out,
                            void* stream) {
    const int max_threads = (kind == 3 || kind == 5) ? 512 : 256;
    if (threads <= 0 || threads > max_threads || threads % 64 != 0 || blocks <= 0 || iters < 0 ||
        out == nullptr)
        return (int)hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (kind == 0)
        hipLaunchKernelGGL(k_probe_mfma, dim3(blocks), dim3(threads), 0, s, out, iters);
    else if (kind == 1)
        hipLaunchKernelGGL(k_probe_valu, dim3(blocks), dim3(threads), 0, s, out, iters);
    else if (kind == 2)
        hipLaunchKernelGGL(k_probe_mixed, dim3(blocks), dim3(threads), 0, s, out, iters);
    else if (kind == 3)
        hipLaunchKernelGGL(k_probe_split, dim3(blocks), dim3(threads), 0, s, out, iters);
    else if (kind == 4)
        hipLaunchKernelGGL(k_probe_bf16, dim3(blocks), dim3(threads), 0, s, out, iters);
    else if (kind == 5)
        hipLaunchKernelGGL(k_probe_split_bf16, dim3(blocks), dim3(threads), 0, s, out, iters);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}
