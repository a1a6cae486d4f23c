// Device helpers shared by the cssd kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cssd {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

// One 16x16x4 fp32 matrix-core step: acc += A(16x4) * B(4x16).
// Lane layout (wave64): lane = i + 16*k holds A[i][k] and B[k][j=i];
// accumulator register r of lane (j + 16*g) is D[4*g + r][j].
__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ double softplus_f64(double v) {
    return fmax(v, 0.0) + log1p(exp(-fabs(v)));
}

// Wrap a phase (radians) into [-pi, pi] in fp64 before it is narrowed to fp32.
__device__ __forceinline__ double wrap_phase(double v) {
    return v - kTwoPi * rint(v * kInvTwoPi);
}

// ----------------------------------------------------------------------------
// Input planes are float32 or bfloat16 bit patterns; arithmetic is fp32.
// ----------------------------------------------------------------------------
struct InF32 {
    typedef float T;
    __device__ __forceinline__ static float load1(const float* p) { return *p; }
    __device__ __forceinline__ static float4 load4(const float* p) {
        return *reinterpret_cast<const float4*>(p);
    }
};

struct InBF16 {
    typedef uint16_t T;
    __device__ __forceinline__ static float cvt(uint32_t bits16) {
        return __uint_as_float(bits16 << 16);
    }
    __device__ __forceinline__ static float load1(const uint16_t* p) { return cvt(*p); }
    __device__ __forceinline__ static float4 load4(const uint16_t* p) {
        uint2 v = *reinterpret_cast<const uint2*>(p);
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
    }
};

// Streaming (non-temporal) float4 accesses for data touched once per launch.
__device__ __forceinline__ float4 nt_load4(const float4* p) {
    const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void nt_store4(const float4& v, float4* p) {
    const floatx4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<floatx4*>(p));
}

__device__ __forceinline__ float f4get(const float4& v, int q) {
    return q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
}

}  // namespace cssd
