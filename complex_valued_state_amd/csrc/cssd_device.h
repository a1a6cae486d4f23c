// Device helpers shared by the cssd kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cssd {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
constexpr double kLog2e = 1.4426950408889634073599246810019;

// One 16x16x4 fp32 matrix-core step: acc += A(16x4) * B(4x16).
// Lane layout (wave64): lane = i + 16*k holds A[i][k] and B[k][j=i];
// accumulator register r of lane (j + 16*g) is D[4*g + r][j].
__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Complex multiply-accumulate of 16x16 tiles with three real MFMA products
// (Gauss): t1 += ar br, t2 += ai bi, t3 += (ar + ai)(br + bi); then
// re = t1 - t2 and im = t3 - t1 - t2.  The caller passes the operand sums.
struct CTile {
    floatx4 t1, t2, t3;
};
__device__ __forceinline__ void ctile_zero(CTile& a) {
    a.t1 = floatx4{0.f, 0.f, 0.f, 0.f};
    a.t2 = a.t1;
    a.t3 = a.t1;
}
__device__ __forceinline__ void ctile_mac(CTile& a, float ar, float ai, float as, float br,
                                          float bi, float bs) {
    a.t1 = mfma4(ar, br, a.t1);
    a.t2 = mfma4(ai, bi, a.t2);
    a.t3 = mfma4(as, bs, a.t3);
}
__device__ __forceinline__ float ctile_re(const CTile& a, int r) { return a.t1[r] - a.t2[r]; }
__device__ __forceinline__ float ctile_im(const CTile& a, int r) {
    return a.t3[r] - a.t1[r] - a.t2[r];
}

// exp(re + i im) for an increment given in log2 units (re2 = re / ln 2) and in
// turns (rev = im / 2 pi, already reduced to [-1/2, 1/2]), on the hardware
// transcendental units: v_exp_f32 computes 2^x, v_sin_f32 / v_cos_f32 take turns.
__device__ __forceinline__ void cexp_scaled(float re2, float rev, float& out_re, float& out_im) {
    const float mag = __builtin_amdgcn_exp2f(re2);
    out_re = mag * __builtin_amdgcn_cosf(rev);
    out_im = mag * __builtin_amdgcn_sinf(rev);
}

// Index of this wave in its workgroup, as a value the compiler knows is
// wave-uniform (so that everything derived from it lives in scalar registers).
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// x moved across lanes by a DPP pattern (both 32-bit halves); lanes the pattern
// or the row mask leaves without a source read 0
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xf, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xf, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// inclusive prefix sum over the 64 lanes in fp64: shifts right by 1, 2, 4, 8
// within each row of 16 lanes, then row 0's total into rows 1 and 3
// (row_bcast:15) and rows 0-1's total into rows 2 and 3 (row_bcast:31).  The
// moves stay in the vector unit (a shuffle-based scan goes through LDS with
// ds_bpermute); the association of the sums differs from a lane-by-lane scan's
// only by fp64 rounding
__device__ __forceinline__ void wave_inclusive_scan(double& v) {
    v += dpp_f64<0x111, 0xf>(v);  // row_shr:1
    v += dpp_f64<0x112, 0xf>(v);  // row_shr:2
    v += dpp_f64<0x114, 0xf>(v);  // row_shr:4
    v += dpp_f64<0x118, 0xf>(v);  // row_shr:8
    v += dpp_f64<0x142, 0xa>(v);  // row_bcast:15
    v += dpp_f64<0x143, 0xc>(v);  // row_bcast:31
}

// the value of lane `l` (wave-uniform l), through the scalar unit
__device__ __forceinline__ double lane_value(double v, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double softplus_f64(double v) {
    return fmax(v, 0.0) + log1p(exp(-fabs(v)));
}

// ----------------------------------------------------------------------------
// Raw buffer accesses: a wave-uniform base and extent in SGPRs, 32-bit per-lane
// element offsets.  A read at or beyond the extent returns 0 and a write there
// is dropped, which is how the kernels mask the padded rows of a partial chunk.
// ----------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t BufRes;
__device__ __forceinline__ BufRes make_buf(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ float buf_f32(BufRes r, uint32_t elem) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, elem * 4u, 0, 0));
}
__device__ __forceinline__ floatx4 buf_f32x4(BufRes r, uint32_t elem) {
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, elem * 4u, 0, 0));
}
__device__ __forceinline__ void buf_store_f32(float v, BufRes r, uint32_t elem) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, elem * 4u, 0, 0);
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
    // buffer forms (element offsets), see make_buf
    __device__ __forceinline__ static float bload1(BufRes r, uint32_t e) { return buf_f32(r, e); }
    __device__ __forceinline__ static floatx4 bload4(BufRes r, uint32_t e) {
        return buf_f32x4(r, e);
    }
    // elements e, e + 1 (e even)
    __device__ __forceinline__ static float2 bload2(BufRes r, uint32_t e) {
        return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, e * 4u, 0, 0));
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
    __device__ __forceinline__ static float bload1(BufRes r, uint32_t e) {
        return cvt(__builtin_amdgcn_raw_buffer_load_b16(r, e * 2u, 0, 0));
    }
    __device__ __forceinline__ static floatx4 bload4(BufRes r, uint32_t e) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, e * 2u, 0, 0));
        return floatx4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
                       __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u)};
    }
    // elements e, e + 1 (e even)
    __device__ __forceinline__ static float2 bload2(BufRes r, uint32_t e) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, e * 2u, 0, 0);
        return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
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
