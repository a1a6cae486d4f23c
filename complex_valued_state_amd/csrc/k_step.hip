// K5: one recurrent decode step for every (batch, head), state updated in place.
//
//   abar = exp(softplus(dt) A);  h[n, :] <- abar h[n, :] + B[n] x;  y = sum_n C[n] h[n, :] + D x
//
// The loop body of the sequential scan (Mamba-3-Lite docs, "Complex-Valued
// State Spaces", walkthrough of the naive scan; "SSD Theory" section 2 notes
// that each step reads and writes the whole state with no reuse, so this is
// bound by memory bandwidth).  The skip term follows the burn-mamba
// step_constant readout.
//
// Mapping: one 256-thread workgroup per (b, h).  The N x D state is streamed as
// float4 rows: D/4 threads cover one row of p, 1024/D rows per pass.  Each
// thread issues all its state loads (non-temporal: the state is touched once
// per step) before the dependent updates, keeps a partial y for its four p
// columns, and the partials are reduced over rows through LDS.  abar is formed
// in fp64 and rounded once to fp32.
#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

template <int N, int D>
__global__ __launch_bounds__(256) void k_step(
    const float* __restrict__ x_re, const float* __restrict__ x_im,
    const float* __restrict__ b_re, const float* __restrict__ b_im,
    const float* __restrict__ c_re, const float* __restrict__ c_im, const float* __restrict__ dt,
    const float* __restrict__ a_re, const float* __restrict__ a_im,
    const float* __restrict__ dskip, float4* __restrict__ h_re, float4* __restrict__ h_im,
    float* __restrict__ y_re, float* __restrict__ y_im, int H) {
    constexpr int TPR = D / 4;                  // threads per state row
    constexpr int RPP = 256 / TPR;              // rows per pass
    constexpr int PASSES = (N + RPP - 1) / RPP;
    const int tid = threadIdx.x;
    const int pc = tid % TPR, rg = tid / TPR;
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % H);

    const double s = softplus_f64((double)dt[bh]);
    const double mag = exp(s * (double)a_re[h]);
    double sn, cs;
    sincos(s * (double)a_im[h], &sn, &cs);
    const float ar = (float)(mag * cs), ai = (float)(mag * sn);

    const float4 xr = reinterpret_cast<const float4*>(x_re + bh * D)[pc];
    const float4 xi = reinterpret_cast<const float4*>(x_im + bh * D)[pc];
    const int64_t sbase = bh * (int64_t)N * (D / 4) + pc;

    float4 hr[PASSES], hi[PASSES];
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
        const int n = rg + k * RPP;
        if (n < N) {
            hr[k] = nt_load4(&h_re[sbase + (int64_t)n * (D / 4)]);
            hi[k] = nt_load4(&h_im[sbase + (int64_t)n * (D / 4)]);
        }
    }
    float4 yr = make_float4(0.f, 0.f, 0.f, 0.f), yi = yr;
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
        const int n = rg + k * RPP;
        if (n < N) {
            const float br = b_re[bh * N + n], bi = b_im[bh * N + n];
            const float cr = c_re[bh * N + n], ci = c_im[bh * N + n];
            float4 nr, ni;
#define CSSD_UPD(f)                                                           \
    nr.f = ar * hr[k].f - ai * hi[k].f + (br * xr.f - bi * xi.f);             \
    ni.f = ar * hi[k].f + ai * hr[k].f + (br * xi.f + bi * xr.f);             \
    yr.f += cr * nr.f - ci * ni.f;                                            \
    yi.f += cr * ni.f + ci * nr.f;
            CSSD_UPD(x)
            CSSD_UPD(y)
            CSSD_UPD(z)
            CSSD_UPD(w)
#undef CSSD_UPD
            nt_store4(nr, &h_re[sbase + (int64_t)n * (D / 4)]);
            nt_store4(ni, &h_im[sbase + (int64_t)n * (D / 4)]);
        }
    }
    __shared__ float4 red_r[256], red_i[256];
    red_r[tid] = yr;
    red_i[tid] = yi;
    __syncthreads();
    if (tid < TPR) {
        float4 sr = red_r[tid], si = red_i[tid];
        for (int k = 1; k < RPP; ++k) {
            const float4 vr = red_r[k * TPR + tid], vi = red_i[k * TPR + tid];
            sr.x += vr.x; sr.y += vr.y; sr.z += vr.z; sr.w += vr.w;
            si.x += vi.x; si.y += vi.y; si.z += vi.z; si.w += vi.w;
        }
        const float dk = dskip != nullptr ? dskip[h] : 0.f;
        sr.x += dk * xr.x; sr.y += dk * xr.y; sr.z += dk * xr.z; sr.w += dk * xr.w;
        si.x += dk * xi.x; si.y += dk * xi.y; si.z += dk * xi.z; si.w += dk * xi.w;
        reinterpret_cast<float4*>(y_re + bh * D)[tid] = sr;
        reinterpret_cast<float4*>(y_im + bh * D)[tid] = si;
    }
}

template <int N>
static void dispatch_d(const StepArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.B * a.H)), block(256);
    float4* hr = reinterpret_cast<float4*>(a.h_re);
    float4* hi = reinterpret_cast<float4*>(a.h_im);
#define CSSD_K5(DD)                                                                         \
    hipLaunchKernelGGL((k_step<N, DD>), grid, block, 0, s, a.x_re, a.x_im, a.b_re, a.b_im,  \
                       a.c_re, a.c_im, a.dt, a.a_re, a.a_im, a.dskip, hr, hi, a.y_re, a.y_im, \
                       (int)a.H)
    switch (a.D) {
        case 16: CSSD_K5(16); break;
        case 32: CSSD_K5(32); break;
        case 64: CSSD_K5(64); break;
        default: CSSD_K5(128); break;
    }
#undef CSSD_K5
}

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
    switch (a.N) {
        case 16: dispatch_d<16>(a, stream); break;
        case 32: dispatch_d<32>(a, stream); break;
        case 64: dispatch_d<64>(a, stream); break;
        default: dispatch_d<128>(a, stream); break;
    }
    return hipGetLastError();
}

}  // namespace cssd
