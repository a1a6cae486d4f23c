// K1: discretisation and chunk-local inclusive cumulative log-decay.
//
// For every (batch b, head h, chunk c) and intra-chunk position l:
//   A_log[l]  = softplus(dt[b, cC+l, h]) * A[h]        (0 on padded positions l >= T - cC)
//   acs[l]    = sum_{u <= l} A_log[u]                  (inclusive, restarts at every chunk;
//                                                      stored as Re/ln2 and Im/2pi: log2 units
//                                                      and turns, ready for exp2 and sin/cos
//                                                      of turns in the output kernel)
//   e[l]      = exp(acs[l])                            readout decay from the chunk start
//   w[l]      = exp(acs[C-1] - acs[l])                 decay from l to the chunk end
//   cd        = exp(acs[C-1])                          whole-chunk decay
// Passages: Mamba-3-Lite docs, "SSD Theory" 4.3 (within-chunk cumulative sum,
// inclusive so the segment matrix has a unit diagonal), 4.5 (chunk total and
// the decay to the chunk end), and "The Chunkwise Complex SSD Algorithm" 4.2
// (log-decay A_log = softplus(dt) A and its cumsum over the chunk axis).
//
// One wave per (b, h, c); lane l holds position l (two positions per lane for
// C = 128).  The scan runs in fp64 across the lanes (DPP row shifts and row
// broadcasts, no LDS round trips): the imaginary part of a
// 128-step chunk reaches thousands of radians, and every consumer later takes
// differences of these sums, so they are kept exact to fp64 and stored as
// fp64.  The exponentials take the fp64 arguments to log2 units and to half a
// turn, then the fp32 hardware exp2 / sin / cos.
// Padded positions get a zero increment, so a partial last chunk's total equals
// the sum over its valid positions and the final state never decays through
// padding.
#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

template <int PER>  // positions per lane: 1 (C <= 64) or 2 (C = 128)
__global__ __launch_bounds__(256) void k_cumsum(const float* __restrict__ dt,
                                                const float* __restrict__ a_re,
                                                const float* __restrict__ a_im, int64_t T, int H,
                                                int nC, int C, int64_t units,
                                                double* __restrict__ acs_re,
                                                double* __restrict__ acs_im,
                                                float* __restrict__ e_re, float* __restrict__ e_im,
                                                float* __restrict__ w_re, float* __restrict__ w_im,
                                                float* __restrict__ cd_re,
                                                float* __restrict__ cd_im) {
    const int64_t unit = (int64_t)blockIdx.x * 4 + wave_id();
    if (unit >= units) return;  // wave-uniform
    const int lane = threadIdx.x & 63;
    const int c = (int)(unit % nC);
    const int64_t bh = unit / nC;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const double are = a_re[h], aim = a_im[h];
    const int64_t t0 = (int64_t)c * C;

    double vr[PER], vi[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int l = lane * PER + j;
        const int64_t t = t0 + l;
        vr[j] = 0.0;
        vi[j] = 0.0;
        if (l < C && t < T) {
            const double s = softplus_f64((double)dt[(b * T + t) * H + h]);
            vr[j] = s * are;
            vi[j] = s * aim;
        }
    }
    // in-lane prefix, then an inclusive wave scan of the lane totals
#pragma unroll
    for (int j = 1; j < PER; ++j) {
        vr[j] += vr[j - 1];
        vi[j] += vi[j - 1];
    }
    double sr = vr[PER - 1], si = vi[PER - 1];
    wave_inclusive_scan(sr);
    wave_inclusive_scan(si);
    const double exr = sr - vr[PER - 1], exi = si - vi[PER - 1];  // exclusive prefix of the lane
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        vr[j] += exr;
        vi[j] += exi;
    }
    // chunk total acs[C-1] lives in lane (C-1)/PER, slot (C-1)%PER
    const int last_lane = (C - 1) / PER;
    double tot_r = vr[PER - 1], tot_i = vi[PER - 1];
    if (PER == 2 && ((C - 1) % PER) == 0) {
        tot_r = vr[0];
        tot_i = vi[0];
    }
    tot_r = lane_value(tot_r, last_lane);
    tot_i = lane_value(tot_i, last_lane);

    // exp of a complex fp64 log-decay, rounded to fp32: the argument is taken to
    // log2 units and to a fraction of a turn in fp64, then the fp32 hardware
    // exp2 / sin / cos (about one ulp each) finish it
    auto cexp_f = [](double re, double im, float& out_re, float& out_im) {
        double t = im * kInvTwoPi;
        t -= rint(t);
        cexp_scaled((float)(re * kLog2e), (float)t, out_re, out_im);
    };
    const int64_t base = bh * (int64_t)nC * C + t0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int l = lane * PER + j;
        if (l < C) {
            acs_re[base + l] = vr[j] * kLog2e;
            acs_im[base + l] = vi[j] * kInvTwoPi;
            float er, ei, wr, wi;
            cexp_f(vr[j], vi[j], er, ei);
            cexp_f(tot_r - vr[j], tot_i - vi[j], wr, wi);
            e_re[base + l] = er;
            e_im[base + l] = ei;
            w_re[base + l] = wr;
            w_im[base + l] = wi;
        }
    }
    if (lane == 0) {
        float dr, di;
        cexp_f(tot_r, tot_i, dr, di);
        cd_re[bh * nC + c] = dr;
        cd_im[bh * nC + c] = di;
    }
}

hipError_t launch_cumsum(const FwdArgs& a, hipStream_t stream) {
    const int64_t units = a.B * a.H * a.nC;
    const dim3 grid((unsigned)((units + 3) / 4)), block(256);
    if (a.C <= 64)
        hipLaunchKernelGGL(k_cumsum<1>, grid, block, 0, stream, a.dt, a.a_re, a.a_im, a.T,
                           (int)a.H, (int)a.nC, (int)a.C, units, a.acs_re, a.acs_im, a.e_re,
                           a.e_im, a.w_re, a.w_im, a.cd_re, a.cd_im);
    else
        hipLaunchKernelGGL(k_cumsum<2>, grid, block, 0, stream, a.dt, a.a_re, a.a_im, a.T,
                           (int)a.H, (int)a.nC, (int)a.C, units, a.acs_re, a.acs_im, a.e_re,
                           a.e_im, a.w_re, a.w_im, a.cd_re, a.cd_im);
    return hipGetLastError();
}

}  // namespace cssd
