// K2: intra-chunk output and the combine, on the fp32 matrix cores.
//
// For chunk c of sequence (b, h), with rows l and columns s of the chunk:
//   G[l, s]  = sum_n C[l, n] B[s, n]                       score matrix C B^T
//   L[l, s]  = exp(acs[l] - acs[s]) * 1[l >= s]            causal segment matrix
//   y[l, :]  = sum_{s<=l} (G . L)[l, s] X[s, :]            Y_diag
//            + exp(acs[l]) sum_n C[l, n] H_c[n, :]         Y_off (carry-in state)
//            + Dskip * X[l, :]
// Passages: Mamba-3-Lite docs, "SSD Theory" 4.3 (segment matrix with inclusive
// diagonal, Y_diag = (C B^T . L) X), 4.5 (readout of the carried state decayed
// from the chunk start), "The Chunkwise Complex SSD Algorithm" 4.3-4.5; the
// skip term follows the burn-mamba step_constant readout.
//
// Mapping (16x16x4 fp32 MFMA, wave64; lane = i + 16 g):
//  * one workgroup per chunk, one wave per 16-row tile lt of l; the wave owns
//    y[l0:l0+16, 0:D] as D/16 accumulator tiles (re and im);
//  * the wave first forms G^T for one 16x16 (s, l) block with A = B rows
//    (lane%16 = s) and B-operand = C rows (lane%16 = l), both read as float4
//    along n; the k-permutation n = 16k + 4g + q is the same for both;
//  * the accumulator of G^T holds G[l = l0 + lane%16][s = s0 + 4g + r] in its
//    register r -- exactly the A-operand layout (lane%16 = row l, k = s) of the
//    next product, so M = G . L is formed in registers (L is evaluated per
//    element: fp64 difference of the fp64 cumsums, phase wrapped to [-pi, pi],
//    then fp32 exp and sincos) and fed straight back to the MFMA against X
//    rows s = s0 + 4g + r -- no LDS round trip, L never leaves registers;
//  * s-tiles strictly below the diagonal need no mask (s < l0 <= l); only the
//    diagonal tile applies the causal mask and the padding mask;
//  * Y_off uses A = exp(acs[l]) C[l, n] (the C rows already in registers) and
//    B-operand = H_c[n, p]; the chunk-state kernel stores H_c in MFMA-fragment
//    order, so each 16x16 operand tile is one contiguous 1 KB float4 load.
// A complex product is four real MFMAs: re += ar br - ai bi, im += ar bi + ai br.
#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

template <typename In, int N, int D>
__global__ __launch_bounds__(512) void k_chunk_scan(
    const typename In::T* __restrict__ x_re, const typename In::T* __restrict__ x_im,
    const typename In::T* __restrict__ b_re, const typename In::T* __restrict__ b_im,
    const typename In::T* __restrict__ c_re, const typename In::T* __restrict__ c_im,
    const float* __restrict__ dskip, const double* __restrict__ acs_re,
    const double* __restrict__ acs_im, const float* __restrict__ e_re,
    const float* __restrict__ e_im, const float* __restrict__ hc_re,
    const float* __restrict__ hc_im, float* __restrict__ y_re, float* __restrict__ y_im,
    int64_t T, int H, int nC, int C) {
    constexpr int NK = N / 16;  // 16-wide tiles of the n axis
    constexpr int PT = D / 16;  // 16-wide tiles of the p axis
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int lt = threadIdx.x >> 6;
    const int64_t chunk = blockIdx.x;
    const int c = (int)(chunk % nC);
    const int64_t bh = chunk / nC;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int64_t t0 = (int64_t)c * C;
    const int valid = (int)min<int64_t>((int64_t)C, T - t0);
    const int l0 = lt * 16;
    if (l0 >= valid) return;  // tile entirely in the padding: nothing to write

    // wave-uniform bases; per-lane offsets below are 32-bit
    const int64_t row0 = (b * T + t0) * H + h;  // row (b, t0, h); time t0+s is row0 + s*H
    const typename In::T* __restrict__ xb_r = x_re + row0 * D;
    const typename In::T* __restrict__ xb_i = x_im + row0 * D;
    const typename In::T* __restrict__ bb_r = b_re + row0 * N;
    const typename In::T* __restrict__ bb_i = b_im + row0 * N;
    const typename In::T* __restrict__ cb_r = c_re + row0 * N;
    const typename In::T* __restrict__ cb_i = c_im + row0 * N;
    const uint32_t sN = (uint32_t)H * N, sD = (uint32_t)H * D;
    const int64_t pbase = bh * (int64_t)nC * C + t0;  // per-position workspace base
    const double* __restrict__ ab_r = acs_re + pbase;
    const double* __restrict__ ab_i = acs_im + pbase;

    // ---- this lane's readout row l = l0 + li (zero when it is padding)
    const int lrow = l0 + li;
    const bool lok = lrow < valid;
    float4 cre[NK], cim[NK];
    {
        const uint32_t off = (uint32_t)(lok ? lrow : valid - 1) * sN + 4 * g;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            cre[k] = In::load4(cb_r + off + 16 * k);
            cim[k] = In::load4(cb_i + off + 16 * k);
        }
        if (!lok) {
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                cre[k] = make_float4(0.f, 0.f, 0.f, 0.f);
                cim[k] = cre[k];
            }
        }
    }
    const double alr = ab_r[lrow], ali = ab_i[lrow];
    const float er = e_re[pbase + lrow], ei = e_im[pbase + lrow];

    floatx4 yr[PT], yi[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
        yr[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
        yi[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- Y_off = diag(exp(acs)) C H_c : contraction over n.  H_c is stored in
    // MFMA-fragment order: tile (k, pt) is 256 contiguous floats, lane-major.
    {
        const float* __restrict__ hb_r = hc_re + (bh * nC + c) * (int64_t)N * D + 4 * lane;
        const float* __restrict__ hb_i = hc_im + (bh * nC + c) * (int64_t)N * D + 4 * lane;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            floatx4 hr[PT], hi[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                hr[pt] = *reinterpret_cast<const floatx4*>(hb_r + (k * PT + pt) * 256);
                hi[pt] = *reinterpret_cast<const floatx4*>(hb_i + (k * PT + pt) * 256);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float cr = f4get(cre[k], q), ci = f4get(cim[k], q);
                const float ar = er * cr - ei * ci;
                const float ai = er * ci + ei * cr;
                const float nai = -ai;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    yr[pt] = mfma4(ar, hr[pt][q], yr[pt]);
                    yr[pt] = mfma4(nai, hi[pt][q], yr[pt]);
                    yi[pt] = mfma4(ar, hi[pt][q], yi[pt]);
                    yi[pt] = mfma4(ai, hr[pt][q], yi[pt]);
                }
            }
        }
    }

    // ---- Y_diag over s-tiles 0..lt (the last one is the diagonal tile)
    for (int st = 0; st <= lt; ++st) {
        const bool diag = (st == lt);  // wave-uniform
        const int s0 = st * 16;
        // G^T block: A = B[s0 + li, n], B-operand = C[l0 + li, n]
        floatx4 gr = floatx4{0.f, 0.f, 0.f, 0.f}, gi = gr;
        {
            const int srow = s0 + li;
            const bool sok = srow < valid;  // always true off the diagonal
            const uint32_t off = (uint32_t)(sok ? srow : valid - 1) * sN + 4 * g;
            float4 bre[NK], bim[NK];
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                bre[k] = In::load4(bb_r + off + 16 * k);
                bim[k] = In::load4(bb_i + off + 16 * k);
            }
            if (!sok) {
#pragma unroll
                for (int k = 0; k < NK; ++k) {
                    bre[k] = make_float4(0.f, 0.f, 0.f, 0.f);
                    bim[k] = bre[k];
                }
            }
#pragma unroll
            for (int k = 0; k < NK; ++k) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float br = f4get(bre[k], q), bi = f4get(bim[k], q);
                    const float cr = f4get(cre[k], q), ci = f4get(cim[k], q);
                    gr = mfma4(br, cr, gr);
                    gr = mfma4(-bi, ci, gr);
                    gi = mfma4(br, ci, gi);
                    gi = mfma4(bi, cr, gi);
                }
            }
        }
        // X rows of this s-tile: step r contracts s = s0 + 4g + r
        float xr[4][PT], xi[4][PT];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = s0 + 4 * g + r;
            const bool xok = s < valid;
            const uint32_t xoff = (uint32_t)(xok ? s : valid - 1) * sD + li;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                xr[r][pt] = xok ? In::load1(xb_r + xoff + pt * 16) : 0.f;
                xi[r][pt] = xok ? In::load1(xb_i + xoff + pt * 16) : 0.f;
            }
        }
        // M = G . L, register r <-> s = s0 + 4g + r, lane row l = lrow
        float mr[4], mi[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = s0 + 4 * g + r;
            const bool keep = !diag || (s <= lrow);
            float lr = 0.f, lim = 0.f;
            if (keep) {
                const double dre = alr - ab_r[s];
                const double dim = wrap_phase(ali - ab_i[s]);
                const float mag = expf((float)dre);
                float sn, cs;
                sincosf((float)dim, &sn, &cs);
                lr = mag * cs;
                lim = mag * sn;
            }
            mr[r] = gr[r] * lr - gi[r] * lim;
            mi[r] = gr[r] * lim + gi[r] * lr;
        }
        // Y += M X
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float nmi = -mi[r];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                yr[pt] = mfma4(mr[r], xr[r][pt], yr[pt]);
                yr[pt] = mfma4(nmi, xi[r][pt], yr[pt]);
                yi[pt] = mfma4(mr[r], xi[r][pt], yi[pt]);
                yi[pt] = mfma4(mi[r], xr[r][pt], yi[pt]);
            }
        }
    }

    // ---- epilogue: skip term and store; register r <-> row l = l0 + 4g + r
    const float dk = dskip != nullptr ? dskip[h] : 0.f;
    float* __restrict__ yb_r = y_re + row0 * D;
    float* __restrict__ yb_i = y_im + row0 * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int l = l0 + 4 * g + r;
        if (l < valid) {
            const uint32_t off = (uint32_t)l * sD + li;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const float xv = In::load1(xb_r + off + pt * 16);
                const float xw = In::load1(xb_i + off + pt * 16);
                yb_r[off + pt * 16] = yr[pt][r] + dk * xv;
                yb_i[off + pt * 16] = yi[pt][r] + dk * xw;
            }
        }
    }
}

template <typename In, int N>
static void dispatch_d(const FwdArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.B * a.H * a.nC)), block((unsigned)(a.C / 16 * 64));
    const auto* xr = static_cast<const typename In::T*>(a.x_re);
    const auto* xi = static_cast<const typename In::T*>(a.x_im);
    const auto* br = static_cast<const typename In::T*>(a.b_re);
    const auto* bi = static_cast<const typename In::T*>(a.b_im);
    const auto* cr = static_cast<const typename In::T*>(a.c_re);
    const auto* ci = static_cast<const typename In::T*>(a.c_im);
#define CSSD_K2(DD)                                                                             \
    hipLaunchKernelGGL((k_chunk_scan<In, N, DD>), grid, block, 0, s, xr, xi, br, bi, cr, ci,    \
                       a.dskip, a.acs_re, a.acs_im, a.e_re, a.e_im, a.st_re, a.st_im, a.y_re,  \
                       a.y_im, a.T, (int)a.H, (int)a.nC, (int)a.C)
    switch (a.D) {
        case 16: CSSD_K2(16); break;
        case 32: CSSD_K2(32); break;
        case 64: CSSD_K2(64); break;
        default: CSSD_K2(128); break;
    }
#undef CSSD_K2
}

template <typename In>
static void dispatch_n(const FwdArgs& a, hipStream_t s) {
    switch (a.N) {
        case 16: dispatch_d<In, 16>(a, s); break;
        case 32: dispatch_d<In, 32>(a, s); break;
        case 64: dispatch_d<In, 64>(a, s); break;
        default: dispatch_d<In, 128>(a, s); break;
    }
}

hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t stream) {
    if (a.in_dtype == 1)
        dispatch_n<InBF16>(a, stream);
    else
        dispatch_n<InF32>(a, stream);
    return hipGetLastError();
}

}  // namespace cssd
