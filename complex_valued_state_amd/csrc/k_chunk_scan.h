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
//  * the C/16 row tiles of a chunk carry unequal work (tile lt has lt + 1 causal
//    s-tiles), so each wave takes the balanced pair {t, C/16 - 1 - t}, one
//    after the other; for a tile it owns y[l0:l0+16, 0:D] as D/16 accumulator
//    tiles (re and im);
//  * Y_off: A = exp(acs[l]) C[l, n] from this lane's C row (float4 along n),
//    B-operand = H_c tiles, which the chunk-state kernels store in
//    MFMA-fragment order (one contiguous 1 KB float4 load per 16x16 tile);
//  * per s-tile, G^T = B C^T with A = B rows (lane%16 = s) and B-operand = C rows
//    (lane%16 = l), both float4 along n (the k-permutation n = 16k + 4g + q is
//    the same for both).  The G^T accumulator holds G[l = l0 + lane%16]
//    [s = s0 + 4g + r] in register r -- exactly the A-operand layout of the next
//    product -- so M = G . L is formed in registers (L per element: fp64
//    difference of the fp64 cumsums in log2 units / turns, phase reduced to
//    half a turn, then the fp32 hardware exp2 / sin / cos; the skip weight is
//    added to the diagonal of M) and fed straight back to the MFMA against X
//    rows s = s0 + 4g + r: L never leaves registers;
//  * B, C, X, H_c are read and y written through raw buffer descriptors whose
//    extent ends at the last real row of the chunk: padded rows read as zero and
//    their stores are dropped, so no masks or clamps are needed;
//  * the s-tile loop is unrolled (C is a template parameter) and the operands
//    of the next H tile / s-tile are loaded before the current tile's MFMAs,
//    when they fit the register budget of two waves per SIMD (N, D <= 64).
// A complex product is three real MFMAs (Gauss): t1 += ar br, t2 += ai bi,
// t3 += (ar + ai)(br + bi); re = t1 - t2, im = t3 - t1 - t2.  On this chip vector
// ALU instructions do not overlap matrix instructions of the same SIMD, so one
// 4-cycle add that saves a 32-cycle MFMA is a clear win.
#pragma once

#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

struct ScanArgs {
    const void *x_re, *x_im, *b_re, *b_im, *c_re, *c_im;
    const float* dskip;
    const double *acs_re, *acs_im;
    const float *e_re, *e_im, *hc_re, *hc_im;
    float *y_re, *y_im;
    int64_t T;
    int H, nC;
    int64_t nchunks;
};

// One wave: the 16 output rows of row tile lt of one chunk.
template <typename In, int C, int N, int D>
__device__ __forceinline__ void chunk_scan_tile(const ScanArgs& a, int64_t chunk, int lt) {
    typedef typename In::T TI;
    constexpr int NK = N / 16;   // 16-wide tiles of the n axis
    constexpr int PT = D / 16;   // 16-wide tiles of the p axis
    constexpr int NLT = C / 16;  // row tiles per chunk
    constexpr bool PF = NK <= 4 && PT <= 4;  // prefetch one tile ahead
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int c = (int)(chunk % a.nC);
    const int64_t bh = chunk / a.nC;
    const int h = (int)(bh % a.H);
    const int64_t b = bh / a.H;
    const int64_t t0 = (int64_t)c * C;
    const int valid = (int)min<int64_t>((int64_t)C, a.T - t0);
    const int l0 = lt * 16;
    if (l0 >= valid) return;  // tile entirely in the padding: nothing to write

    // per-chunk buffer views; rows >= valid lie past their extent
    const int64_t row0 = (b * a.T + t0) * a.H + h;  // row (b, t0, h); time t0+s is row0 + s*H
    const uint32_t sN = (uint32_t)a.H * N, sD = (uint32_t)a.H * D;
    const uint32_t extN = (uint32_t)(valid - 1) * sN + N, extD = (uint32_t)(valid - 1) * sD + D;
    const BufRes rb_r = make_buf(static_cast<const TI*>(a.b_re) + row0 * N, extN * sizeof(TI));
    const BufRes rb_i = make_buf(static_cast<const TI*>(a.b_im) + row0 * N, extN * sizeof(TI));
    const BufRes rc_r = make_buf(static_cast<const TI*>(a.c_re) + row0 * N, extN * sizeof(TI));
    const BufRes rc_i = make_buf(static_cast<const TI*>(a.c_im) + row0 * N, extN * sizeof(TI));
    const BufRes rx_r = make_buf(static_cast<const TI*>(a.x_re) + row0 * D, extD * sizeof(TI));
    const BufRes rx_i = make_buf(static_cast<const TI*>(a.x_im) + row0 * D, extD * sizeof(TI));
    const BufRes ry_r = make_buf(a.y_re + row0 * D, extD * 4);
    const BufRes ry_i = make_buf(a.y_im + row0 * D, extD * 4);
    const BufRes rh_r = make_buf(a.hc_re + (bh * a.nC + c) * (int64_t)N * D, N * D * 4);
    const BufRes rh_i = make_buf(a.hc_im + (bh * a.nC + c) * (int64_t)N * D, N * D * 4);
    const int64_t pbase = bh * (int64_t)a.nC * C + t0;  // per-position workspace base
    const double* __restrict__ ab_r = a.acs_re + pbase;  // log2 units
    const double* __restrict__ ab_i = a.acs_im + pbase;  // turns

    struct HTile {
        floatx4 r[PT], i[PT];
    };
    struct STile {
        floatx4 br[NK], bi[NK];
        float xr[4][PT], xi[4][PT];
    };
    auto load_h = [&](int k, HTile& o) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            o.r[pt] = buf_f32x4(rh_r, (uint32_t)(k * PT + pt) * 256 + 4 * lane);
            o.i[pt] = buf_f32x4(rh_i, (uint32_t)(k * PT + pt) * 256 + 4 * lane);
        }
    };
    // B rows s0 + li (float4 along n) and X rows s0 + 4g + r of s-tile st
    auto load_s = [&](int st, STile& o) {
        const uint32_t boff = (uint32_t)(st * 16 + li) * sN + 4 * g;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            o.br[k] = In::bload4(rb_r, boff + 16 * k);
            o.bi[k] = In::bload4(rb_i, boff + 16 * k);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t xoff = (uint32_t)(st * 16 + 4 * g + r) * sD + li;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                o.xr[r][pt] = In::bload1(rx_r, xoff + pt * 16);
                o.xi[r][pt] = In::bload1(rx_i, xoff + pt * 16);
            }
        }
    };

    // ---- this lane's readout row l = l0 + li (zero past the end of the chunk)
    const int lrow = l0 + li;
    floatx4 cre[NK], cim[NK];
    {
        const uint32_t off = (uint32_t)lrow * sN + 4 * g;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            cre[k] = In::bload4(rc_r, off + 16 * k);
            cim[k] = In::bload4(rc_i, off + 16 * k);
        }
    }
    HTile hcur;
    load_h(0, hcur);
    const double alr = ab_r[lrow], ali = ab_i[lrow];
    const float er = a.e_re[pbase + lrow], ei = a.e_im[pbase + lrow];
    const float dk = a.dskip != nullptr ? a.dskip[h] : 0.f;

    CTile y[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) ctile_zero(y[pt]);
    // operand sums of the C row for the score products, formed once per tile
    floatx4 csum[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) csum[k] = cre[k] + cim[k];

    // ---- Y_off = diag(exp(acs)) C H_c : contraction over n
    STile s_tiles[NLT];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        HTile hnxt;
        if (PF) {
            if (k + 1 < NK)
                load_h(k + 1, hnxt);
            else
                load_s(0, s_tiles[0]);  // first s-tile while the last H tile runs
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float cr = cre[k][q], ci = cim[k][q];
            const float ar = er * cr - ei * ci;
            const float ai = er * ci + ei * cr;
            const float as = ar + ai;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                ctile_mac(y[pt], ar, ai, as, hcur.r[pt][q], hcur.i[pt][q],
                          hcur.r[pt][q] + hcur.i[pt][q]);
        }
        if (k + 1 < NK) {
            if (PF)
                hcur = hnxt;
            else
                load_h(k + 1, hcur);
        }
    }

    // ---- Y_diag over the causal s-tiles 0..lt (lt is the diagonal tile)
#pragma unroll
    for (int st = 0; st < NLT; ++st) {
        if (st <= lt) {  // wave-uniform
            const bool diag = (st == lt);
            const int s0 = st * 16;
            if (PF) {
                if (st + 1 < NLT && st + 1 <= lt) load_s(st + 1, s_tiles[st + 1]);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                load_s(st, s_tiles[st]);
            }
            const STile& o = s_tiles[st];
            // G^T block: A = B[s0 + li, n], B-operand = C[l0 + li, n]
            CTile gt;
            ctile_zero(gt);
#pragma unroll
            for (int k = 0; k < NK; ++k) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float br = o.br[k][q], bi = o.bi[k][q];
                    ctile_mac(gt, br, bi, br + bi, cre[k][q], cim[k][q], csum[k][q]);
                }
            }
            floatx4 gr, gi;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                gr[r] = ctile_re(gt, r);
                gi[r] = ctile_im(gt, r);
            }
            // M = G . L + Dskip on the diagonal; register r <-> s = s0 + 4g + r
            float mr[4], mi[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = s0 + 4 * g + r;
                float lr = 0.f, lim = 0.f;
                if (!diag || s <= lrow) {
                    const double d2 = alr - ab_r[s];
                    double dv = ali - ab_i[s];
                    dv -= rint(dv);
                    cexp_scaled((float)d2, (float)dv, lr, lim);
                }
                mr[r] = gr[r] * lr - gi[r] * lim + ((diag && s == lrow) ? dk : 0.f);
                mi[r] = gr[r] * lim + gi[r] * lr;
            }
            // Y += M X
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ms = mr[r] + mi[r];
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
                    ctile_mac(y[pt], mr[r], mi[r], ms, o.xr[r][pt], o.xi[r][pt],
                              o.xr[r][pt] + o.xi[r][pt]);
            }
        }
    }

    // ---- store; register r <-> row l = l0 + 4g + r (padded rows are dropped)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t off = (uint32_t)(l0 + 4 * g + r) * sD + li;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            buf_store_f32(ctile_re(y[pt], r), ry_r, off + pt * 16);
            buf_store_f32(ctile_im(y[pt], r), ry_i, off + pt * 16);
        }
    }
}

// A 256-thread block holds 4 / (waves per chunk) whole chunks, so the waves of
// a chunk share a CU; each wave runs the balanced pair of row tiles.
template <typename In, int C, int N, int D>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(N * D > 64 * 128 ? 1 : 2))) void k_chunk_scan(ScanArgs a) {
    constexpr int NLT = C / 16;
    constexpr int WPC = NLT >= 2 ? NLT / 2 : 1;  // waves per chunk
    const int wave = wave_id();
    const int64_t chunk = (int64_t)blockIdx.x * (4 / WPC) + wave / WPC;
    if (chunk >= a.nchunks) return;  // wave-uniform
    const int t = wave % WPC;
    chunk_scan_tile<In, C, N, D>(a, chunk, t);
    if (NLT - 1 - t != t) chunk_scan_tile<In, C, N, D>(a, chunk, NLT - 1 - t);
}

// Launch of the register-operand kernel above (any supported shape and dtype).
template <int C>
hipError_t launch_chunk_scan_regs(const FwdArgs& f, hipStream_t s) {
    ScanArgs a;
    a.x_re = f.x_re; a.x_im = f.x_im; a.b_re = f.b_re; a.b_im = f.b_im;
    a.c_re = f.c_re; a.c_im = f.c_im; a.dskip = f.dskip;
    a.acs_re = f.acs_re; a.acs_im = f.acs_im; a.e_re = f.e_re; a.e_im = f.e_im;
    a.hc_re = f.st_re; a.hc_im = f.st_im; a.y_re = f.y_re; a.y_im = f.y_im;
    a.T = f.T; a.H = (int)f.H; a.nC = (int)f.nC;
    a.nchunks = f.B * f.H * f.nC;
    constexpr int WPC = C / 16 >= 2 ? C / 32 : 1;
    constexpr int CPB = 4 / WPC;  // chunks per block
    const dim3 grid((unsigned)((a.nchunks + CPB - 1) / CPB)), block(256);
#define CSSD_K2(IN, NN, DD) hipLaunchKernelGGL((k_chunk_scan<IN, C, NN, DD>), grid, block, 0, s, a)
#define CSSD_K2_D(IN, NN)                  \
    switch (f.D) {                         \
        case 16: CSSD_K2(IN, NN, 16); break; \
        case 32: CSSD_K2(IN, NN, 32); break; \
        case 64: CSSD_K2(IN, NN, 64); break; \
        default: CSSD_K2(IN, NN, 128); break; \
    }
#define CSSD_K2_N(IN)                         \
    switch (f.N) {                            \
        case 16: CSSD_K2_D(IN, 16) break;     \
        case 32: CSSD_K2_D(IN, 32) break;     \
        case 64: CSSD_K2_D(IN, 64) break;     \
        default: CSSD_K2_D(IN, 128) break;    \
    }
    if (f.in_dtype == 1) {
        CSSD_K2_N(InBF16)
    } else {
        CSSD_K2_N(InF32)
    }
#undef CSSD_K2_N
#undef CSSD_K2_D
#undef CSSD_K2
    return hipGetLastError();
}

}  // namespace cssd
