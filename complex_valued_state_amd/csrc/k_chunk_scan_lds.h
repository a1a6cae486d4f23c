// K2 for fp32 inputs whose chunk fits in LDS (C <= 64, C * N <= 4096): the same
// output as k_chunk_scan (see k_chunk_scan.h for the formulas and passages),
// organised so that every input row of the chunk is fetched from memory once.
//
// A workgroup of D/16 waves computes one chunk; wave w owns the 16 output
// columns [16w, 16w + 16) of every row.
//  0. staging, in two groups: first the chunk's C rows (both planes), its fp64
//     cumsums and exp(acs), and each wave's 16-column block of H_c; then the B
//     rows and each wave's block of X.  Rows go to LDS by direct-to-LDS buffer
//     loads (buffer_load_dwordx4 ... lds: lane i's 16 bytes land at the
//     instruction's LDS base + 16 i), with their 16-byte chunks XOR-swizzled by
//     the row index, so that the MFMA operand reads below (16 rows, one 16-byte
//     chunk each) hit distinct LDS banks.  Padded rows of a partial chunk read
//     as zero through the buffer extent.
//  1. as soon as the first group is in: Y_off on the wave's 16 columns, C rows
//     from LDS times H_c, then the per-row factor exp(acs[l]) on the finished
//     accumulator.  The second group arrives meanwhile.
//  2. score tiles: the NP = NLT(NLT+1)/2 causal 16x16 tiles are split evenly
//     over the waves; G^T = B C^T from LDS, then M = G . L (+ Dskip on the
//     diagonal) in registers, in the A-operand lane order of the next product.
//  3. barrier; the M tiles overwrite the B rows in LDS; barrier.
//  4. Y_diag: every causal tile's M from LDS times the wave's columns of X.
// Two workgroups share a CU (the LDS bounds it), so one's staging overlaps the
// other's matrix work; three at N = D = C = 64, where the B rows are staged in
// halves (below).
#pragma once

#include "k_chunk_scan.h"

namespace cssd {

typedef __attribute__((address_space(3))) void* LdsPtr;

// 16-byte chunk swizzle of a staged row: logical chunk c of row `row` sits at
// physical chunk c ^ f(row).  f takes as many low row bits as make 16
// consecutive rows cover all banks for a fixed logical chunk.
template <int N>
__device__ __forceinline__ int lds_swz(int row, int c) {
    constexpr int shift = N >= 64 ? 0 : (N == 32 ? 1 : 2);
    return c ^ ((row & 15) >> shift);
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (gfx9 encoding: vmcnt low bits [3:0], high bits [15:14]; expcnt and lgkmcnt
// left at their maxima, i.e. not waited on).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// At N = D = C = 64 the B rows are staged in two halves (rows 0-31 for the score
// tiles of the first two column tiles, then rows 32-63 for the other three), so
// that a workgroup takes 52 KB of LDS instead of 68 and three fit on a CU, with
// the registers held to three waves per SIMD.
template <int C, int N, int D>
constexpr bool k2_half_b() {
    return C == 64 && N == 64 && D == 64;
}

template <int C, int N, int D>
__global__ __launch_bounds__(64 * (D / 16))
__attribute__((amdgpu_waves_per_eu(k2_half_b<C, N, D>() ? 3 : 1))) void k_chunk_scan_lds(
    ScanArgs a) {
    constexpr int NK = N / 16;                // 16-wide tiles of the n axis
    constexpr int W = D / 16;                 // waves = 16-wide column tiles of p
    constexpr int NLT = C / 16;               // row tiles per chunk
    constexpr int NP = NLT * (NLT + 1) / 2;   // causal tiles (lt >= st), lt-major
    constexpr int MQ = (NP + W - 1) / W;      // most tiles one wave owns
    constexpr int PLANE = C * N;              // floats of one staged plane
    constexpr int IPP = PLANE / 256;          // 64-lane x 16-byte loads per plane
    constexpr int MFL = NP * 512;             // floats of the M tiles
    constexpr bool HB = k2_half_b<C, N, D>();
    constexpr int BPLANE = HB ? PLANE / 2 : PLANE;  // floats of one staged B plane
    constexpr int BIPP = BPLANE / 256;
    // B planes; later the M tiles (which go over the C rows when B is staged in halves)
    constexpr int BREG = HB ? 2 * BPLANE : (2 * PLANE > MFL ? 2 * PLANE : MFL);
    static_assert(!HB || MFL <= 2 * PLANE, "the M tiles must fit over the C rows");
    // vector-memory operations every wave issues after the first staging group
    // (a lower bound: each B plane gives a wave at least IPP / W blocks; then
    // its X loads), so waiting down to LATE outstanding completes the first group
    constexpr int LATE = 2 * (BIPP / W) + (HB ? 0 : 2 * 4 * NLT);
    static_assert(PLANE % 256 == 0, "staged plane must be whole 1 KB blocks");
    static_assert(LATE < 64, "vmcnt holds at most 63");
    static_assert(8 * C <= 1024, "a chunk's cumsums must fit one 1 KB slot");
    // three separate LDS objects, so that the compiler's wait for pending
    // direct-to-LDS writes before an LDS read covers only the object read
    __shared__ floatx4 lds_b4[BREG / 4];      // B rows, later the M tiles
    __shared__ floatx4 lds_c4[2 * PLANE / 4];  // C rows
    __shared__ floatx4 lds_a4[1024 / 4];       // acs re, acs im, e re, e im
    float* const lds = reinterpret_cast<float*>(lds_b4);
    float* const ldc = reinterpret_cast<float*>(lds_c4);
    float* const lda = reinterpret_cast<float*>(lds_a4);
    float* const ldm = HB ? ldc : lds;  // the M tiles
    const double* const lacs_r = reinterpret_cast<const double*>(lda);
    const double* const lacs_i = reinterpret_cast<const double*>(lda + 256);
    const float* const le_r = lda + 512;
    const float* const le_i = lda + 768;

    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int w = wave_id();
    const int64_t chunk = blockIdx.x;
    const int c = (int)(chunk % a.nC);
    const int64_t bh = chunk / a.nC;
    const int h = (int)(bh % a.H);
    const int64_t b = bh / a.H;
    const int64_t t0 = (int64_t)c * C;
    const int valid = (int)min<int64_t>((int64_t)C, a.T - t0);

    const int64_t row0 = (b * a.T + t0) * a.H + h;  // row (b, t0, h); time t0+s is row0 + s*H
    const uint32_t sN = (uint32_t)a.H * N, sD = (uint32_t)a.H * D;
    const uint32_t extN = (uint32_t)(valid - 1) * sN + N, extD = (uint32_t)(valid - 1) * sD + D;
    const BufRes rx_r = make_buf(static_cast<const float*>(a.x_re) + row0 * D, extD * 4);
    const BufRes rx_i = make_buf(static_cast<const float*>(a.x_im) + row0 * D, extD * 4);
    const BufRes ry_r = make_buf(a.y_re + row0 * D, extD * 4);
    const BufRes ry_i = make_buf(a.y_im + row0 * D, extD * 4);
    const BufRes rh_r = make_buf(a.hc_re + chunk * (int64_t)N * D, N * D * 4);
    const BufRes rh_i = make_buf(a.hc_im + chunk * (int64_t)N * D, N * D * 4);
    const int64_t pbase = bh * (int64_t)a.nC * C + t0;  // per-position workspace base
    const float dk = a.dskip != nullptr ? a.dskip[h] : 0.f;

    // one staged plane (rows r0 .. r0 + nblk * 256 / N - 1): its nblk 1 KB blocks,
    // dealt round-robin to the waves; rows are swizzled by their staged index
    auto stage_plane = [&](const void* src, float* dst_plane, int first, int r0, int nblk) {
        const BufRes r = make_buf(static_cast<const float*>(src) + row0 * N, extN * 4);
        for (int blk = (w - first + W) % W; blk < nblk; blk += W) {  // wave-uniform
            const int u = blk * 64 + lane;  // physical 16-byte chunk within the plane
            const int row = u / (N / 4), pc = u % (N / 4);
            const uint32_t voff = ((uint32_t)(r0 + row) * sN + 4 * lds_swz<N>(row, pc)) * 4;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(dst_plane + blk * 256), 16, voff,
                                                     0, 0, 0);
        }
    };

    // ---- 0a. first group: C rows, cumsums, exp(acs), H_c block
    stage_plane(a.c_re, ldc, 0, 0, IPP);
    stage_plane(a.c_im, ldc + PLANE, IPP % W, 0, IPP);
    if (w == W - 1) {
        // cumsums (fp64, 8C bytes each) and exp(acs) (fp32, 4C bytes each), one
        // 1 KB slot each; lanes past the end read zero into the rest of the slot
        const void* const aux[4] = {a.acs_re + pbase, a.acs_im + pbase, a.e_re + pbase,
                                    a.e_im + pbase};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_buf(aux[j], (j < 2 ? 8 : 4) * C),
                                                     (LdsPtr)(lda + 256 * j), 16, 16 * lane,
                                                     0, 0, 0);
    }
    // H_c[16k + 4g + e][16w + li] (fragment order)
    floatx4 hreg_r[NK], hreg_i[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        hreg_r[k] = buf_f32x4(rh_r, (uint32_t)(k * W + w) * 256 + 4 * lane);
        hreg_i[k] = buf_f32x4(rh_i, (uint32_t)(k * W + w) * 256 + 4 * lane);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the two groups in issue order
    // ---- 0b. second group: B rows, X block X[16 st + 4g + r][16w + li]
    stage_plane(a.b_re, lds, (2 * IPP) % W, 0, BIPP);
    stage_plane(a.b_im, lds + BPLANE, (3 * IPP) % W, 0, BIPP);
    float xreg_r[NLT][4], xreg_i[NLT][4];
    if constexpr (!HB) {
#pragma unroll
        for (int st = 0; st < NLT; ++st)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t off = (uint32_t)(st * 16 + 4 * g + r) * sD + 16 * w + li;
                xreg_r[st][r] = buf_f32(rx_r, off);
                xreg_i[st][r] = buf_f32(rx_i, off);
            }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(LATE));  // the first group is in
    __syncthreads();

    auto row4 = [&](const float* plane, int row, int ch) -> floatx4 {
        return *reinterpret_cast<const floatx4*>(plane + row * N + 4 * lds_swz<N>(row, ch));
    };

    // ---- 1. Y_off = diag(exp(acs)) C H_c on this wave's columns
    CTile acc[NLT];
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) ctile_zero(acc[lt]);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        const floatx4 hr = hreg_r[k], hi = hreg_i[k];
        const floatx4 hs = hr + hi;
#pragma unroll
        for (int lt = 0; lt < NLT; ++lt) {
            const floatx4 cr = row4(ldc, lt * 16 + li, 4 * k + g);
            const floatx4 ci = row4(ldc + PLANE, lt * 16 + li, 4 * k + g);
            const floatx4 cs = cr + ci;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ctile_mac(acc[lt], cr[e], ci[e], cs[e], hr[e], hi[e], hs[e]);
        }
    }
    // accumulator register r <-> row l = 16 lt + 4g + r: multiply by exp(acs[l])
    // and put the result back in Gauss form (t1 = re, t2 = 0, t3 = re + im)
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) {
        const floatx4 er = *reinterpret_cast<const floatx4*>(le_r + lt * 16 + 4 * g);
        const floatx4 ei = *reinterpret_cast<const floatx4*>(le_i + lt * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float re = ctile_re(acc[lt], r), im = ctile_im(acc[lt], r);
            const float nr = er[r] * re - ei[r] * im;
            const float ni = er[r] * im + ei[r] * re;
            acc[lt].t1[r] = nr;
            acc[lt].t2[r] = 0.f;
            acc[lt].t3[r] = nr + ni;
        }
    }

    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the second group is in
    __syncthreads();

    // ---- 2. score tiles -> M in registers
    floatx4 m_r[MQ], m_i[MQ];
    const int q0 = (w * NP) / W, q1 = ((w + 1) * NP) / W;  // without the half split
    int qidx[MQ], nq;  // the tile index of each kept M and their number
    // tile (lt, st) from the B rows staged from row b0 on
    auto score_tile = [&](int lt, int st, int b0, floatx4& mr, floatx4& mi) {
        const int l0 = lt * 16, s0 = st * 16;
        CTile gt;
        ctile_zero(gt);
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            const floatx4 br = row4(lds, s0 - b0 + li, 4 * k + g);
            const floatx4 bi = row4(lds + BPLANE, s0 - b0 + li, 4 * k + g);
            const floatx4 cr = row4(ldc, l0 + li, 4 * k + g);
            const floatx4 ci = row4(ldc + PLANE, l0 + li, 4 * k + g);
            const floatx4 bs = br + bi, cs = cr + ci;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ctile_mac(gt, br[e], bi[e], bs[e], cr[e], ci[e], cs[e]);
        }
        // register r <-> (l = l0 + li, s = s0 + 4g + r)
        const int lrow = l0 + li;
        const bool diag = (lt == st);
        const double alr = lacs_r[lrow], ali = lacs_i[lrow];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = s0 + 4 * g + r;
            const float gr = ctile_re(gt, r), gi = ctile_im(gt, r);
            float lr = 0.f, lim = 0.f;
            if (!diag || s <= lrow) {
                const double d2 = alr - lacs_r[s];
                double dv = ali - lacs_i[s];
                dv -= rint(dv);
                cexp_scaled((float)d2, (float)dv, lr, lim);
            }
            mr[r] = gr * lr - gi * lim + ((diag && s == lrow) ? dk : 0.f);
            mi[r] = gr * lim + gi * lr;
        }
    };
    // the tiles this wave owns, as (lt, st) in fixed slots (wave-uniform values):
    // with B in halves, the seven tiles with st < 2 (lt-major, idx -> ((idx + 1) / 2,
    // (idx + 1) % 2) for idx >= 1) two per wave and one for wave 3, then (2,2) to
    // wave 1, (3,2) to wave 2 and (3,3) to wave 3; else the NP tiles in lt-major
    // order, split evenly
    if constexpr (HB) {
        int own_lt[MQ], own_st[MQ], nown;
        static_assert(MQ == 3 && W == 4 && NLT == 4, "the split is for C = D = 64");
        auto a_tile = [](int idx, int& lt, int& st) {
            lt = idx == 0 ? 0 : (idx + 1) / 2;
            st = idx == 0 ? 0 : (idx + 1) % 2;
        };
        a_tile(2 * w, own_lt[0], own_st[0]);
        if (w < 3) {
            a_tile(2 * w + 1, own_lt[1], own_st[1]);
        } else {
            own_lt[1] = 3;
            own_st[1] = 3;
        }
        own_lt[2] = w == 1 ? 2 : 3;
        own_st[2] = 2;
        nown = (w == 1 || w == 2) ? 3 : 2;
        nq = nown;
#pragma unroll
        for (int j = 0; j < MQ; ++j) qidx[j] = own_lt[j] * (own_lt[j] + 1) / 2 + own_st[j];
#pragma unroll
        for (int j = 0; j < MQ; ++j)
            if (j < nown && own_st[j] < 2) score_tile(own_lt[j], own_st[j], 0, m_r[j], m_i[j]);
        __syncthreads();  // every wave is done with B rows 0-31
        stage_plane(a.b_re, lds, 0, C / 2, BIPP);
        stage_plane(a.b_im, lds + BPLANE, BIPP % W, C / 2, BIPP);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
#pragma unroll
        for (int j = 0; j < MQ; ++j)
            if (j < nown && own_st[j] >= 2) score_tile(own_lt[j], own_st[j], C / 2, m_r[j], m_i[j]);
    } else {
        nq = q1 - q0;
#pragma unroll
        for (int j = 0; j < MQ; ++j) qidx[j] = q0 + j;
        {
            int lt = 0, st = q0;  // lt-major decode of q0
            while (st > lt) {
                st -= lt + 1;
                ++lt;
            }
#pragma unroll
            for (int j = 0; j < MQ; ++j) {
                if (q0 + j < q1) {  // wave-uniform
                    const int l0 = lt * 16, s0 = st * 16;
                    CTile gt;
                    ctile_zero(gt);
#pragma unroll
                    for (int k = 0; k < NK; ++k) {
                        const floatx4 br = row4(lds, s0 + li, 4 * k + g);
                        const floatx4 bi = row4(lds + PLANE, s0 + li, 4 * k + g);
                        const floatx4 cr = row4(ldc, l0 + li, 4 * k + g);
                        const floatx4 ci = row4(ldc + PLANE, l0 + li, 4 * k + g);
                        const floatx4 bs = br + bi, cs = cr + ci;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            ctile_mac(gt, br[e], bi[e], bs[e], cr[e], ci[e], cs[e]);
                    }
                    // register r <-> (l = l0 + li, s = s0 + 4g + r)
                    const int lrow = l0 + li;
                    const bool diag = (lt == st);
                    const double alr = lacs_r[lrow], ali = lacs_i[lrow];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int s = s0 + 4 * g + r;
                        const float gr = ctile_re(gt, r), gi = ctile_im(gt, r);
                        float lr = 0.f, lim = 0.f;
                        if (!diag || s <= lrow) {
                            const double d2 = alr - lacs_r[s];
                            double dv = ali - lacs_i[s];
                            dv -= rint(dv);
                            cexp_scaled((float)d2, (float)dv, lr, lim);
                        }
                        m_r[j][r] = gr * lr - gi * lim + ((diag && s == lrow) ? dk : 0.f);
                        m_i[j][r] = gr * lim + gi * lr;
                    }
                    if (++st > lt) {
                        st = 0;
                        ++lt;
                    }
                }
            }
        }
    }
    if constexpr (HB) {
        // the X block, late: its registers would not fit during the scores
#pragma unroll
        for (int st = 0; st < NLT; ++st)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t off = (uint32_t)(st * 16 + 4 * g + r) * sD + 16 * w + li;
                xreg_r[st][r] = buf_f32(rx_r, off);
                xreg_i[st][r] = buf_f32(rx_i, off);
            }
    }

    // ---- 3. the M tiles replace the B rows (or, with B in halves, the C rows)
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MQ; ++j) {
        if (j < nq) {
            const int q = qidx[j];
            *reinterpret_cast<floatx4*>(ldm + (2 * q) * 256 + 4 * lane) = m_r[j];
            *reinterpret_cast<floatx4*>(ldm + (2 * q + 1) * 256 + 4 * lane) = m_i[j];
        }
    }
    __syncthreads();

    // ---- 4. Y_diag: y[lt] += M(lt, st) X[st rows, this wave's columns]
#pragma unroll
    for (int st = 0; st < NLT; ++st) {
        float xs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) xs[r] = xreg_r[st][r] + xreg_i[st][r];
#pragma unroll
        for (int lt = st; lt < NLT; ++lt) {
            const int q = lt * (lt + 1) / 2 + st;
            const floatx4 mr = *reinterpret_cast<const floatx4*>(ldm + (2 * q) * 256 + 4 * lane);
            const floatx4 mi = *reinterpret_cast<const floatx4*>(ldm + (2 * q + 1) * 256 + 4 * lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ctile_mac(acc[lt], mr[r], mi[r], mr[r] + mi[r], xreg_r[st][r], xreg_i[st][r],
                          xs[r]);
        }
    }

    // ---- store; register r <-> row l = 16 lt + 4g + r (padded rows are dropped)
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t off = (uint32_t)(lt * 16 + 4 * g + r) * sD + 16 * w + li;
            buf_store_f32(ctile_re(acc[lt], r), ry_r, off);
            buf_store_f32(ctile_im(acc[lt], r), ry_i, off);
        }
    }
}

// Shapes the staged kernel takes: fp32 inputs, C <= 64, C * N <= 4096 (the
// chunk's B and C rows fit in LDS twice per CU), D/16 <= 4 waves, and not
// (C = 64, D = 16), where one wave would own all ten score tiles.
template <int C, int N, int D>
constexpr bool staged_shape() {
    return C <= 64 && C * N <= 4096 && D <= 64 && !(C == 64 && D == 16);
}

template <int C, int N, int D>
hipError_t launch_staged(const FwdArgs& f, hipStream_t s) {
    if constexpr (staged_shape<C, N, D>()) {
        ScanArgs a;
        a.x_re = f.x_re; a.x_im = f.x_im; a.b_re = f.b_re; a.b_im = f.b_im;
        a.c_re = f.c_re; a.c_im = f.c_im; a.dskip = f.dskip;
        a.acs_re = f.acs_re; a.acs_im = f.acs_im; a.e_re = f.e_re; a.e_im = f.e_im;
        a.hc_re = f.st_re; a.hc_im = f.st_im; a.y_re = f.y_re; a.y_im = f.y_im;
        a.T = f.T; a.H = (int)f.H; a.nC = (int)f.nC;
        a.nchunks = f.B * f.H * f.nC;
        hipLaunchKernelGGL((k_chunk_scan_lds<C, N, D>), dim3((unsigned)a.nchunks), dim3(4 * D), 0,
                           s, a);
        return hipGetLastError();
    } else {
        return launch_chunk_scan_regs<C>(f, s);
    }
}

template <int C, int N>
hipError_t launch_staged_d(const FwdArgs& f, hipStream_t s) {
    switch (f.D) {
        case 16: return launch_staged<C, N, 16>(f, s);
        case 32: return launch_staged<C, N, 32>(f, s);
        case 64: return launch_staged<C, N, 64>(f, s);
        default: return launch_staged<C, N, 128>(f, s);
    }
}

// The LDS-staged kernel where its shape allows, the register-operand kernel
// otherwise (and for bf16 inputs).

}  // namespace cssd
