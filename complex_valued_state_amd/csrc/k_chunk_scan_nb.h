// K2 for fp32 inputs at C = 64, N = 128, D = 64 (the phase-associative-memory
// shape, whose chunk rows do not fit in LDS at once): the same output as
// k_chunk_scan (see k_chunk_scan.h for the formulas and passages), with the
// state dimension n taken in two blocks of 64.
//
// A workgroup of four waves computes one chunk; wave w owns the output columns
// [16 w, 16 w + 16) of every row.  For each n block, the chunk's C and B rows
// restricted to that block are staged in LDS by direct-to-LDS buffer loads
// (16-byte pieces XOR-swizzled by the row, as in k_chunk_scan_lds), each wave
// loads its column block of H_c for those n, and two contractions over the
// block's n accumulate in registers:
//   Y_off += C[:, blk] H_c[blk, cols]    (every row tile)
//   G^T   += B[s tile, blk] C[l tile, blk]^T   (the wave's causal score tiles)
// After the second block: Y_off times exp(acs[l]) per row, M = G . L (+ Dskip on
// the diagonal) in registers, the M tiles exchanged through LDS over the B rows,
// the wave's block of X loaded, Y_diag = M X, and the stores.  68 KB of LDS:
// two workgroups per CU.
#pragma once

#include "k_chunk_scan_lds.h"

namespace cssd {

template <int C, int N, int D>
__global__ __launch_bounds__(64 * (D / 16)) __attribute__((amdgpu_waves_per_eu(2))) void
k_chunk_scan_nb(ScanArgs a) {
    constexpr int NB = 64;                    // n per block
    constexpr int NBLK = N / NB;              // blocks
    constexpr int KB = NB / 16;               // 16-wide n tiles per block
    constexpr int W = D / 16;                 // waves = column tiles of p
    constexpr int NLT = C / 16;               // row tiles per chunk
    constexpr int NP = NLT * (NLT + 1) / 2;   // causal tiles, lt-major
    constexpr int MQ = (NP + W - 1) / W;      // most tiles one wave owns
    constexpr int PLANE = C * NB;             // floats of one staged block plane
    constexpr int IPP = PLANE / 256;          // 64-lane x 16-byte loads per plane
    static_assert(C == 64 && N % NB == 0 && W == 4, "built for C = 64, D = 64, N = 64 k");
    static_assert(2 * NP * 256 <= 2 * PLANE, "the M tiles must fit over the B rows");
    static_assert(8 * C <= 1024, "a chunk's cumsums must fit one 1 KB slot");
    __shared__ floatx4 lds_b4[2 * PLANE / 4];  // B rows of the block, later the M tiles
    __shared__ floatx4 lds_c4[2 * PLANE / 4];  // C rows of the block
    __shared__ floatx4 lds_a4[1024 / 4];        // acs re, acs im, e re, e im
    float* const ldb = reinterpret_cast<float*>(lds_b4);
    float* const ldc = reinterpret_cast<float*>(lds_c4);
    float* const lda = reinterpret_cast<float*>(lds_a4);
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
    const int64_t row0 = (b * a.T + t0) * a.H + h;
    const uint32_t sN = (uint32_t)a.H * N, sD = (uint32_t)a.H * D;
    const uint32_t extN = (uint32_t)(valid - 1) * sN + N, extD = (uint32_t)(valid - 1) * sD + D;
    const BufRes rx_r = make_buf(static_cast<const float*>(a.x_re) + row0 * D, extD * 4);
    const BufRes rx_i = make_buf(static_cast<const float*>(a.x_im) + row0 * D, extD * 4);
    const BufRes ry_r = make_buf(a.y_re + row0 * D, extD * 4);
    const BufRes ry_i = make_buf(a.y_im + row0 * D, extD * 4);
    const BufRes rh_r = make_buf(a.hc_re + chunk * (int64_t)N * D, N * D * 4);
    const BufRes rh_i = make_buf(a.hc_im + chunk * (int64_t)N * D, N * D * 4);
    const int64_t pbase = bh * (int64_t)a.nC * C + t0;
    const float dk = a.dskip != nullptr ? a.dskip[h] : 0.f;

    // columns [NB blk, NB blk + NB) of one input plane's chunk rows: IPP 1 KB blocks
    // dealt round-robin to the waves; lane i's 16 bytes land at base + 16 i
    auto stage_plane = [&](const void* src, float* dst, int first, int blk) {
        const BufRes r = make_buf(static_cast<const float*>(src) + row0 * N, extN * 4);
        for (int q = (w - first + W) % W; q < IPP; q += W) {  // wave-uniform
            const int u = q * 64 + lane;  // physical 16-byte piece within the plane
            const int row = u / (NB / 4), pc = u % (NB / 4);
            const uint32_t voff = ((uint32_t)row * sN + NB * blk + 4 * lds_swz<NB>(row, pc)) * 4;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(dst + q * 256), 16, voff, 0, 0, 0);
        }
    };
    auto row4 = [&](const float* plane, int row, int ch) -> floatx4 {
        return *reinterpret_cast<const floatx4*>(plane + row * NB + 4 * lds_swz<NB>(row, ch));
    };

    // the score tiles this wave owns: q in [q0, q1), lt-major
    const int q0 = (w * NP) / W, q1 = ((w + 1) * NP) / W;
    int own_lt[MQ], own_st[MQ];
    {
        int lt = 0, st = q0;
        while (st > lt) {
            st -= lt + 1;
            ++lt;
        }
#pragma unroll
        for (int j = 0; j < MQ; ++j) {
            own_lt[j] = lt;
            own_st[j] = st;
            if (++st > lt) {
                st = 0;
                ++lt;
            }
        }
    }

    CTile acc[NLT];  // Y_off, then y
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) ctile_zero(acc[lt]);
    CTile gt[MQ];  // G^T of the owned score tiles
#pragma unroll
    for (int j = 0; j < MQ; ++j) ctile_zero(gt[j]);

#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
        if (blk > 0) __syncthreads();  // every wave is done with the previous block's rows
        stage_plane(a.c_re, ldc, 0, blk);
        stage_plane(a.c_im, ldc + PLANE, IPP % W, blk);
        stage_plane(a.b_re, ldb, (2 * IPP) % W, blk);
        stage_plane(a.b_im, ldb + PLANE, (3 * IPP) % W, blk);
        if (blk == 0 && w == W - 1) {
            const void* const aux[4] = {a.acs_re + pbase, a.acs_im + pbase, a.e_re + pbase,
                                        a.e_im + pbase};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(make_buf(aux[j], (j < 2 ? 8 : 4) * C),
                                                         (LdsPtr)(lda + 256 * j), 16, 16 * lane,
                                                         0, 0, 0);
        }
        // H_c[n = NB blk + 16 k + 4 g + e][16 w + li] (fragment order)
        floatx4 hreg_r[KB], hreg_i[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const uint32_t tile = (uint32_t)((KB * blk + k) * W + w);
            hreg_r[k] = buf_f32x4(rh_r, tile * 256 + 4 * lane);
            hreg_i[k] = buf_f32x4(rh_i, tile * 256 + 4 * lane);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
        // Y_off += C[:, blk] H_c[blk, cols]
#pragma unroll
        for (int k = 0; k < KB; ++k) {
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
        // G^T += B[s tile, blk] C[l tile, blk]^T for the owned tiles
#pragma unroll
        for (int j = 0; j < MQ; ++j) {
            if (q0 + j < q1) {  // wave-uniform
                const int l0 = own_lt[j] * 16, s0 = own_st[j] * 16;
#pragma unroll
                for (int k = 0; k < KB; ++k) {
                    const floatx4 br = row4(ldb, s0 + li, 4 * k + g);
                    const floatx4 bi = row4(ldb + PLANE, s0 + li, 4 * k + g);
                    const floatx4 cr = row4(ldc, l0 + li, 4 * k + g);
                    const floatx4 ci = row4(ldc + PLANE, l0 + li, 4 * k + g);
                    const floatx4 bs = br + bi, cs = cr + ci;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ctile_mac(gt[j], br[e], bi[e], bs[e], cr[e], ci[e], cs[e]);
                }
            }
        }
    }

    // accumulator register r <-> row l = 16 lt + 4 g + r: times exp(acs[l]), back
    // in Gauss form (t1 = re, t2 = 0, t3 = re + im)
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
    // M = G . L (+ Dskip on the diagonal); register r <-> (l = l0 + li, s = s0 + 4 g + r)
    floatx4 m_r[MQ], m_i[MQ];
#pragma unroll
    for (int j = 0; j < MQ; ++j) {
        if (q0 + j < q1) {
            const int lt = own_lt[j], st = own_st[j];
            const int lrow = lt * 16 + li;
            const bool diag = (lt == st);
            const double alr = lacs_r[lrow], ali = lacs_i[lrow];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = st * 16 + 4 * g + r;
                const float gr = ctile_re(gt[j], r), gi = ctile_im(gt[j], r);
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
        }
    }
    // the wave's block of X: X[16 st + 4 g + r][16 w + li]
    float xreg_r[NLT][4], xreg_i[NLT][4];
#pragma unroll
    for (int st = 0; st < NLT; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t off = (uint32_t)(st * 16 + 4 * g + r) * sD + 16 * w + li;
            xreg_r[st][r] = buf_f32(rx_r, off);
            xreg_i[st][r] = buf_f32(rx_i, off);
        }
    // the M tiles replace the B rows
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MQ; ++j) {
        if (q0 + j < q1) {
            const int q = q0 + j;
            *reinterpret_cast<floatx4*>(ldb + (2 * q) * 256 + 4 * lane) = m_r[j];
            *reinterpret_cast<floatx4*>(ldb + (2 * q + 1) * 256 + 4 * lane) = m_i[j];
        }
    }
    __syncthreads();
    // Y_diag: y[lt] += M(lt, st) X[st rows, this wave's columns]
#pragma unroll
    for (int st = 0; st < NLT; ++st) {
        float xs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) xs[r] = xreg_r[st][r] + xreg_i[st][r];
#pragma unroll
        for (int lt = st; lt < NLT; ++lt) {
            const int q = lt * (lt + 1) / 2 + st;
            const floatx4 mr = *reinterpret_cast<const floatx4*>(ldb + (2 * q) * 256 + 4 * lane);
            const floatx4 mi = *reinterpret_cast<const floatx4*>(ldb + (2 * q + 1) * 256 + 4 * lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ctile_mac(acc[lt], mr[r], mi[r], mr[r] + mi[r], xreg_r[st][r], xreg_i[st][r],
                          xs[r]);
        }
    }
    // stores; register r <-> row l = 16 lt + 4 g + r (padded rows are dropped)
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

template <int C, int N, int D>
hipError_t launch_chunk_scan_nb(const FwdArgs& f, hipStream_t s) {
    ScanArgs a;
    a.x_re = f.x_re; a.x_im = f.x_im; a.b_re = f.b_re; a.b_im = f.b_im;
    a.c_re = f.c_re; a.c_im = f.c_im; a.dskip = f.dskip;
    a.acs_re = f.acs_re; a.acs_im = f.acs_im; a.e_re = f.e_re; a.e_im = f.e_im;
    a.hc_re = f.st_re; a.hc_im = f.st_im; a.y_re = f.y_re; a.y_im = f.y_im;
    a.T = f.T; a.H = (int)f.H; a.nC = (int)f.nC;
    a.nchunks = f.B * f.H * f.nC;
    hipLaunchKernelGGL((k_chunk_scan_nb<C, N, D>), dim3((unsigned)a.nchunks), dim3(4 * D), 0, s, a);
    return hipGetLastError();
}

}  // namespace cssd
