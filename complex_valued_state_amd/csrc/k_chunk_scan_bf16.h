// K2 for bf16 inputs on the bf16 matrix cores (C = 64; N, D in {32, 64}): the
// same output as k_chunk_scan (see k_chunk_scan.h for the formulas and
// passages), with every product on v_mfma_f32_16x16x32_bf16 and fp32
// accumulation.
//
// That instruction takes A[i][k] from lane i + 16 (k / 8), slot k % 8, B[k][j]
// from lane j + 16 (k / 8), slot k % 8, and leaves D[4g + r][j] in register r
// of lane j + 16 g.  So an operand is "row i, the 8 values of k-chunk g":
//  * C and B rows are staged in LDS as bf16 by direct-to-LDS loads, 16-byte
//    chunks XOR-swizzled by the row (16 consecutive rows reading one logical
//    chunk hit 16 distinct bank slots), and one 16-byte read is an operand of
//    G^T = B C^T (A: B rows, B: C rows) or of the carried-state term C H_c (A:
//    C rows).
//  * G^T comes out with register r of lane l + 16g holding G[l][s = 4g + r]:
//    the layout of the fp32 kernel's score tiles, so M = G . L (+ Dskip on the
//    diagonal) is formed the same way in fp32 and only then rounded to bf16
//    (an operand, never a state) and exchanged through LDS.
//  * Y_diag contracts s in 32-steps pairing score tiles 2k, 2k + 1: slot j < 4
//    is s = 32k + 4g + j, slot j >= 4 is s = 32k + 16 + 4g + j - 4, which is
//    where the score tiles leave them; the X block is loaded in that order.
//  * The carried state H_c stays fp32 in memory; its fragment-order layout
//    gives each lane its 8 consecutive n as two float4 loads, rounded to bf16
//    for the product.
// Complex products are four real products (no Gauss form: sums of bf16
// operands would round), the imaginary operand negated once where needed.
#pragma once

#include "k_chunk_scan_lds.h"
#include "k_chunk_scan_nb.h"
#include "k_chunk_scan_wide.h"

namespace cssd {

typedef __bf16 bf16x8_k2 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_k2 __attribute__((ext_vector_type(4)));

// swizzled 16-byte chunk of a staged bf16 row of N values
template <int N>
__device__ __forceinline__ int bswz(int row, int c) {
    constexpr int RPW = 128 / N;  // rows per 256-byte bank window
    constexpr int NCH = N / 8;    // 16-byte chunks per row
    return c ^ ((row / RPW) & (NCH - 1));
}

__device__ __forceinline__ bf16x8_k2 bneg(bf16x8_k2 v) {
    uint4 u = __builtin_bit_cast(uint4, v);
    u.x ^= 0x80008000u;
    u.y ^= 0x80008000u;
    u.z ^= 0x80008000u;
    u.w ^= 0x80008000u;
    return __builtin_bit_cast(bf16x8_k2, u);
}

__device__ __forceinline__ floatx4 mfma_bf(bf16x8_k2 a, bf16x8_k2 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int N, int D>
__global__ __launch_bounds__(64 * (D / 16)) void k_chunk_scan_bf16(ScanArgs a) {
    constexpr int C = 64, NLT = 4, NP = 10;
    constexpr int W = D / 16;            // waves = 16-wide column tiles of p
    constexpr int NKS = N / 32;          // 32-wide k-steps over n
    constexpr int NCH = N / 8;           // 16-byte chunks per staged row
    constexpr int PLANE_B = C * N * 2;   // bytes of one staged plane
    constexpr int IPP = PLANE_B / 1024;  // 64-lane x 16-byte loads per plane
    constexpr int MQ = (NP + W - 1) / W;
    static_assert(PLANE_B % 1024 == 0, "whole 1 KB blocks");
    __shared__ __align__(16) unsigned char lds_b[2 * PLANE_B];  // B rows, re then im
    __shared__ __align__(16) unsigned char lds_c[2 * PLANE_B];  // C rows
    __shared__ __align__(16) unsigned char lds_m[NP * 1024];    // M tiles: [q][re, im][lane] 8 B
    __shared__ floatx4 lds_a4[1024 / 4];                        // acs re, acs im, e re, e im
    const float* const lda = reinterpret_cast<const float*>(lds_a4);
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
    const BufRes rx_r = make_buf(static_cast<const uint16_t*>(a.x_re) + row0 * D, extD * 2);
    const BufRes rx_i = make_buf(static_cast<const uint16_t*>(a.x_im) + row0 * D, extD * 2);
    const BufRes ry_r = make_buf(a.y_re + row0 * D, extD * 4);
    const BufRes ry_i = make_buf(a.y_im + row0 * D, extD * 4);
    const int64_t pbase = bh * (int64_t)a.nC * C + t0;
    const float dk = a.dskip != nullptr ? a.dskip[h] : 0.f;

    // ---- staging: C and B rows (bf16, swizzled 16-byte chunks), cumsums, exp(acs)
    auto stage_plane = [&](const void* src, unsigned char* dst, int first) {
        const BufRes r = make_buf(static_cast<const uint16_t*>(src) + row0 * N, extN * 2);
        for (int blk = (w - first + W) % W; blk < IPP; blk += W) {  // wave-uniform
            const int u = blk * 64 + lane;  // physical 16-byte chunk within the plane
            const int row = u / NCH, pc = u % NCH;
            const uint32_t voff = ((uint32_t)row * sN + 8 * bswz<N>(row, pc)) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(dst + blk * 1024), 16, voff, 0, 0, 0);
        }
    };
    stage_plane(a.c_re, lds_c, 0);
    stage_plane(a.c_im, lds_c + PLANE_B, IPP % W);
    stage_plane(a.b_re, lds_b, (2 * IPP) % W);
    stage_plane(a.b_im, lds_b + PLANE_B, (3 * IPP) % W);
    if (w == W - 1) {
        const void* const aux[4] = {a.acs_re + pbase, a.acs_im + pbase, a.e_re + pbase,
                                    a.e_im + pbase};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_buf(aux[j], (j < 2 ? 8 : 4) * C),
                                                     (LdsPtr)(reinterpret_cast<const char*>(lda) + 1024 * j),
                                                     16, 16 * lane, 0, 0, 0);
    }
    // H_c block, B operand of C H_c: slot j <-> n = 32 ks + 8g + j, p = 16w + li
    bf16x8_k2 h_r[NKS], h_i[NKS], h_ni[NKS];
    {
        const BufRes rh_r = make_buf(a.hc_re + chunk * (int64_t)N * D, N * D * 4);
        const BufRes rh_i = make_buf(a.hc_im + chunk * (int64_t)N * D, N * D * 4);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const uint32_t f0 = (uint32_t)((((2 * ks + (g >> 1)) * W + w) * 4 + 2 * (g & 1)) * 64 + li * 4);
            const floatx4 r0 = buf_f32x4(rh_r, f0), r1 = buf_f32x4(rh_r, f0 + 64);
            const floatx4 i0 = buf_f32x4(rh_i, f0), i1 = buf_f32x4(rh_i, f0 + 64);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h_r[ks][j] = (__bf16)r0[j];
                h_r[ks][j + 4] = (__bf16)r1[j];
                h_i[ks][j] = (__bf16)i0[j];
                h_i[ks][j + 4] = (__bf16)i1[j];
            }
            h_ni[ks] = bneg(h_i[ks]);
        }
    }
    // X block, B operand of M X: slot j <-> s = 32 k2 + 4g + j (j < 4), 32 k2 + 16 + 4g + j - 4
    bf16x8_k2 x_r[2], x_i[2], x_ni[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = 32 * k2 + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
            const uint32_t off = (uint32_t)s * sD + 16 * w + li;
            x_r[k2][j] = __builtin_bit_cast(__bf16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rx_r, off * 2u, 0, 0));
            x_i[k2][j] = __builtin_bit_cast(__bf16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rx_i, off * 2u, 0, 0));
        }
        x_ni[k2] = bneg(x_i[k2]);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();

    // operand: row `row` of a staged plane, logical 16-byte chunk `ch`
    auto rowop = [&](const unsigned char* plane, int row, int ch) -> bf16x8_k2 {
        return *reinterpret_cast<const bf16x8_k2*>(plane + row * (N * 2) + 16 * bswz<N>(row, ch));
    };

    // ---- 1. Y_off = diag(exp(acs)) C H_c on this wave's columns
    floatx4 yr[NLT], yi[NLT];
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) {
        yr[lt] = floatx4{0.f, 0.f, 0.f, 0.f};
        yi[lt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8_k2 cr = rowop(lds_c, 16 * lt + li, 4 * ks + g);
            const bf16x8_k2 ci = rowop(lds_c + PLANE_B, 16 * lt + li, 4 * ks + g);
            yr[lt] = mfma_bf(cr, h_r[ks], yr[lt]);
            yr[lt] = mfma_bf(ci, h_ni[ks], yr[lt]);
            yi[lt] = mfma_bf(cr, h_i[ks], yi[lt]);
            yi[lt] = mfma_bf(ci, h_r[ks], yi[lt]);
        }
        // register r <-> row l = 16 lt + 4g + r: multiply by exp(acs[l])
        const floatx4 er = *reinterpret_cast<const floatx4*>(le_r + lt * 16 + 4 * g);
        const floatx4 ei = *reinterpret_cast<const floatx4*>(le_i + lt * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float re = yr[lt][r], im = yi[lt][r];
            yr[lt][r] = er[r] * re - ei[r] * im;
            yi[lt][r] = er[r] * im + ei[r] * re;
        }
    }

    // ---- 2. score tiles q in [q0, q1): G^T = B C^T, M = G . L (+ Dskip) -> LDS (bf16)
    const int q0 = (w * NP) / W, q1 = ((w + 1) * NP) / W;
    {
        int lt = 0, st = q0;  // lt-major decode of q0
        while (st > lt) {
            st -= lt + 1;
            ++lt;
        }
#pragma unroll
        for (int jq = 0; jq < MQ; ++jq) {
            if (q0 + jq < q1) {  // wave-uniform
                const int l0 = lt * 16, s0 = st * 16;
                floatx4 gr = {0.f, 0.f, 0.f, 0.f}, gi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8_k2 br = rowop(lds_b, s0 + li, 4 * ks + g);
                    const bf16x8_k2 bi = rowop(lds_b + PLANE_B, s0 + li, 4 * ks + g);
                    const bf16x8_k2 cr = rowop(lds_c, l0 + li, 4 * ks + g);
                    const bf16x8_k2 ci = rowop(lds_c + PLANE_B, l0 + li, 4 * ks + g);
                    gr = mfma_bf(br, cr, gr);
                    gr = mfma_bf(bneg(bi), ci, gr);
                    gi = mfma_bf(br, ci, gi);
                    gi = mfma_bf(bi, cr, gi);
                }
                // register r <-> (l = l0 + li, s = s0 + 4g + r)
                const int lrow = l0 + li;
                const bool diag = (lt == st);
                const double alr = lacs_r[lrow], ali = lacs_i[lrow];
                bf16x4_k2 mr, mi;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = s0 + 4 * g + r;
                    float lr = 0.f, lim = 0.f;
                    if (!diag || s <= lrow) {
                        const double d2 = alr - lacs_r[s];
                        double dv = ali - lacs_i[s];
                        dv -= rint(dv);
                        cexp_scaled((float)d2, (float)dv, lr, lim);
                    }
                    mr[r] = (__bf16)(gr[r] * lr - gi[r] * lim + ((diag && s == lrow) ? dk : 0.f));
                    mi[r] = (__bf16)(gr[r] * lim + gi[r] * lr);
                }
                const int q = q0 + jq;
                *reinterpret_cast<bf16x4_k2*>(lds_m + q * 1024 + lane * 8) = mr;
                *reinterpret_cast<bf16x4_k2*>(lds_m + q * 1024 + 512 + lane * 8) = mi;
                if (++st > lt) {
                    st = 0;
                    ++lt;
                }
            }
        }
    }
    __syncthreads();

    // ---- 3. Y_diag: y[lt] += M(lt, .) X, s in 32-steps over the tile pairs (2k, 2k + 1)
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            if (2 * k2 > lt) continue;
            const int qa = lt * (lt + 1) / 2 + 2 * k2;
            const bool hi_tile = 2 * k2 + 1 <= lt;
            const bf16x4_k2 ar = *reinterpret_cast<const bf16x4_k2*>(lds_m + qa * 1024 + lane * 8);
            const bf16x4_k2 ai = *reinterpret_cast<const bf16x4_k2*>(lds_m + qa * 1024 + 512 + lane * 8);
            bf16x4_k2 br = {}, bi = {};
            if (hi_tile) {
                br = *reinterpret_cast<const bf16x4_k2*>(lds_m + (qa + 1) * 1024 + lane * 8);
                bi = *reinterpret_cast<const bf16x4_k2*>(lds_m + (qa + 1) * 1024 + 512 + lane * 8);
            }
            const bf16x8_k2 mr = {ar[0], ar[1], ar[2], ar[3], br[0], br[1], br[2], br[3]};
            const bf16x8_k2 mi = {ai[0], ai[1], ai[2], ai[3], bi[0], bi[1], bi[2], bi[3]};
            yr[lt] = mfma_bf(mr, x_r[k2], yr[lt]);
            yr[lt] = mfma_bf(mi, x_ni[k2], yr[lt]);
            yi[lt] = mfma_bf(mr, x_i[k2], yi[lt]);
            yi[lt] = mfma_bf(mi, x_r[k2], yi[lt]);
        }
    }

    // ---- store; register r <-> row l = 16 lt + 4g + r (padded rows are dropped)
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t off = (uint32_t)(lt * 16 + 4 * g + r) * sD + 16 * w + li;
            buf_store_f32(yr[lt][r], ry_r, off);
            buf_store_f32(yi[lt][r], ry_i, off);
        }
    }
}

template <int N, int D>
hipError_t launch_chunk_scan_bf16(const FwdArgs& f, hipStream_t s) {
    ScanArgs a;
    a.x_re = f.x_re; a.x_im = f.x_im; a.b_re = f.b_re; a.b_im = f.b_im;
    a.c_re = f.c_re; a.c_im = f.c_im; a.dskip = f.dskip;
    a.acs_re = f.acs_re; a.acs_im = f.acs_im; a.e_re = f.e_re; a.e_im = f.e_im;
    a.hc_re = f.st_re; a.hc_im = f.st_im; a.y_re = f.y_re; a.y_im = f.y_im;
    a.T = f.T; a.H = (int)f.H; a.nC = (int)f.nC;
    a.nchunks = f.B * f.H * f.nC;
    hipLaunchKernelGGL((k_chunk_scan_bf16<N, D>), dim3((unsigned)a.nchunks), dim3(4 * D), 0, s, a);
    return hipGetLastError();
}

// The chunk-scan step for chunk size C: bf16 inputs with C = 64 and N, D in
// {32, 64} on the bf16 matrix cores; fp32 inputs on the LDS-staged kernel where
// its shape rule holds; everything else on the register-operand kernel.
template <int C>
hipError_t launch_chunk_scan_c(const FwdArgs& f, hipStream_t s) {
    if (f.in_dtype != 0) {
        if constexpr (C == 64) {
            if (f.N == 64 && f.D == 64) return launch_chunk_scan_bf16<64, 64>(f, s);
            if (f.N == 64 && f.D == 32) return launch_chunk_scan_bf16<64, 32>(f, s);
            if (f.N == 32 && f.D == 64) return launch_chunk_scan_bf16<32, 64>(f, s);
            if (f.N == 32 && f.D == 32) return launch_chunk_scan_bf16<32, 32>(f, s);
        }
        return launch_chunk_scan_regs<C>(f, s);
    }
    if constexpr (C == 64) {
        if (f.N == 128 && f.D == 64) return launch_chunk_scan_nb<64, 128, 64>(f, s);
    }
    if constexpr (C == 128) {
        if (f.N == 128 && f.D == 64) return launch_chunk_scan_wide<128, 128, 64>(f, s);
    }
    switch (f.N) {
        case 16: return launch_staged_d<C, 16>(f, s);
        case 32: return launch_staged_d<C, 32>(f, s);
        case 64: return launch_staged_d<C, 64>(f, s);
        default: return launch_staged_d<C, 128>(f, s);
    }
}

}  // namespace cssd
