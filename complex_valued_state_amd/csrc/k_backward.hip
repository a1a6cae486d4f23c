// Gradient kernels of the chunkwise scan (fp32 inputs).
//
// The gradient of a real loss with respect to a complex value u + i v is the
// pair (dL/du, dL/dv), i.e. the complex number dL/du + i dL/dv -- the
// convention of the complex autograd the pages train this scan with
// (Mamba-3-Lite docs, "SSD Theory", autograd notes).  For w = c z the gradient
// reaching z is conj(c) grad(w) and the one reaching c is grad(w) conj(z).
//
// Walking the recurrence h_t = a_t h_{t-1} + B_t (x) x_t, y_t = C_t . h_t + D x_t
// backwards, G_t = dL/dh_t obeys G_t = conj(C_t) (x) dy_t + conj(a_{t+1}) G_{t+1},
// and dx_t = conj(B_t) . G_t + D dy_t, dB_t = G_t conj(x_t), dC_t = dy_t conj(h_t).
// Chunkwise (chunk c, rows t, l; L, e, w, cd, H_c as in the forward kernels;
// R_{c+1} = dL/dH_{c+1}, the gradient reaching the end of the chunk):
//   P   = dY X^H                                   (C x C)
//   dX  = (G . L)^H dY + diag(conj w) conj(B) R_{c+1} + D dY
//   dB  = (conj(L) . P)^T conj(C) + diag(conj w) conj(X) R_{c+1}^T
//   dC  = (conj(L) . P) conj(B) + diag(conj e) dY H_c^H
// with G = C B^T the forward score matrix.  R comes from the adjoint chunk
// pass R_c = Q_c + conj(cd[c]) R_{c+1}, Q_c = C^H diag(conj e) dY (the
// chunk-state and state-pass kernels in their adjoint modes).
//
// The log-decay gradient needs no per-element bookkeeping: summing the
// recurrence for G_t . conj(h_t) telescopes to
//   dz_t = sum_{l >= t} q_l + <dhT, hT>,
//   q_l  = sum_p dy_l[p] conj(y_l[p] - D x_l[p]) - conj(x_l[p]) (dx_l[p] - D dy_l[p])
// (z_t = softplus(dt_t) A, <u, v> = sum u conj(v)).  As y_l - D x_l = C_l . h_l and
// dC_l = dy_l conj(h_l), the first sum is conj(C_l) . dC_l, which the dC kernels
// form from their own output: y is never read, and q does not take the rounding
// of whatever forward produced y.  The part of the sum for dz_t from
// the start of chunk c + 1 onwards is <R_{c+1}, H_{c+1}> (the same telescoping
// stopped at a chunk boundary).  So for t in chunk c
//   dz_t = sum_{l >= t, l in chunk c} q_l + <R_{c+1}, H_{c+1}>,
// a chunk-local suffix sum plus a boundary term taken from the states, which
// keeps rounding from accumulating over the whole sequence.  Then ddt_t =
// sigmoid(dt_t) Re(dz_t conj(A)) and dA = sum_t softplus(dt_t) dz_t.
//
// MFMA mapping (16x16x4 fp32, lane = i + 16 g, Gauss complex products as in the
// forward kernels).  dX and dB (two kernels, PART 0 and 1): one wave per pair of
// row tiles {t, NLT-1-t} of the l axis (tile lt sums over the NLT - lt tiles
// tt >= lt).  For each (tt, lt), G (for dX) or P (for dB) comes out with
// register r holding [t = t0 + 4g + r][l = l0 + lane%16], which is the A-operand
// layout for the product with dY rows (dX) or conj(C) rows (dB).
// k_bwd_dc: one wave per pair of row tiles of the t axis; P is formed as
// conj(X) dY^T so that register r holds [t = t0 + lane%16][l = l0 + 4g + r], the
// A-operand layout for the product with conj(B) rows.  The state terms read
// R_{c+1} and H_c from their MFMA-fragment layout, directly for products that
// contract over n and element-wise (four loads per fragment row) for the
// transposed products that contract over p.
// At N = D = C = 64 the same three products run in the chunk-staged kernels
// k_bwd_lds<true> (dX), k_bwd_lds<false> (dB) and k_bwd_dc_lds (dC): one
// workgroup per chunk with its rows in LDS, the organisation of the forward
// chunk-scan kernel (the comments at those kernels give the details).
#include "cssd_device.h"
#include "cssd_launch.h"
#include "k_chunk_scan_lds.h"

namespace cssd {

namespace {

// element (n, p) of an N x D state block in MFMA-fragment order
template <int D>
__device__ __forceinline__ uint32_t frag_index(int n, int p) {
    return (uint32_t)((((n >> 4) * (D / 16) + (p >> 4)) * 4 + ((n & 15) >> 2)) * 64 +
                      (p & 15) * 4 + (n & 3));
}

// multiply the accumulator rows by a complex factor and put them back in Gauss form
__device__ __forceinline__ void ctile_scale(CTile& t, int r, float fr, float fi) {
    const float re = ctile_re(t, r), im = ctile_im(t, r);
    const float nr = fr * re - fi * im, ni = fr * im + fi * re;
    t.t1[r] = nr;
    t.t2[r] = 0.f;
    t.t3[r] = nr + ni;
}

// exp(acs[t] - acs[s]) or its conjugate, from the fp64 cumsums (log2 units / turns)
__device__ __forceinline__ void seg_exp(const double* ar, const double* ai, int t, int s, bool conj,
                                        float& lr, float& li) {
    const double d2 = ar[t] - ar[s];
    double dv = ai[t] - ai[s];
    dv -= rint(dv);
    cexp_scaled((float)d2, (float)(conj ? -dv : dv), lr, li);
}

// sum over the 16 lanes of a lane group, complete in the group's last lane
// (lane % 16 == 15): inclusive prefix sums by DPP row shifts of 1, 2, 4, 8, whose
// out-of-row sources read 0; the moves stay in the vector unit
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_total(float v) {
    v += dpp_f32<0x111>(v);  // row_shr:1
    v += dpp_f32<0x112>(v);  // row_shr:2
    v += dpp_f32<0x114>(v);  // row_shr:4
    v += dpp_f32<0x118>(v);  // row_shr:8
    return v;
}

// sum over the 16 lanes of a lane group (lane % 16 varies, lane / 16 fixed)
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// sum over the four lane groups (lane / 16 varies, lane % 16 fixed)
__device__ __forceinline__ float sum_groups(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

struct ChunkView {
    int64_t row0, pbase, chunk;
    int h, valid;
    uint32_t sN, sD, extN, extD;
};

__device__ __forceinline__ ChunkView chunk_view(const BwdArgs& a, int64_t chunk, int C, int N,
                                                int D) {
    ChunkView v;
    const FwdArgs& f = a.f;
    v.chunk = chunk;
    const int c = (int)(chunk % f.nC);
    const int64_t bh = chunk / f.nC;
    v.h = (int)(bh % f.H);
    const int64_t b = bh / f.H;
    const int64_t t0 = (int64_t)c * C;
    v.valid = (int)min<int64_t>((int64_t)C, f.T - t0);
    v.row0 = (b * f.T + t0) * f.H + v.h;
    v.pbase = bh * f.nC * C + t0;
    v.sN = (uint32_t)f.H * N;
    v.sD = (uint32_t)f.H * D;
    v.extN = (uint32_t)(v.valid - 1) * v.sN + N;
    v.extD = (uint32_t)(v.valid - 1) * v.sD + D;
    return v;
}

}  // namespace

// ----------------------------------------------------------------------------
// dX (DX = true) or dB (DX = false) for row tile lt of one chunk.  The two are
// separate kernels: dX needs only the forward scores G and dB only P, so the
// split does no extra matrix work and halves the live accumulators.
// ----------------------------------------------------------------------------
template <int C, int N, int D, bool DX>
__device__ __forceinline__ void dxdb_tile(const BwdArgs& a, int64_t chunk, int lt) {
    constexpr int NK = N / 16, PT = D / 16, NLT = C / 16;
    constexpr int NO = DX ? PT : NK;  // output column tiles
    const FwdArgs& f = a.f;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const ChunkView v = chunk_view(a, chunk, C, N, D);
    const int l0 = lt * 16;
    if (l0 >= v.valid) return;
    const BufRes rb_r = make_buf(static_cast<const float*>(f.b_re) + v.row0 * N, v.extN * 4);
    const BufRes rb_i = make_buf(static_cast<const float*>(f.b_im) + v.row0 * N, v.extN * 4);
    const BufRes rc_r = make_buf(static_cast<const float*>(f.c_re) + v.row0 * N, v.extN * 4);
    const BufRes rc_i = make_buf(static_cast<const float*>(f.c_im) + v.row0 * N, v.extN * 4);
    const BufRes rx_r = make_buf(static_cast<const float*>(f.x_re) + v.row0 * D, v.extD * 4);
    const BufRes rx_i = make_buf(static_cast<const float*>(f.x_im) + v.row0 * D, v.extD * 4);
    const BufRes rg_r = make_buf(a.dy_re + v.row0 * D, v.extD * 4);
    const BufRes rg_i = make_buf(a.dy_im + v.row0 * D, v.extD * 4);
    const BufRes rr_r = make_buf(a.r_re + chunk * (int64_t)N * D, N * D * 4);
    const BufRes rr_i = make_buf(a.r_im + chunk * (int64_t)N * D, N * D * 4);
    const double* __restrict__ ar = f.acs_re + v.pbase;
    const double* __restrict__ ai = f.acs_im + v.pbase;

    // rows l0 + li of B (dX) or X (dB): the A operand of the state term and the
    // B operand of the scores G (or P)
    constexpr int NQ = DX ? NK : PT;
    floatx4 oq_r[NQ], oq_i[NQ];
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        if constexpr (DX) {
            oq_r[k] = buf_f32x4(rb_r, (uint32_t)(l0 + li) * v.sN + 16 * k + 4 * g);
            oq_i[k] = buf_f32x4(rb_i, (uint32_t)(l0 + li) * v.sN + 16 * k + 4 * g);
        } else {
            oq_r[k] = buf_f32x4(rx_r, (uint32_t)(l0 + li) * v.sD + 16 * k + 4 * g);
            oq_i[k] = buf_f32x4(rx_i, (uint32_t)(l0 + li) * v.sD + 16 * k + 4 * g);
        }
    }

    // accumulators: register r <-> row l = l0 + 4g + r, column 16 tile + li
    CTile acc[NO];
#pragma unroll
    for (int k = 0; k < NO; ++k) ctile_zero(acc[k]);

    // ---- state term: conj(B) R (dX) or conj(X) R^T (dB), then the row factor conj(w[l])
    if constexpr (DX) {
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            const floatx4 br = oq_r[k], bi = -oq_i[k], bs = br + bi;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                // R[16k + 4g + e][16pt + li]
                const floatx4 rr = buf_f32x4(rr_r, (uint32_t)(k * PT + pt) * 256 + 4 * lane);
                const floatx4 ri = buf_f32x4(rr_i, (uint32_t)(k * PT + pt) * 256 + 4 * lane);
                const floatx4 rs = rr + ri;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ctile_mac(acc[pt], br[e], bi[e], bs[e], rr[e], ri[e], rs[e]);
            }
        }
    } else {
#pragma unroll
        for (int pk = 0; pk < PT; ++pk) {
            const floatx4 xr = oq_r[pk], xi = -oq_i[pk], xs = xr + xi;
#pragma unroll
            for (int nt = 0; nt < NK; ++nt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // R^T[p = 16pk + 4g + e][n = 16nt + li] = R[n][p]
                    const uint32_t fi = frag_index<D>(16 * nt + li, 16 * pk + 4 * g + e);
                    const float tr = buf_f32(rr_r, fi), ti = buf_f32(rr_i, fi);
                    ctile_mac(acc[nt], xr[e], xi[e], xs[e], tr, ti, tr + ti);
                }
            }
        }
    }
    {
        const floatx4 wr = *reinterpret_cast<const floatx4*>(f.w_re + v.pbase + l0 + 4 * g);
        const floatx4 wi = *reinterpret_cast<const floatx4*>(f.w_im + v.pbase + l0 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int k = 0; k < NO; ++k) ctile_scale(acc[k], r, wr[r], -wi[r]);
    }

    // ---- causal terms over the tiles tt >= lt
#pragma unroll
    for (int tt = 0; tt < NLT; ++tt) {
        if (tt < lt) continue;  // wave-uniform
        const int t0 = tt * 16;
        // dX: G[t][l] = C[t] . B[l];  dB: P[t][l] = dY[t] . conj(X[l]);
        // register r <-> t = t0 + 4g + r, l = l0 + li
        CTile sq;
        ctile_zero(sq);
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            if constexpr (DX) {
                const floatx4 cr = buf_f32x4(rc_r, (uint32_t)(t0 + li) * v.sN + 16 * k + 4 * g);
                const floatx4 ci = buf_f32x4(rc_i, (uint32_t)(t0 + li) * v.sN + 16 * k + 4 * g);
                const floatx4 cs = cr + ci, bs = oq_r[k] + oq_i[k];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ctile_mac(sq, cr[e], ci[e], cs[e], oq_r[k][e], oq_i[k][e], bs[e]);
            } else {
                const floatx4 gr = buf_f32x4(rg_r, (uint32_t)(t0 + li) * v.sD + 16 * k + 4 * g);
                const floatx4 gi = buf_f32x4(rg_i, (uint32_t)(t0 + li) * v.sD + 16 * k + 4 * g);
                const floatx4 gs = gr + gi, xs = oq_r[k] - oq_i[k];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ctile_mac(sq, gr[e], gi[e], gs[e], oq_r[k][e], -oq_i[k][e], xs[e]);
            }
        }
        float m_r[4], m_i[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 4 * g + r, l = l0 + li;
            float lr = 0.f, lim = 0.f;
            if (tt > lt || t >= l) seg_exp(ar, ai, t, l, false, lr, lim);
            const float s_r = ctile_re(sq, r), s_i = ctile_im(sq, r);
            if constexpr (DX) {
                m_r[r] = s_r * lr - s_i * lim;  // conj(G L)
                m_i[r] = -(s_r * lim + s_i * lr);
            } else {
                m_r[r] = lr * s_r + lim * s_i;  // conj(L) P
                m_i[r] = lr * s_i - lim * s_r;
            }
        }
        // dX += conj(G L)^T dY[tt];  dB += (conj(L) P)^T conj(C[tt]);
        // k-step r <-> t = t0 + 4g + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t trow = (uint32_t)(t0 + 4 * g + r);
            const float ms = m_r[r] + m_i[r];
#pragma unroll
            for (int k = 0; k < NO; ++k) {
                float yr, yi;
                if constexpr (DX) {
                    yr = buf_f32(rg_r, trow * v.sD + 16 * k + li);
                    yi = buf_f32(rg_i, trow * v.sD + 16 * k + li);
                } else {
                    yr = buf_f32(rc_r, trow * v.sN + 16 * k + li);
                    yi = -buf_f32(rc_i, trow * v.sN + 16 * k + li);
                }
                ctile_mac(acc[k], m_r[r], m_i[r], ms, yr, yi, yr + yi);
            }
        }
    }

    // ---- stores; for dX also the skip term and q1[l] = -sum_p conj(x[l][p]) dx[l][p]
    // (before the skip term); register r <-> row l = l0 + 4g + r
    if constexpr (DX) {
        const float dk = f.dskip != nullptr ? f.dskip[v.h] : 0.f;
        const BufRes rdx_r = make_buf(a.dx_re + v.row0 * D, v.extD * 4);
        const BufRes rdx_i = make_buf(a.dx_im + v.row0 * D, v.extD * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t lrow = (uint32_t)(l0 + 4 * g + r);
            float qr = 0.f, qi = 0.f;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const uint32_t off = lrow * v.sD + 16 * pt + li;
                const float xr = buf_f32(rx_r, off), xi = buf_f32(rx_i, off);
                const float gr = buf_f32(rg_r, off), gi = buf_f32(rg_i, off);
                const float vr = ctile_re(acc[pt], r), vi = ctile_im(acc[pt], r);
                qr += xr * vr + xi * vi;  // conj(x) dx
                qi += xr * vi - xi * vr;
                buf_store_f32(vr + dk * gr, rdx_r, off);
                buf_store_f32(vi + dk * gi, rdx_i, off);
            }
            qr = sum16(qr);
            qi = sum16(qi);
            if (li == 0) {
                a.q1_re[v.pbase + lrow] = -qr;
                a.q1_im[v.pbase + lrow] = -qi;
            }
        }
    } else {
        const BufRes rdb_r = make_buf(a.db_re + v.row0 * N, v.extN * 4);
        const BufRes rdb_i = make_buf(a.db_im + v.row0 * N, v.extN * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t lrow = (uint32_t)(l0 + 4 * g + r);
#pragma unroll
            for (int nt = 0; nt < NK; ++nt) {
                const uint32_t off = lrow * v.sN + 16 * nt + li;
                buf_store_f32(ctile_re(acc[nt], r), rdb_r, off);
                buf_store_f32(ctile_im(acc[nt], r), rdb_i, off);
            }
        }
    }
}

// ----------------------------------------------------------------------------
// dX for N = D = C = 64 with the chunk's rows staged through LDS (the forward
// chunk-scan kernel's organisation): one workgroup of four waves per chunk, wave
// w owning the output columns p in [16 w, 16 w + 16) of every row l.
//  0. the chunk's C and B rows (both planes) go to LDS by direct-to-LDS loads
//     (16-byte pieces, XOR-swizzled by row as in the forward kernel), with the
//     fp64 cumsums and w; each wave loads its column block of R_{c+1}
//     (fragment order) and of dY into registers.
//  1. state term: conj(B) R_{c+1} on the wave's columns, rows scaled by conj(w[l]).
//  2. the ten causal 16 x 16 tiles (t tile >= l tile) of G = C B^T are split over
//     the waves; M' = conj(G . L) comes out with register r holding
//     [l = l0 + lane%16][t = t0 + 4 (lane/16) + r], the A-operand layout of the
//     product with dY rows; the tiles are exchanged through LDS (over the C rows).
//  3. dX[l, p] += sum_t M'[l, t] dY[t, p] on the wave's columns, then the skip
//     term D dY, and q1[l] = -sum_p conj(x[l, p]) dx[l, p] (before the skip),
//     summed over the four waves' columns through LDS.
// Each operand row is fetched from memory once per chunk (the tile kernel read
// C and dY rows once per row tile it served, and R twice per wave).
// ----------------------------------------------------------------------------
template <bool DX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_bwd_lds(
    BwdArgs a) {
    constexpr int C = 64, N = 64, D = 64, NK = N / 16, W = D / 16, NLT = C / 16;
    static_assert(N == D, "the two staged row sets share one row width");
    constexpr int NP = NLT * (NLT + 1) / 2;  // causal tiles (tt >= lt), tt-major
    constexpr int MQ = (NP + W - 1) / W;
    constexpr int PLANE = C * N, IPP = PLANE / 256;
    constexpr int SPLANE = PLANE / 2, SIPP = SPLANE / 256;  // half of the first row set
    static_assert(NP * 512 <= 2 * PLANE, "the M tiles must fit over the second row set");
    // The first row set (the scores' A operand: C rows for dX, dY rows for dB) is
    // staged in halves, rows 32-63 for the seven tiles with tt >= 2, then rows
    // 0-31 for the other three; the second (B rows for dX, X rows for dB) whole.
    // That is 52 KB of LDS, three workgroups per CU.
    __shared__ floatx4 lds_s4[2 * SPLANE / 4];  // later the q1 partials (dX)
    __shared__ floatx4 lds_o4[2 * PLANE / 4];   // later the M tiles
    __shared__ floatx4 lds_a4[1024 / 4];       // acs re, acs im (fp64), w re, w im
    float* const lds_s = reinterpret_cast<float*>(lds_s4);
    float* const lds_o = reinterpret_cast<float*>(lds_o4);
    float* const lda = reinterpret_cast<float*>(lds_a4);
    const double* const lacs_r = reinterpret_cast<const double*>(lda);
    const double* const lacs_i = reinterpret_cast<const double*>(lda + 256);
    const float* const lw_r = lda + 512;
    const float* const lw_i = lda + 768;

    const FwdArgs& f = a.f;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int w = wave_id();
    const int64_t chunk = blockIdx.x;
    const ChunkView v = chunk_view(a, chunk, C, N, D);

    // ---- 0. staging
    // rows r0 .. r0 + nblk * 256 / N - 1 of one plane, swizzled by staged row index
    auto stage_plane = [&](const void* src, float* dst_plane, int first, int r0, int nblk) {
        const BufRes r = make_buf(static_cast<const float*>(src) + v.row0 * N, v.extN * 4);
        for (int blk = (w - first + W) % W; blk < nblk; blk += W) {  // wave-uniform
            const int u = blk * 64 + lane;  // physical 16-byte piece within the plane
            const int row = u / (N / 4), pc = u % (N / 4);
            const uint32_t voff = ((uint32_t)(r0 + row) * v.sN + 4 * lds_swz<N>(row, pc)) * 4;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(dst_plane + blk * 256), 16, voff,
                                                     0, 0, 0);
        }
    };
    const void* const s_re = DX ? f.c_re : a.dy_re;
    const void* const s_im = DX ? f.c_im : a.dy_im;
    stage_plane(s_re, lds_s, 0, C / 2, SIPP);
    stage_plane(s_im, lds_s + SPLANE, SIPP % W, C / 2, SIPP);
    stage_plane(DX ? f.b_re : f.x_re, lds_o, 0, 0, IPP);
    stage_plane(DX ? f.b_im : f.x_im, lds_o + PLANE, IPP % W, 0, IPP);
    if (w == W - 1) {
        const void* const aux[4] = {f.acs_re + v.pbase, f.acs_im + v.pbase, f.w_re + v.pbase,
                                    f.w_im + v.pbase};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_buf(aux[j], (j < 2 ? 8 : 4) * C),
                                                     (LdsPtr)(lda + 256 * j), 16, 16 * lane,
                                                     0, 0, 0);
    }
    const BufRes rr_r = make_buf(a.r_re + chunk * (int64_t)N * D, N * D * 4);
    const BufRes rr_i = make_buf(a.r_im + chunk * (int64_t)N * D, N * D * 4);
    // the state term's B operand: R_{c+1}[16k + 4g + e][16w + li] (dX, over n) or
    // R_{c+1}[16w + li][16k + 4g + e] (dB, over p, element-wise from the fragments)
    floatx4 rreg_r[NK], rreg_i[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        if constexpr (DX) {
            rreg_r[k] = buf_f32x4(rr_r, (uint32_t)(k * W + w) * 256 + 4 * lane);
            rreg_i[k] = buf_f32x4(rr_i, (uint32_t)(k * W + w) * 256 + 4 * lane);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t fi = frag_index<D>(16 * w + li, 16 * k + 4 * g + e);
                rreg_r[k][e] = buf_f32(rr_r, fi);
                rreg_i[k][e] = buf_f32(rr_i, fi);
            }
        }
    }
    // the causal product's B operand, rows 16 tt + 4g + r, column 16w + li:
    // dY (dX; also the skip term) or conj(C) (dB)
    const BufRes rg_r = DX ? make_buf(a.dy_re + v.row0 * D, v.extD * 4)
                           : make_buf(static_cast<const float*>(f.c_re) + v.row0 * N, v.extN * 4);
    const BufRes rg_i = DX ? make_buf(a.dy_im + v.row0 * D, v.extD * 4)
                           : make_buf(static_cast<const float*>(f.c_im) + v.row0 * N, v.extN * 4);
    float gy_r[NLT][4], gy_i[NLT][4];  // loaded after the scores (registers)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();

    auto row4 = [&](const float* plane, int row, int ch) -> floatx4 {
        return *reinterpret_cast<const floatx4*>(plane + row * N + 4 * lds_swz<N>(row, ch));
    };

    // ---- 1. state term conj(B[l]) R (dX) or conj(X[l]) R^T (dB), then the row
    // factor conj(w[l])
    CTile acc[NLT];
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) ctile_zero(acc[lt]);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        const floatx4 rr = rreg_r[k], ri = rreg_i[k], rs = rr + ri;
#pragma unroll
        for (int lt = 0; lt < NLT; ++lt) {
            const floatx4 br = row4(lds_o, lt * 16 + li, 4 * k + g);
            const floatx4 bi = -row4(lds_o + PLANE, lt * 16 + li, 4 * k + g);
            const floatx4 bs = br + bi;
#pragma unroll
            for (int e = 0; e < 4; ++e) ctile_mac(acc[lt], br[e], bi[e], bs[e], rr[e], ri[e], rs[e]);
        }
    }
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) {
        const floatx4 wr = *reinterpret_cast<const floatx4*>(lw_r + lt * 16 + 4 * g);
        const floatx4 wi = *reinterpret_cast<const floatx4*>(lw_i + lt * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) ctile_scale(acc[lt], r, wr[r], -wi[r]);
    }

    // ---- 2. score tiles -> M in registers:
    // dX: G = C B^T, M = conj(G L);  dB: P = dY X^H, M = conj(L) P
    floatx4 m_r[MQ], m_i[MQ];
    // tile q (tt-major) with the first row set staged from row s0 on
    auto score_tile = [&](int q, int s0, floatx4& mr, floatx4& mi) {
        int tt = 0, lt = q;  // tt-major decode
        while (lt > tt) {
            lt -= tt + 1;
            ++tt;
        }
        const int t0 = tt * 16, l0 = lt * 16;
        CTile sq;
        ctile_zero(sq);
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            const floatx4 cr = row4(lds_s, t0 - s0 + li, 4 * k + g);
            const floatx4 ci = row4(lds_s + SPLANE, t0 - s0 + li, 4 * k + g);
            const floatx4 br = row4(lds_o, l0 + li, 4 * k + g);
            const floatx4 bi0 = row4(lds_o + PLANE, l0 + li, 4 * k + g);
            const floatx4 bi = DX ? bi0 : -bi0;
            const floatx4 cs = cr + ci, bs = br + bi;
#pragma unroll
            for (int e = 0; e < 4; ++e) ctile_mac(sq, cr[e], ci[e], cs[e], br[e], bi[e], bs[e]);
        }
        // register r <-> (t = t0 + 4g + r, l = l0 + li)
        const int l = l0 + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 4 * g + r;
            float lr = 0.f, lim = 0.f;
            if (tt > lt || t >= l) seg_exp(lacs_r, lacs_i, t, l, false, lr, lim);
            const float s_r = ctile_re(sq, r), s_i = ctile_im(sq, r);
            if constexpr (DX) {
                mr[r] = s_r * lr - s_i * lim;  // conj(G L)
                mi[r] = -(s_r * lim + s_i * lr);
            } else {
                mr[r] = lr * s_r + lim * s_i;  // conj(L) P
                mi[r] = lr * s_i - lim * s_r;
            }
        }
    };
    // tiles per wave, in fixed slots: the seven with tt >= 2 (q = 3 .. 9) as
    // q = 3 + 2w and 4 + 2w (wave 3: 9 only), then q = 0, 1, 2 to waves 1, 2, 3
    int qs[MQ];
    qs[0] = 3 + 2 * w;
    qs[1] = w < 3 ? 4 + 2 * w : 2;
    qs[2] = w == 1 ? 0 : 1;
    const int nq = (w == 1 || w == 2) ? 3 : 2;
    static_assert(MQ == 3 && W == 4 && NLT == 4, "the split is for C = 64");
#pragma unroll
    for (int j = 0; j < MQ; ++j)
        if (j < nq && qs[j] >= 3) score_tile(qs[j], C / 2, m_r[j], m_i[j]);
    __syncthreads();  // every wave is done with rows 32-63 of the first set
    stage_plane(s_re, lds_s, 0, 0, SIPP);
    stage_plane(s_im, lds_s + SPLANE, SIPP % W, 0, SIPP);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MQ; ++j)
        if (j < nq && qs[j] < 3) score_tile(qs[j], 0, m_r[j], m_i[j]);
    // the causal product's B operand, rows 16 tt + 4g + r, column 16w + li
#pragma unroll
    for (int tt = 0; tt < NLT; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t off = (uint32_t)(tt * 16 + 4 * g + r) * (DX ? v.sD : v.sN) + 16 * w + li;
            gy_r[tt][r] = buf_f32(rg_r, off);
            gy_i[tt][r] = DX ? buf_f32(rg_i, off) : -buf_f32(rg_i, off);
        }

    // ---- the M tiles replace the second row set
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MQ; ++j) {
        if (j < nq) {
            const int q = qs[j];
            *reinterpret_cast<floatx4*>(lds_o + (2 * q) * 256 + 4 * lane) = m_r[j];
            *reinterpret_cast<floatx4*>(lds_o + (2 * q + 1) * 256 + 4 * lane) = m_i[j];
        }
    }
    __syncthreads();

    // dX: x[16 lt + 4g + r][16w + li] for q1, in flight during the products below
    // (loaded only at the stores, its latency was not hidden: 0.79 -> 0.62 ms)
    const BufRes rx_r = make_buf(static_cast<const float*>(f.x_re) + v.row0 * D, v.extD * 4);
    const BufRes rx_i = make_buf(static_cast<const float*>(f.x_im) + v.row0 * D, v.extD * 4);
    float xb_r[NLT][4], xb_i[NLT][4];
    if constexpr (DX) {
#pragma unroll
        for (int lt = 0; lt < NLT; ++lt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t off = (uint32_t)(lt * 16 + 4 * g + r) * v.sD + 16 * w + li;
                xb_r[lt][r] = buf_f32(rx_r, off);
                xb_i[lt][r] = buf_f32(rx_i, off);
            }
    }

    // ---- 3. out[lt] += M(lt, tt) . (dY or conj C)[tt rows, this wave's columns], tt >= lt
#pragma unroll
    for (int tt = 0; tt < NLT; ++tt) {
        float ys[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ys[r] = gy_r[tt][r] + gy_i[tt][r];
#pragma unroll
        for (int lt = 0; lt <= tt; ++lt) {
            const int q = tt * (tt + 1) / 2 + lt;
            const floatx4 mr = *reinterpret_cast<const floatx4*>(lds_o + (2 * q) * 256 + 4 * lane);
            const floatx4 mi = *reinterpret_cast<const floatx4*>(lds_o + (2 * q + 1) * 256 + 4 * lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ctile_mac(acc[lt], mr[r], mi[r], mr[r] + mi[r], gy_r[tt][r], gy_i[tt][r], ys[r]);
        }
    }

    if constexpr (!DX) {
        // ---- dB stores; register r <-> row l = 16 lt + 4g + r, column n = 16w + li
        const BufRes rdb_r = make_buf(a.db_re + v.row0 * N, v.extN * 4);
        const BufRes rdb_i = make_buf(a.db_im + v.row0 * N, v.extN * 4);
#pragma unroll
        for (int lt = 0; lt < NLT; ++lt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t off = (uint32_t)(lt * 16 + 4 * g + r) * v.sN + 16 * w + li;
                buf_store_f32(ctile_re(acc[lt], r), rdb_r, off);
                buf_store_f32(ctile_im(acc[lt], r), rdb_i, off);
            }
        return;
    } else {
        // ---- dX stores: dx = acc + D dY; q1 partials of this wave's 16 columns
        const float dk = f.dskip != nullptr ? f.dskip[v.h] : 0.f;
        const BufRes rdx_r = make_buf(a.dx_re + v.row0 * D, v.extD * 4);
        const BufRes rdx_i = make_buf(a.dx_im + v.row0 * D, v.extD * 4);
        float* const qpart = lds_s;  // [wave][row][re, im]; the first row set is no longer read
        // conj(x) dx for the 16 rows m = 4 lt + r of this lane's column
        float pr[16], pi[16];
#pragma unroll
        for (int lt = 0; lt < NLT; ++lt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int lrow = lt * 16 + 4 * g + r;
                const uint32_t off = (uint32_t)lrow * v.sD + 16 * w + li;
                const float xr = xb_r[lt][r], xi = xb_i[lt][r];
                const float vr = ctile_re(acc[lt], r), vi = ctile_im(acc[lt], r);
                pr[4 * lt + r] = xr * vr + xi * vi;
                pi[4 * lt + r] = xr * vi - xi * vr;
                buf_store_f32(vr + dk * gy_r[lt][r], rdx_r, off);
                buf_store_f32(vi + dk * gy_i[lt][r], rdx_i, off);
            }
        // sum each row over the wave's 16 columns (a butterfly that leaves lane li
        // with row li measured slower than these per-row sums)
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            pr[m] = sum16(pr[m]);
            pi[m] = sum16(pi[m]);
        }
        if (li == 0)
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int lrow = (m >> 2) * 16 + 4 * g + (m & 3);
                qpart[(w * C + lrow) * 2] = pr[m];
                qpart[(w * C + lrow) * 2 + 1] = pi[m];
            }
        __syncthreads();
        if (threadIdx.x < 2 * C) {
            const int lrow = threadIdx.x >> 1, part = threadIdx.x & 1;
            float sum = 0.f;
#pragma unroll
            for (int ww = 0; ww < W; ++ww) sum += qpart[(ww * C + lrow) * 2 + part];
            (part ? a.q1_im : a.q1_re)[v.pbase + lrow] = -sum;
        }
    }
}
// ----------------------------------------------------------------------------
// dC for N = D = C = 64, staged per chunk like k_bwd_lds: one workgroup per
// chunk, wave w owning the output columns n in [16 w, 16 w + 16) of every row t.
// The chunk's dY and X rows go to LDS; each wave loads its column blocks of
// conj(H_c) (element-wise from the fragments) and conj(B) into registers.
//  1. state term dY H_c^H on the wave's columns, rows scaled by conj(e[t]);
//     wave w also forms the dD partial of rows [16 w, 16 w + 16).
//  2. the causal tiles of P^T = conj(X) dY^T (t tile >= l tile) split over the
//     waves; K = conj(L) P comes out with register r holding
//     [t = t0 + lane%16][l = l0 + 4 (lane/16) + r], the A-operand layout of
//     the product with conj(B) rows; exchanged through LDS (over the X rows).
//  3. dC[t, n] += sum_l K[t, l] conj(B[l, n]); then q2[t] = conj(C[t]) . dC[t].
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_bwd_dc_lds(
    BwdArgs a) {
    constexpr int C = 64, N = 64, D = 64, NK = N / 16, PT = D / 16, W = N / 16, NLT = C / 16;
    static_assert(N == D, "the two staged row sets share one row width");
    constexpr int NP = NLT * (NLT + 1) / 2;  // causal tiles (tt >= lt), tt-major
    constexpr int MQ = (NP + W - 1) / W;
    constexpr int PLANE = C * D, IPP = PLANE / 256;
    constexpr int XPLANE = PLANE / 2, XIPP = XPLANE / 256;  // half of the X rows
    // The X rows are staged in halves: rows 0-31 for the seven tiles with lt < 2
    // (and the dD rows of waves 0 and 1), then rows 32-63 for the other three
    // (and waves 2 and 3): 52 KB of LDS, three workgroups per CU.
    __shared__ floatx4 lds_g4[2 * PLANE / 4];   // dY rows, later the K tiles
    __shared__ floatx4 lds_x4[2 * XPLANE / 4];  // X rows, half at a time
    __shared__ floatx4 lds_a4[1024 / 4];       // acs re, acs im (fp64), e re, e im
    float* const ldg = reinterpret_cast<float*>(lds_g4);
    float* const ldx = reinterpret_cast<float*>(lds_x4);
    float* const lda = reinterpret_cast<float*>(lds_a4);
    const double* const lacs_r = reinterpret_cast<const double*>(lda);
    const double* const lacs_i = reinterpret_cast<const double*>(lda + 256);
    const float* const le_r = lda + 512;
    const float* const le_i = lda + 768;

    const FwdArgs& f = a.f;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int w = wave_id();
    const int64_t chunk = blockIdx.x;
    const ChunkView v = chunk_view(a, chunk, C, N, D);

    // ---- 0. staging
    // rows r0 .. r0 + nblk * 256 / D - 1 of one plane, swizzled by staged row index
    auto stage_plane = [&](const void* src, float* dst_plane, int first, int r0, int nblk) {
        const BufRes r = make_buf(static_cast<const float*>(src) + v.row0 * D, v.extD * 4);
        for (int blk = (w - first + W) % W; blk < nblk; blk += W) {  // wave-uniform
            const int u = blk * 64 + lane;  // physical 16-byte piece within the plane
            const int row = u / (D / 4), pc = u % (D / 4);
            const uint32_t voff = ((uint32_t)(r0 + row) * v.sD + 4 * lds_swz<D>(row, pc)) * 4;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(dst_plane + blk * 256), 16, voff,
                                                     0, 0, 0);
        }
    };
    stage_plane(a.dy_re, ldg, 0, 0, IPP);
    stage_plane(a.dy_im, ldg + PLANE, IPP % W, 0, IPP);
    stage_plane(f.x_re, ldx, 0, 0, XIPP);
    stage_plane(f.x_im, ldx + XPLANE, XIPP % W, 0, XIPP);
    if (w == W - 1) {
        const void* const aux[4] = {f.acs_re + v.pbase, f.acs_im + v.pbase, f.e_re + v.pbase,
                                    f.e_im + v.pbase};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_buf(aux[j], (j < 2 ? 8 : 4) * C),
                                                     (LdsPtr)(lda + 256 * j), 16, 16 * lane,
                                                     0, 0, 0);
    }
    // conj(H_c[16w + li][16k + 4g + e]), the B operand of the state term
    const BufRes rh_r = make_buf(f.st_re + chunk * (int64_t)N * D, N * D * 4);
    const BufRes rh_i = make_buf(f.st_im + chunk * (int64_t)N * D, N * D * 4);
    floatx4 hreg_r[PT], hreg_i[PT];
#pragma unroll
    for (int k = 0; k < PT; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t fi = frag_index<D>(16 * w + li, 16 * k + 4 * g + e);
            hreg_r[k][e] = buf_f32(rh_r, fi);
            hreg_i[k][e] = -buf_f32(rh_i, fi);
        }
    // conj(B[16 lt + 4g + r][16w + li]), the B operand of step 3 (loaded after the scores)
    const BufRes rb_r = make_buf(static_cast<const float*>(f.b_re) + v.row0 * N, v.extN * 4);
    const BufRes rb_i = make_buf(static_cast<const float*>(f.b_im) + v.row0 * N, v.extN * 4);
    float cb_r[NLT][4], cb_i[NLT][4];
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();

    auto row4 = [&](const float* plane, int row, int ch) -> floatx4 {
        return *reinterpret_cast<const floatx4*>(plane + row * D + 4 * lds_swz<D>(row, ch));
    };

    // ---- the dD partial Re(dy . conj(x)) for row t = 16 w + li, with the X rows
    // staged from row x0 on (called in the phase that holds row t)
    auto dd_row = [&](int x0) {
        const int t = 16 * w + li;
        float dd = 0.f;
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const floatx4 gr = row4(ldg, t, 4 * k + g), gi = row4(ldg + PLANE, t, 4 * k + g);
            const floatx4 xr = row4(ldx, t - x0, 4 * k + g);
            const floatx4 xi = row4(ldx + XPLANE, t - x0, 4 * k + g);
#pragma unroll
            for (int e = 0; e < 4; ++e) dd += gr[e] * xr[e] + gi[e] * xi[e];
        }
        dd = sum_groups(dd);
        if (g == 0) a.ddp[v.pbase + t] = dd;
    };
    if (w < 2) dd_row(0);

    // ---- 1. state term dY H_c^H, then the row factor conj(e[t])
    CTile acc[NLT];
#pragma unroll
    for (int tt = 0; tt < NLT; ++tt) ctile_zero(acc[tt]);
#pragma unroll
    for (int k = 0; k < PT; ++k) {
        const floatx4 hr = hreg_r[k], hi = hreg_i[k], hs = hr + hi;
#pragma unroll
        for (int tt = 0; tt < NLT; ++tt) {
            const floatx4 gr = row4(ldg, tt * 16 + li, 4 * k + g);
            const floatx4 gi = row4(ldg + PLANE, tt * 16 + li, 4 * k + g);
            const floatx4 gs = gr + gi;
#pragma unroll
            for (int e = 0; e < 4; ++e) ctile_mac(acc[tt], gr[e], gi[e], gs[e], hr[e], hi[e], hs[e]);
        }
    }
#pragma unroll
    for (int tt = 0; tt < NLT; ++tt) {
        const floatx4 er = *reinterpret_cast<const floatx4*>(le_r + tt * 16 + 4 * g);
        const floatx4 ei = *reinterpret_cast<const floatx4*>(le_i + tt * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) ctile_scale(acc[tt], r, er[r], -ei[r]);
    }

    // ---- 2. tiles (tt, lt), lt <= tt: P^T = conj(X) dY^T, K = conj(L) P
    floatx4 m_r[MQ], m_i[MQ];
    // tile q (tt-major) with the X rows staged from row x0 on
    auto score_tile = [&](int q, int x0, floatx4& mr, floatx4& mi) {
        int tt = 0, lt = q;  // tt-major decode
        while (lt > tt) {
            lt -= tt + 1;
            ++tt;
        }
        const int t0 = tt * 16, l0 = lt * 16;
        CTile pq;
        ctile_zero(pq);
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const floatx4 xr = row4(ldx, l0 - x0 + li, 4 * k + g);
            const floatx4 xi = -row4(ldx + XPLANE, l0 - x0 + li, 4 * k + g);
            const floatx4 gr = row4(ldg, t0 + li, 4 * k + g);
            const floatx4 gi = row4(ldg + PLANE, t0 + li, 4 * k + g);
            const floatx4 xs = xr + xi, gs = gr + gi;
#pragma unroll
            for (int e = 0; e < 4; ++e) ctile_mac(pq, xr[e], xi[e], xs[e], gr[e], gi[e], gs[e]);
        }
        // register r <-> (t = t0 + li, l = l0 + 4g + r)
        const int t = t0 + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int l = l0 + 4 * g + r;
            float lr = 0.f, lim = 0.f;
            if (lt < tt || t >= l) seg_exp(lacs_r, lacs_i, t, l, false, lr, lim);
            const float p_r = ctile_re(pq, r), p_i = ctile_im(pq, r);
            mr[r] = lr * p_r + lim * p_i;  // conj(L) P
            mi[r] = lr * p_i - lim * p_r;
        }
    };
    // tiles per wave, in fixed slots: the seven with lt < 2 (q = 0 1 2 3 4 6 7)
    // two per wave (wave 3 one), then q = 5, 8, 9 to waves 1, 2, 3
    auto a_tile = [](int i) { return i < 5 ? i : i + 1; };
    int qs[MQ];
    qs[0] = a_tile(2 * w);
    qs[1] = w < 3 ? a_tile(2 * w + 1) : 9;
    qs[2] = w == 1 ? 5 : 8;
    const int nq = (w == 1 || w == 2) ? 3 : 2;
    static_assert(MQ == 3 && W == 4 && NLT == 4, "the split is for C = 64");
    auto second_half = [](int q) { return q == 5 || q >= 8; };
#pragma unroll
    for (int j = 0; j < MQ; ++j)
        if (j < nq && !second_half(qs[j])) score_tile(qs[j], 0, m_r[j], m_i[j]);
    __syncthreads();  // every wave is done with X rows 0-31
    stage_plane(f.x_re, ldx, 0, C / 2, XIPP);
    stage_plane(f.x_im, ldx + XPLANE, XIPP % W, C / 2, XIPP);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (w >= 2) dd_row(C / 2);
#pragma unroll
    for (int j = 0; j < MQ; ++j)
        if (j < nq && second_half(qs[j])) score_tile(qs[j], C / 2, m_r[j], m_i[j]);
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t off = (uint32_t)(lt * 16 + 4 * g + r) * v.sN + 16 * w + li;
            cb_r[lt][r] = buf_f32(rb_r, off);
            cb_i[lt][r] = -buf_f32(rb_i, off);
        }

    // ---- the K tiles replace the dY rows
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MQ; ++j) {
        if (j < nq) {
            const int q = qs[j];
            *reinterpret_cast<floatx4*>(ldg + (2 * q) * 256 + 4 * lane) = m_r[j];
            *reinterpret_cast<floatx4*>(ldg + (2 * q + 1) * 256 + 4 * lane) = m_i[j];
        }
    }
    __syncthreads();

    // ---- 3. dC[tt] += K(tt, lt) conj(B)[lt rows, this wave's columns], lt <= tt.
    // Row tile lt of dC is complete after step lt (it sums the tiles lt' <= lt):
    // it is stored there, and its part of q2[t] = conj(C[t]) . dC[t] (this wave's
    // 16 columns, summed over the lane group) goes to LDS, where the cumsums and e
    // are no longer read (two barriers since step 2); the C values are loaded at
    // the top of the step, ahead of its matrix products.
    const BufRes rdc_r = make_buf(a.dc_re + v.row0 * N, v.extN * 4);
    const BufRes rdc_i = make_buf(a.dc_im + v.row0 * N, v.extN * 4);
    const BufRes rc_r = make_buf(static_cast<const float*>(f.c_re) + v.row0 * N, v.extN * 4);
    const BufRes rc_i = make_buf(static_cast<const float*>(f.c_im) + v.row0 * N, v.extN * 4);
    float* const lq = lda;  // [W][C][2]
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) {
        float qc_r[4], qc_i[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t off = (uint32_t)(lt * 16 + 4 * g + r) * v.sN + 16 * w + li;
            qc_r[r] = buf_f32(rc_r, off);
            qc_i[r] = buf_f32(rc_i, off);
        }
        float bs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) bs[r] = cb_r[lt][r] + cb_i[lt][r];
#pragma unroll
        for (int tt = lt; tt < NLT; ++tt) {
            const int q = tt * (tt + 1) / 2 + lt;
            const floatx4 mr = *reinterpret_cast<const floatx4*>(ldg + (2 * q) * 256 + 4 * lane);
            const floatx4 mi = *reinterpret_cast<const floatx4*>(ldg + (2 * q + 1) * 256 + 4 * lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ctile_mac(acc[tt], mr[r], mi[r], mr[r] + mi[r], cb_r[lt][r], cb_i[lt][r], bs[r]);
        }
        // stores and q2 part of row tile lt; register r <-> row t = 16 lt + 4g + r,
        // column n = 16w + li
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = lt * 16 + 4 * g + r;
            const uint32_t off = (uint32_t)t * v.sN + 16 * w + li;
            const float dr = ctile_re(acc[lt], r), di = ctile_im(acc[lt], r);
            buf_store_f32(dr, rdc_r, off);
            buf_store_f32(di, rdc_i, off);
            const float pr = row_total(qc_r[r] * dr + qc_i[r] * di);
            const float pi = row_total(qc_r[r] * di - qc_i[r] * dr);
            if (li == 15) {
                lq[(w * C + t) * 2] = pr;
                lq[(w * C + t) * 2 + 1] = pi;
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < C) {
        const int t = threadIdx.x;
        float qr = 0.f, qi = 0.f;
#pragma unroll
        for (int u = 0; u < W; ++u) {
            qr += lq[(u * C + t) * 2];
            qi += lq[(u * C + t) * 2 + 1];
        }
        a.q2_re[v.pbase + t] = qr;
        a.q2_im[v.pbase + t] = qi;
    }
}

// ----------------------------------------------------------------------------
// dC for row tile tt of one chunk, plus the dC half of q and the dD partials
// ----------------------------------------------------------------------------
template <int C, int N, int D>
__device__ __forceinline__ void dc_tile(const BwdArgs& a, int64_t chunk, int tt) {
    constexpr int NK = N / 16, PT = D / 16;
    const FwdArgs& f = a.f;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const ChunkView v = chunk_view(a, chunk, C, N, D);
    const int t0 = tt * 16;
    if (t0 >= v.valid) return;
    const BufRes rb_r = make_buf(static_cast<const float*>(f.b_re) + v.row0 * N, v.extN * 4);
    const BufRes rb_i = make_buf(static_cast<const float*>(f.b_im) + v.row0 * N, v.extN * 4);
    const BufRes rx_r = make_buf(static_cast<const float*>(f.x_re) + v.row0 * D, v.extD * 4);
    const BufRes rx_i = make_buf(static_cast<const float*>(f.x_im) + v.row0 * D, v.extD * 4);
    const BufRes rg_r = make_buf(a.dy_re + v.row0 * D, v.extD * 4);
    const BufRes rg_i = make_buf(a.dy_im + v.row0 * D, v.extD * 4);
    const BufRes rh_r = make_buf(f.st_re + chunk * (int64_t)N * D, N * D * 4);
    const BufRes rh_i = make_buf(f.st_im + chunk * (int64_t)N * D, N * D * 4);
    const double* __restrict__ ar = f.acs_re + v.pbase;
    const double* __restrict__ ai = f.acs_im + v.pbase;

    // rows t0 + li of dY, as A-operand (over p) and as B-operand of conj(X) dY^T
    floatx4 gq_r[PT], gq_i[PT];
#pragma unroll
    for (int k = 0; k < PT; ++k) {
        gq_r[k] = buf_f32x4(rg_r, (uint32_t)(t0 + li) * v.sD + 16 * k + 4 * g);
        gq_i[k] = buf_f32x4(rg_i, (uint32_t)(t0 + li) * v.sD + 16 * k + 4 * g);
    }

    // ---- the dD partial Re(dy . conj(x)) for rows t = t0 + li
    {
        float dd = 0.f;
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const uint32_t off = (uint32_t)(t0 + li) * v.sD + 16 * k + 4 * g;
            const floatx4 xr = buf_f32x4(rx_r, off), xi = buf_f32x4(rx_i, off);
#pragma unroll
            for (int e = 0; e < 4; ++e) dd += gq_r[k][e] * xr[e] + gq_i[k][e] * xi[e];
        }
        dd = sum_groups(dd);
        if (g == 0) a.ddp[v.pbase + t0 + li] = dd;
    }

    // accumulators: register r <-> row t = t0 + 4g + r, column n = 16 nt + li
    CTile dc[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) ctile_zero(dc[k]);

    // ---- carried-state term dY H_c^H, then the row factor conj(e[t])
#pragma unroll
    for (int pk = 0; pk < PT; ++pk) {
        const floatx4 gs = gq_r[pk] + gq_i[pk];
#pragma unroll
        for (int nt = 0; nt < NK; ++nt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // conj(H[n = 16nt + li][p = 16pk + 4g + e])
                const uint32_t fi = frag_index<D>(16 * nt + li, 16 * pk + 4 * g + e);
                const float hr = buf_f32(rh_r, fi), hi = -buf_f32(rh_i, fi);
                ctile_mac(dc[nt], gq_r[pk][e], gq_i[pk][e], gs[e], hr, hi, hr + hi);
            }
        }
    }
    {
        const floatx4 er = *reinterpret_cast<const floatx4*>(f.e_re + v.pbase + t0 + 4 * g);
        const floatx4 ei = *reinterpret_cast<const floatx4*>(f.e_im + v.pbase + t0 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int k = 0; k < NK; ++k) ctile_scale(dc[k], r, er[r], -ei[r]);
    }

    // ---- causal terms over the tiles lt <= tt
#pragma unroll
    for (int lt = 0; lt < C / 16; ++lt) {
        if (lt > tt) continue;  // wave-uniform
        const int l0 = lt * 16;
        // P[t][l] as conj(X[l]) . dY[t]; register r <-> t = t0 + li, l = l0 + 4g + r
        CTile pq;
        ctile_zero(pq);
#pragma unroll
        for (int pk = 0; pk < PT; ++pk) {
            const floatx4 xr = buf_f32x4(rx_r, (uint32_t)(l0 + li) * v.sD + 16 * pk + 4 * g);
            const floatx4 xi = -buf_f32x4(rx_i, (uint32_t)(l0 + li) * v.sD + 16 * pk + 4 * g);
            const floatx4 xs = xr + xi, gs = gq_r[pk] + gq_i[pk];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ctile_mac(pq, xr[e], xi[e], xs[e], gq_r[pk][e], gq_i[pk][e], gs[e]);
        }
        float kk_r[4], kk_i[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + li, l = l0 + 4 * g + r;
            float lr = 0.f, lim = 0.f;
            if (lt < tt || t >= l) seg_exp(ar, ai, t, l, false, lr, lim);
            const float p_r = ctile_re(pq, r), p_i = ctile_im(pq, r);
            kk_r[r] = lr * p_r + lim * p_i;  // conj(L) P
            kk_i[r] = lr * p_i - lim * p_r;
        }
        // dC += K conj(B[lt]); k-step r <-> l = l0 + 4g + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t lrow = (uint32_t)(l0 + 4 * g + r);
            const float ks = kk_r[r] + kk_i[r];
#pragma unroll
            for (int nt = 0; nt < NK; ++nt) {
                const float br = buf_f32(rb_r, lrow * v.sN + 16 * nt + li);
                const float bi = -buf_f32(rb_i, lrow * v.sN + 16 * nt + li);
                ctile_mac(dc[nt], kk_r[r], kk_i[r], ks, br, bi, br + bi);
            }
        }
    }

    const BufRes rdc_r = make_buf(a.dc_re + v.row0 * N, v.extN * 4);
    const BufRes rdc_i = make_buf(a.dc_im + v.row0 * N, v.extN * 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t trow = (uint32_t)(t0 + 4 * g + r);
#pragma unroll
        for (int nt = 0; nt < NK; ++nt) {
            buf_store_f32(ctile_re(dc[nt], r), rdc_r, trow * v.sN + 16 * nt + li);
            buf_store_f32(ctile_im(dc[nt], r), rdc_i, trow * v.sN + 16 * nt + li);
        }
    }

    // ---- the dC half of q, conj(C[t]) . dC[t], for rows t = t0 + 4g + r
    const BufRes rc_r = make_buf(static_cast<const float*>(f.c_re) + v.row0 * N, v.extN * 4);
    const BufRes rc_i = make_buf(static_cast<const float*>(f.c_im) + v.row0 * N, v.extN * 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t trow = (uint32_t)(t0 + 4 * g + r);
        float pr = 0.f, pi = 0.f;
#pragma unroll
        for (int nt = 0; nt < NK; ++nt) {
            const float cr = buf_f32(rc_r, trow * v.sN + 16 * nt + li);
            const float ci = buf_f32(rc_i, trow * v.sN + 16 * nt + li);
            const float dr = ctile_re(dc[nt], r), di = ctile_im(dc[nt], r);
            pr += cr * dr + ci * di;
            pi += cr * di - ci * dr;
        }
        pr = row_total(pr);
        pi = row_total(pi);
        if (li == 15) {
            a.q2_re[v.pbase + trow] = pr;
            a.q2_im[v.pbase + trow] = pi;
        }
    }
}

// Balanced pairs of row tiles {t, NLT-1-t} per wave, 4 / WPC chunks per block.
// PART: 0 dX, 1 dB, 2 dC.  Waves per SIMD: 1 for the large states; otherwise 3
// where the live tiles (complex accumulators, 12 registers each, and resident
// operand fragments, 8 each) fit, else 2 (more waves spill there).
constexpr int bwd_waves(int C, int N, int D, int PART) {
    const int no = PART == 0 ? D / 16 : N / 16;  // accumulator tiles
    const int nq = PART == 0 ? N / 16 : D / 16;  // resident operand fragments
    return N * D > 64 * 64 ? 1 : (12 * no + 8 * nq <= 80 && C <= 64 ? 3 : 2);
}

template <int C, int N, int D, int PART>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(bwd_waves(C, N, D, PART)))) void k_bwd_tiles(BwdArgs a) {
    constexpr int NLT = C / 16;
    constexpr int WPC = NLT >= 2 ? NLT / 2 : 1;
    const int wave = wave_id();
    const int64_t chunk = (int64_t)blockIdx.x * (4 / WPC) + wave / WPC;
    if (chunk >= a.f.B * a.f.H * a.f.nC) return;  // wave-uniform
    const int t = wave % WPC;
    if constexpr (PART == 2) {
        dc_tile<C, N, D>(a, chunk, t);
        if (NLT - 1 - t != t) dc_tile<C, N, D>(a, chunk, NLT - 1 - t);
    } else {
        dxdb_tile<C, N, D, PART == 0>(a, chunk, t);
        if (NLT - 1 - t != t) dxdb_tile<C, N, D, PART == 0>(a, chunk, NLT - 1 - t);
    }
}

// ----------------------------------------------------------------------------
// Z[c] = <R_{c+1}, H_{c+1}>: the tail of the log-decay gradient sum past chunk c,
// stored as two partials per chunk (the fused adjoint scan writes one per half
// of the n rows; this kernel writes the whole term and a zero).
// R_{c+1} is slot c of the adjoint buffer, H_{c+1} slot c + 1 of the carry-in
// states (both MFMA-fragment order); for the last chunk it is <dhT, hT> (both in
// the caller's layout), or 0 without dhT.  One wave per (b, h, c), fp64 sums.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_zbound(BwdArgs a) {
    const FwdArgs& f = a.f;
    const int64_t chunk = (int64_t)blockIdx.x * 4 + wave_id();
    if (chunk >= f.B * f.H * f.nC) return;  // wave-uniform
    const int lane = threadIdx.x & 63;
    const int c = (int)(chunk % f.nC);
    const int64_t bh = chunk / f.nC;
    const int64_t ND = f.N * f.D;
    const float *ur, *ui, *vr, *vi;
    if (c + 1 < f.nC) {
        ur = a.r_re + chunk * ND;
        ui = a.r_im + chunk * ND;
        vr = f.st_re + (chunk + 1) * ND;
        vi = f.st_im + (chunk + 1) * ND;
    } else if (a.dhT_re != nullptr) {
        ur = a.dhT_re + bh * ND;
        ui = a.dhT_im + bh * ND;
        vr = a.hT_re + bh * ND;
        vi = a.hT_im + bh * ND;
    } else {
        ur = nullptr;
    }
    double zr = 0.0, zi = 0.0;
    if (ur != nullptr) {
        for (int64_t k = 4 * lane; k < ND; k += 256) {
            const float4 a4 = *reinterpret_cast<const float4*>(ur + k);
            const float4 b4 = *reinterpret_cast<const float4*>(ui + k);
            const float4 c4 = *reinterpret_cast<const float4*>(vr + k);
            const float4 d4 = *reinterpret_cast<const float4*>(vi + k);
            const float xr[4] = {a4.x, a4.y, a4.z, a4.w}, xi[4] = {b4.x, b4.y, b4.z, b4.w};
            const float yr[4] = {c4.x, c4.y, c4.z, c4.w}, yi[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                zr += (double)xr[q] * yr[q] + (double)xi[q] * yi[q];
                zi += (double)xi[q] * yr[q] - (double)xr[q] * yi[q];
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            zr += __shfl_xor(zr, off, 64);
            zi += __shfl_xor(zi, off, 64);
        }
    }
    if (lane == 0) {  // the whole term in the first of the chunk's two partials
        a.z_re[2 * chunk] = zr;
        a.z_im[2 * chunk] = zi;
        a.z_re[2 * chunk + 1] = 0.0;
        a.z_im[2 * chunk + 1] = 0.0;
    }
}

// ----------------------------------------------------------------------------
// dz_t = (suffix sum of q within chunk c) + Z[c]  ->  ddt, and partials of dA
// and dDskip.  The sum never crosses a chunk boundary, so the positions of one
// (b, h) are cut into spans of max(C, 64) whole chunks, one wave each (the
// partials of every span are kept apart and summed later in a fixed order).
// A wave walks its span from the end in blocks of 64: a chunk of 16 or 32
// positions lies inside one block (segmented suffix sum); a chunk of 128 spans
// two blocks, and its tail carries from the later block to the earlier one.
// ----------------------------------------------------------------------------
__host__ __device__ inline int64_t dz_span(int64_t C) { return C > 64 ? C : 64; }
__host__ __device__ inline int64_t dz_spans(int64_t nC, int64_t C) {
    return (nC * C + dz_span(C) - 1) / dz_span(C);
}

__global__ __launch_bounds__(256) void k_bwd_dz(BwdArgs a) {
    const FwdArgs& f = a.f;
    const int64_t C = f.C, S = dz_span(C), nsp = dz_spans(f.nC, C);
    const int64_t unit = (int64_t)blockIdx.x * 4 + wave_id();
    if (unit >= f.B * f.H * nsp) return;  // wave-uniform
    const int64_t bh = unit / nsp, sp = unit % nsp;
    const int lane = threadIdx.x & 63;
    const int h = (int)(bh % f.H);
    const int64_t b = bh / f.H;
    const double Ar = f.a_re[h], Ai = f.a_im[h];
    const int64_t pb = bh * f.nC * C;
    double gar = 0.0, gai = 0.0, gd = 0.0;
    double tail_r = 0.0, tail_i = 0.0;  // q of the current chunk in later blocks
    // the span starts and ends on chunk boundaries, and it holds at least one
    // position t < T (its first position is a chunk start before nC C)
    const int64_t blk_first = sp * S / 64;
    const int64_t blk_last = min((sp * S + S) / 64 - 1, (f.T - 1) / 64);
    for (int64_t blk = blk_last; blk >= blk_first; --blk) {
        const int64_t t = blk * 64 + lane;
        double sr = 0.0, si = 0.0;
        if (t < f.T) {
            sr = (double)a.q1_re[pb + t] + (double)a.q2_re[pb + t];
            si = (double)a.q1_im[pb + t] + (double)a.q2_im[pb + t];
            gd += (double)a.ddp[pb + t];
        }
        // inclusive suffix sum within each chunk's part of the block
        const int64_t ct = t / C;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double ur = __shfl_down(sr, off, 64), ui = __shfl_down(si, off, 64);
            if (lane + off < 64 && (t + off) / C == ct) {
                sr += ur;
                si += ui;
            }
        }
        // the chunk containing the block's last position may continue into the
        // next block (C = 128); its later positions are in tail
        const int64_t c_last = (blk * 64 + 63) / C;
        const bool straddles = (c_last + 1) * C > blk * 64 + 64;
        // (lanes past T may sit in a chunk past the last one: clamp their read)
        const int64_t cz = min(ct, (int64_t)f.nC - 1);
        const int64_t zk = 2 * (bh * f.nC + cz);
        const double cr = (ct == c_last && straddles ? tail_r : 0.0) + (a.z_re[zk] + a.z_re[zk + 1]);
        const double ci = (ct == c_last && straddles ? tail_i : 0.0) + (a.z_im[zk] + a.z_im[zk + 1]);
        if (t < f.T) {
            const double zr = sr + cr, zi = si + ci;
            const int64_t row = (b * f.T + t) * f.H + h;
            const double v = (double)f.dt[row];
            const double s = softplus_f64(v);
            a.ddt[row] = (float)((zr * Ar + zi * Ai) / (1.0 + exp(-v)));
            gar += s * zr;
            gai += s * zi;
        }
        // carry for the chunk that starts before this block: its part in this block
        const int64_t c_first = (blk * 64) / C;
        const bool starts_before = c_first * C < blk * 64;
        if (starts_before) {
            // lane 0 holds the suffix sum of chunk c_first over this whole block
            const double br = __shfl(sr, 0, 64), bi = __shfl(si, 0, 64);
            const bool same = (c_first == c_last) && straddles;
            tail_r = br + (same ? tail_r : 0.0);
            tail_i = bi + (same ? tail_i : 0.0);
        } else {
            tail_r = tail_i = 0.0;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        gar += __shfl_xor(gar, off, 64);
        gai += __shfl_xor(gai, off, 64);
        gd += __shfl_xor(gd, off, 64);
    }
    if (lane == 0) {
        a.pa[3 * unit] = gar;
        a.pa[3 * unit + 1] = gai;
        a.pa[3 * unit + 2] = gd;
    }
}

// dA[h], dDskip[h]: the per-span partials summed over b and the spans in a fixed order.
__global__ __launch_bounds__(256) void k_bwd_reduce(BwdArgs a) {
    // one wave per head: lane l sums spans l, l + 64, ... of every batch row in
    // order, then a butterfly over the 64 lanes adds the lane sums, the same order
    // on every run (one thread per head, summing all its partials in a row, took
    // 0.040 ms at B 8, T 2048, H 48: 256 dependent loads a head)
    const int64_t h = (int64_t)blockIdx.x * 4 + wave_id();
    if (h >= a.f.H) return;  // wave-uniform
    const int lane = threadIdx.x & 63;
    const int64_t nsp = dz_spans(a.f.nC, a.f.C);
    double sr = 0.0, si = 0.0, sd = 0.0;
    for (int64_t b = 0; b < a.f.B; ++b)
        for (int64_t sp = lane; sp < nsp; sp += 64) {
            const int64_t u = (b * a.f.H + h) * nsp + sp;
            sr += a.pa[3 * u];
            si += a.pa[3 * u + 1];
            sd += a.pa[3 * u + 2];
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        sr += __shfl_xor(sr, off, 64);
        si += __shfl_xor(si, off, 64);
        sd += __shfl_xor(sd, off, 64);
    }
    if (lane == 0) {
        a.da_re[h] = (float)sr;
        a.da_im[h] = (float)si;
        if (a.dd != nullptr) a.dd[h] = (float)sd;
    }
}

template <int C, int N, int PART>
static hipError_t launch_tiles_d(const BwdArgs& a, hipStream_t s) {
    constexpr int WPC = C / 16 >= 2 ? C / 32 : 1;
    constexpr int CPB = 4 / WPC;
    const int64_t nchunks = a.f.B * a.f.H * a.f.nC;
    const dim3 grid((unsigned)((nchunks + CPB - 1) / CPB)), block(256);
    switch (a.f.D) {
        case 16: hipLaunchKernelGGL((k_bwd_tiles<C, N, 16, PART>), grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((k_bwd_tiles<C, N, 32, PART>), grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL((k_bwd_tiles<C, N, 64, PART>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((k_bwd_tiles<C, N, 128, PART>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

template <int C, int PART>
static hipError_t launch_tiles_n(const BwdArgs& a, hipStream_t s) {
    switch (a.f.N) {
        case 16: return launch_tiles_d<C, 16, PART>(a, s);
        case 32: return launch_tiles_d<C, 32, PART>(a, s);
        case 64: return launch_tiles_d<C, 64, PART>(a, s);
        default: return launch_tiles_d<C, 128, PART>(a, s);
    }
}

template <int PART>
static hipError_t launch_tiles(const BwdArgs& a, hipStream_t s) {
    switch (a.f.C) {
        case 16: return launch_tiles_n<16, PART>(a, s);
        case 32: return launch_tiles_n<32, PART>(a, s);
        case 64: return launch_tiles_n<64, PART>(a, s);
        default: return launch_tiles_n<128, PART>(a, s);
    }
}

// N = D = C = 64: the chunk-staged kernels; other shapes: the tile kernels
static bool bwd_staged(const BwdArgs& a) { return a.f.C == 64 && a.f.N == 64 && a.f.D == 64; }

hipError_t launch_bwd_dx(const BwdArgs& a, hipStream_t s) {
    if (!bwd_staged(a)) return launch_tiles<0>(a, s);
    hipLaunchKernelGGL(k_bwd_lds<true>, dim3((unsigned)(a.f.B * a.f.H * a.f.nC)), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}
hipError_t launch_bwd_db(const BwdArgs& a, hipStream_t s) {
    if (!bwd_staged(a)) return launch_tiles<1>(a, s);
    hipLaunchKernelGGL(k_bwd_lds<false>, dim3((unsigned)(a.f.B * a.f.H * a.f.nC)), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}
hipError_t launch_bwd_dc(const BwdArgs& a, hipStream_t s) {
    if (!bwd_staged(a)) return launch_tiles<2>(a, s);
    hipLaunchKernelGGL(k_bwd_dc_lds, dim3((unsigned)(a.f.B * a.f.H * a.f.nC)), dim3(256), 0, s,
                       a);
    return hipGetLastError();
}

hipError_t launch_bwd_dz(const BwdArgs& a, bool with_zbound, hipStream_t s) {
    const int64_t nchunks = a.f.B * a.f.H * a.f.nC;
    hipError_t e;
    if (with_zbound) {
        hipLaunchKernelGGL(k_bwd_zbound, dim3((unsigned)((nchunks + 3) / 4)), dim3(256), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t units = a.f.B * a.f.H * dz_spans(a.f.nC, a.f.C);
    hipLaunchKernelGGL(k_bwd_dz, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_bwd_reduce, dim3((unsigned)((a.f.H + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace cssd
