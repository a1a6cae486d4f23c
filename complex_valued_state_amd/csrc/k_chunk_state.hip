// K3: per-chunk end states, as a complex GEMM on the fp32 matrix cores.  The
// forward computes them fused with the chunk-to-chunk pass (k_state_scan.hip);
// this kernel serves the gradient pass, in its conjugate-weight mode.
//
//   S_c[n, p] = sum_l  w[l] B[l, n] X[l, p],   w[l] = exp(acs[C-1] - acs[l])
//
// i.e. S_c = (diag(w) B)^T X, the state chunk c would leave behind if it
// started from zero (Mamba-3-Lite docs, "SSD Theory" 4.5, and "The Chunkwise
// Complex SSD Algorithm" 4.5, the per-chunk states einsum).  Padded positions
// of a partial last chunk contribute nothing.
//
// Mapping: one workgroup per chunk, one wave per 16-row tile nt of n; each wave
// owns all D/16 column tiles of p (accumulators).  Step j of the 16x16x4 MFMA
// contracts time l = (C/4) g + j (g = lane/16), so each lane's C/4 weights w are
// contiguous and load as float4; B and X operands are read with lane%16 along
// their contiguous axis (one 64-byte row segment per 16-lane group), through
// raw buffer descriptors whose extent ends at the chunk's last real row (padded
// rows read as zero, no masks); the operands of the next DIST k-steps are loaded
// into a register ring before the current step's MFMAs are issued, so memory
// latency overlaps the matrix work.  w is folded into B on the vector ALU.  A
// complex product is three real MFMAs (Gauss: ar br, ai bi, (ar + ai)(br + bi)).
//
// S_c is written in MFMA-fragment order: within the N x D block of one
// (b, h, c), element (n, p) sits at
//   (((n/16) * (D/16) + p/16) * 4 + (n%16)/4) * 64 + (p%16) * 4 + n%4
// so each accumulator tile is one contiguous 1 KB float4 store, and the output
// kernel later reads the carry-in states back the same way.
#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

// CONJW: conjugate the weighted rows, S_c = (diag(w) B)^H X.  The gradient pass
// uses it for the adjoint chunk states Q_c = C^H diag(conj(e)) dY.
template <typename In, int C, int D, bool CONJW = false>
__global__ __launch_bounds__(512) void k_chunk_state(
    const typename In::T* __restrict__ x_re, const typename In::T* __restrict__ x_im,
    const typename In::T* __restrict__ b_re, const typename In::T* __restrict__ b_im,
    const float* __restrict__ w_re, const float* __restrict__ w_im, float* __restrict__ st_re,
    float* __restrict__ st_im, int64_t T, int H, int N, int nC) {
    typedef typename In::T TI;
    constexpr int KJ = C / 4;   // MFMA k-steps per chunk
    constexpr int PT = D / 16;  // column tiles (p)
    // operands of DIST future k-steps are kept in flight (register ring)
    constexpr int DW = PT <= 4 ? 4 : 2;
    constexpr int DIST = DW < KJ ? DW : KJ;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int nt = wave_id();  // n tile of this wave
    const int64_t chunk = blockIdx.x;
    const int c = (int)(chunk % nC);
    const int64_t bh = chunk / nC;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int64_t t0 = (int64_t)c * C;
    const int valid = (int)min<int64_t>((int64_t)C, T - t0);

    // per-chunk buffer views whose extent ends at the last real row: rows of a
    // partial chunk past it read as zero.  Consecutive time steps are H*N (H*D)
    // elements apart.
    const int64_t row0 = (b * T + t0) * H + h;
    const uint32_t sN = (uint32_t)H * N, sD = (uint32_t)H * D;
    const uint32_t extN = (uint32_t)(valid - 1) * sN + N, extD = (uint32_t)(valid - 1) * sD + D;
    const BufRes rb_r = make_buf(b_re + row0 * N, extN * sizeof(TI));
    const BufRes rb_i = make_buf(b_im + row0 * N, extN * sizeof(TI));
    const BufRes rx_r = make_buf(x_re + row0 * D, extD * sizeof(TI));
    const BufRes rx_i = make_buf(x_im + row0 * D, extD * sizeof(TI));

    struct Ops {
        float br, bi, xr[PT], xi[PT];
    };
    auto load = [&](int j, Ops& o) {
        const uint32_t l = (uint32_t)(KJ * g + j);
        o.br = In::bload1(rb_r, l * sN + nt * 16 + li);
        o.bi = In::bload1(rb_i, l * sN + nt * 16 + li);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            o.xr[pt] = In::bload1(rx_r, l * sD + pt * 16 + li);
            o.xi[pt] = In::bload1(rx_i, l * sD + pt * 16 + li);
        }
    };

    Ops ring[DIST];
#pragma unroll
    for (int j = 0; j < DIST; ++j) load(j, ring[j]);

    float wr[KJ], wi[KJ];
    {
        const float* wpr = w_re + bh * (int64_t)nC * C + t0 + KJ * g;
        const float* wpi = w_im + bh * (int64_t)nC * C + t0 + KJ * g;
#pragma unroll
        for (int j = 0; j < KJ; j += 4) {
            const float4 a = *reinterpret_cast<const float4*>(wpr + j);
            const float4 e = *reinterpret_cast<const float4*>(wpi + j);
            wr[j] = a.x; wr[j + 1] = a.y; wr[j + 2] = a.z; wr[j + 3] = a.w;
            wi[j] = e.x; wi[j + 1] = e.y; wi[j + 2] = e.z; wi[j + 3] = e.w;
        }
    }

    CTile acc[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) ctile_zero(acc[pt]);

#pragma unroll
    for (int j = 0; j < KJ; ++j) {
        Ops o = ring[j % DIST];
        if (j + DIST < KJ) load(j + DIST, ring[j % DIST]);
        __builtin_amdgcn_sched_barrier(0);
        const float pr = wr[j] * o.br - wi[j] * o.bi;  // (w B)[l, n], or its conjugate
        const float pi = CONJW ? -(wr[j] * o.bi + wi[j] * o.br) : wr[j] * o.bi + wi[j] * o.br;
        const float ps = pr + pi;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
            ctile_mac(acc[pt], pr, pi, ps, o.xr[pt], o.xi[pt], o.xr[pt] + o.xi[pt]);
    }

    // accumulator tile (nt, pt) -> 256 contiguous floats, lane-major
    const int64_t blk = (bh * nC + c) * (int64_t)N * D + 4 * lane;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
        const int64_t off = blk + (int64_t)(nt * PT + pt) * 256;
        floatx4 vr, vi;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            vr[r] = ctile_re(acc[pt], r);
            vi[r] = ctile_im(acc[pt], r);
        }
        *reinterpret_cast<floatx4*>(st_re + off) = vr;
        *reinterpret_cast<floatx4*>(st_im + off) = vi;
    }
}

// Adjoint chunk states for the gradient pass (fp32 planes):
//   Q_c[n, p] = sum_l conj(e[l] C[l, n]) dY[l, p]
// the same contraction as S_c with B -> C, w -> e (conjugated) and X -> dY.
template <int C>
static void launch_adjoint_d(const FwdArgs& a, const float* dy_re, const float* dy_im,
                             float* q_re, float* q_im, hipStream_t s) {
    const float* cr = static_cast<const float*>(a.c_re);
    const float* ci = static_cast<const float*>(a.c_im);
#define CSSD_K3A(DD)                                                                           \
    {                                                                                          \
        const dim3 grid((unsigned)(a.B * a.H * a.nC)), block((unsigned)(4 * a.N));             \
        hipLaunchKernelGGL((k_chunk_state<InF32, C, DD, true>), grid, block, 0, s, dy_re, dy_im, \
                           cr, ci, a.e_re, a.e_im, q_re, q_im, a.T, (int)a.H, (int)a.N,        \
                           (int)a.nC);                                                         \
    }
    switch (a.D) {
        case 16: CSSD_K3A(16); break;
        case 32: CSSD_K3A(32); break;
        case 64: CSSD_K3A(64); break;
        default: CSSD_K3A(128); break;
    }
#undef CSSD_K3A
}

hipError_t launch_chunk_state_adjoint(const FwdArgs& a, const float* dy_re, const float* dy_im,
                                      float* q_re, float* q_im, hipStream_t stream) {
    switch (a.C) {
        case 16: launch_adjoint_d<16>(a, dy_re, dy_im, q_re, q_im, stream); break;
        case 32: launch_adjoint_d<32>(a, dy_re, dy_im, q_re, q_im, stream); break;
        case 64: launch_adjoint_d<64>(a, dy_re, dy_im, q_re, q_im, stream); break;
        default: launch_adjoint_d<128>(a, dy_re, dy_im, q_re, q_im, stream); break;
    }
    return hipGetLastError();
}

}  // namespace cssd
