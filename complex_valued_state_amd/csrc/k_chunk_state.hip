// K3: per-chunk end states, as a complex GEMM on the fp32 matrix cores.
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
// their contiguous axis (one 64-byte row segment per 16-lane group), and the
// operands of the next DIST k-steps are loaded into a register ring before the
// current step's MFMAs are issued, so memory latency overlaps the matrix work.
// A complex product is four real MFMAs; w is folded into B on the vector ALU.
//
// S_c is written in MFMA-fragment order: within the N x D block of one
// (b, h, c), element (n, p) sits at
//   (((n/16) * (D/16) + p/16) * 4 + (n%16)/4) * 64 + (p%16) * 4 + n%4
// so each accumulator tile is one contiguous 1 KB float4 store, and the output
// kernel later reads the carry-in states back the same way.
#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

template <typename In, int C, int D>
__global__ __launch_bounds__(512) void k_chunk_state(
    const typename In::T* __restrict__ x_re, const typename In::T* __restrict__ x_im,
    const typename In::T* __restrict__ b_re, const typename In::T* __restrict__ b_im,
    const float* __restrict__ w_re, const float* __restrict__ w_im, float* __restrict__ st_re,
    float* __restrict__ st_im, int64_t T, int H, int N, int nC) {
    constexpr int KJ = C / 4;   // MFMA k-steps per chunk
    constexpr int PT = D / 16;  // column tiles (p)
    // operands of DIST future k-steps are kept in flight (register ring)
#ifndef CSSD_K3_DIST
#define CSSD_K3_DIST 4
#endif
    constexpr int DW = PT <= 4 ? CSSD_K3_DIST : CSSD_K3_DIST / 2;
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

    // wave-uniform bases; consecutive time steps are H*N (H*D) elements apart
    const int64_t row0 = (b * T + t0) * H + h;
    const typename In::T* __restrict__ bb_r = b_re + row0 * N + nt * 16 + li;
    const typename In::T* __restrict__ bb_i = b_im + row0 * N + nt * 16 + li;
    const typename In::T* __restrict__ xb_r = x_re + row0 * D + li;
    const typename In::T* __restrict__ xb_i = x_im + row0 * D + li;
    const uint32_t sN = (uint32_t)H * N, sD = (uint32_t)H * D;

    struct Ops {
        float br, bi, xr[PT], xi[PT];
    };
    // rows past the end of a partial chunk are clamped (in bounds) and zeroed later
    auto load = [&](int j, Ops& o) {
        const int l = KJ * g + j;
        const uint32_t lc = (uint32_t)(l < valid ? l : valid - 1);
        o.br = In::load1(bb_r + lc * sN);
        o.bi = In::load1(bb_i + lc * sN);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            o.xr[pt] = In::load1(xb_r + lc * sD + pt * 16);
            o.xi[pt] = In::load1(xb_i + lc * sD + pt * 16);
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

    floatx4 sr[PT], si[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
        sr[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
        si[pt] = sr[pt];
    }

#pragma unroll
    for (int j = 0; j < KJ; ++j) {
        Ops o = ring[j % DIST];
        if (j + DIST < KJ) load(j + DIST, ring[j % DIST]);
        __builtin_amdgcn_sched_barrier(0);
        const bool ok = KJ * g + j < valid;
        const float br = ok ? o.br : 0.f, bi = ok ? o.bi : 0.f;
        const float pr = wr[j] * br - wi[j] * bi;  // (w B)[l, n]
        const float pi = wr[j] * bi + wi[j] * br;
        const float npi = -pi;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const float xr = ok ? o.xr[pt] : 0.f, xi = ok ? o.xi[pt] : 0.f;
            sr[pt] = mfma4(pr, xr, sr[pt]);
            sr[pt] = mfma4(npi, xi, sr[pt]);
            si[pt] = mfma4(pr, xi, si[pt]);
            si[pt] = mfma4(pi, xr, si[pt]);
        }
    }

    // accumulator tile (nt, pt) -> 256 contiguous floats, lane-major
    const int64_t blk = (bh * nC + c) * (int64_t)N * D + 4 * lane;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
        const int64_t off = blk + (int64_t)(nt * PT + pt) * 256;
        *reinterpret_cast<floatx4*>(st_re + off) = sr[pt];
        *reinterpret_cast<floatx4*>(st_im + off) = si[pt];
    }
}

template <typename In, int C>
static void launch_d(const FwdArgs& a, hipStream_t s) {
    const auto* xr = static_cast<const typename In::T*>(a.x_re);
    const auto* xi = static_cast<const typename In::T*>(a.x_im);
    const auto* br = static_cast<const typename In::T*>(a.b_re);
    const auto* bi = static_cast<const typename In::T*>(a.b_im);
    const dim3 grid((unsigned)(a.B * a.H * a.nC)), block((unsigned)(4 * a.N));
#define CSSD_K3(DD)                                                                            \
    hipLaunchKernelGGL((k_chunk_state<In, C, DD>), grid, block, 0, s, xr, xi, br, bi, a.w_re,  \
                       a.w_im, a.st_re, a.st_im, a.T, (int)a.H, (int)a.N, (int)a.nC)
    switch (a.D) {
        case 16: CSSD_K3(16); break;
        case 32: CSSD_K3(32); break;
        case 64: CSSD_K3(64); break;
        default: CSSD_K3(128); break;
    }
#undef CSSD_K3
}

template <typename In>
static void launch_c(const FwdArgs& a, hipStream_t s) {
    switch (a.C) {
        case 16: launch_d<In, 16>(a, s); break;
        case 32: launch_d<In, 32>(a, s); break;
        case 64: launch_d<In, 64>(a, s); break;
        default: launch_d<In, 128>(a, s); break;
    }
}

hipError_t launch_chunk_state(const FwdArgs& a, hipStream_t stream) {
    if (a.in_dtype == 1)
        launch_c<InBF16>(a, stream);
    else
        launch_c<InF32>(a, stream);
    return hipGetLastError();
}

}  // namespace cssd
