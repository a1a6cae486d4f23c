// K3: per-chunk end states, as a complex GEMM on the fp32 matrix cores.
//
//   S_c[n, p] = sum_l  B[l, n] * w[l] * X[l, p],   w[l] = exp(acs[C-1] - acs[l])
//
// i.e. S_c = (diag(w) B)^T X, the state a chunk would leave behind if it
// started from zero (Mamba-3-Lite docs, "SSD Theory" 4.5, and "The Chunkwise
// Complex SSD Algorithm" 4.5, first einsum).  Padded positions contribute
// nothing.
//
// Mapping: one workgroup per chunk, one wave per 16-row tile of n; each wave
// owns all D/16 column tiles of p.  The contraction index is time l: step j of
// the 16x16x4 MFMA contracts l = 4j + g, where g = lane/16.  A complex product
// is four real MFMAs (re*re - im*im, re*im + im*re); the weight w is folded into
// B on the vector ALU before the MFMA.  Both operands are read with lane%16
// running along the contiguous axis (n for B, p for X), so every load of a
// 16-lane group is one contiguous 64-byte row segment.
#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

template <typename In, int N, int D>
__global__ __launch_bounds__(4 * N) void k_chunk_state(
    const typename In::T* __restrict__ x_re, const typename In::T* __restrict__ x_im,
    const typename In::T* __restrict__ b_re, const typename In::T* __restrict__ b_im,
    const float* __restrict__ w_re, const float* __restrict__ w_im, float* __restrict__ st_re,
    float* __restrict__ st_im, int64_t T, int H, int nC, int C) {
    constexpr int PT = D / 16;  // column tiles (p)
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int nt = threadIdx.x >> 6;  // n tile of this wave
    const int64_t chunk = blockIdx.x;
    const int c = (int)(chunk % nC);
    const int64_t bh = chunk / nC;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int64_t t0 = (int64_t)c * C;
    const int valid = (int)min<int64_t>((int64_t)C, T - t0);

    // row (b, t0, h) bases; consecutive time steps are H*N (H*D) elements apart
    const int64_t rowB = ((b * T + t0) * H + h) * (int64_t)N + nt * 16 + li;
    const int64_t rowX = ((b * T + t0) * H + h) * (int64_t)D + li;
    const int64_t strideB = (int64_t)H * N, strideX = (int64_t)H * D;
    const int64_t wbase = bh * (int64_t)nC * C + t0;

    floatx4 sr[PT], si[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
        sr[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
        si[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

#pragma unroll 4
    for (int j = 0; j < C / 4; ++j) {
        const int l = 4 * j + g;
        const bool ok = l < valid;
        const int lc = ok ? l : valid - 1;  // clamped row: always in bounds
        const float br = ok ? In::load1(b_re + rowB + lc * strideB) : 0.f;
        const float bi = ok ? In::load1(b_im + rowB + lc * strideB) : 0.f;
        const float wr = w_re[wbase + l], wi = w_im[wbase + l];
        const float pr = wr * br - wi * bi;  // (w B)[l, n]
        const float pi = wr * bi + wi * br;
        const float npi = -pi;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const float xr = ok ? In::load1(x_re + rowX + lc * strideX + pt * 16) : 0.f;
            const float xi = ok ? In::load1(x_im + rowX + lc * strideX + pt * 16) : 0.f;
            sr[pt] = mfma4(pr, xr, sr[pt]);
            sr[pt] = mfma4(npi, xi, sr[pt]);
            si[pt] = mfma4(pr, xi, si[pt]);
            si[pt] = mfma4(pi, xr, si[pt]);
        }
    }

    // accumulator register r of lane (li + 16 g) is S[n = nt*16 + 4g + r][p = pt*16 + li]
    const int64_t sbase = (bh * nC + c) * (int64_t)N * D;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t off = sbase + (int64_t)(nt * 16 + 4 * g + r) * D + pt * 16 + li;
            st_re[off] = sr[pt][r];
            st_im[off] = si[pt][r];
        }
    }
}

template <typename In, int N>
static void dispatch_d(const FwdArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.B * a.H * a.nC)), block(4 * N);
    const auto* xr = static_cast<const typename In::T*>(a.x_re);
    const auto* xi = static_cast<const typename In::T*>(a.x_im);
    const auto* br = static_cast<const typename In::T*>(a.b_re);
    const auto* bi = static_cast<const typename In::T*>(a.b_im);
#define CSSD_K3(DD)                                                                            \
    hipLaunchKernelGGL((k_chunk_state<In, N, DD>), grid, block, 0, s, xr, xi, br, bi, a.w_re,  \
                       a.w_im, a.st_re, a.st_im, a.T, (int)a.H, (int)a.nC, (int)a.C)
    switch (a.D) {
        case 16: CSSD_K3(16); break;
        case 32: CSSD_K3(32); break;
        case 64: CSSD_K3(64); break;
        default: CSSD_K3(128); break;
    }
#undef CSSD_K3
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

hipError_t launch_chunk_state(const FwdArgs& a, hipStream_t stream) {
    if (a.in_dtype == 1)
        dispatch_n<InBF16>(a, stream);
    else
        dispatch_n<InF32>(a, stream);
    return hipGetLastError();
}

}  // namespace cssd
