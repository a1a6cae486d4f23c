// K4: the chunk-level scan that carries the state from chunk to chunk.  The
// forward computes it fused with the chunk states (k_state_scan.hip); this
// kernel serves the gradient pass in its reverse (adjoint) mode.
//
//   H_0 = h0 (or 0);   H_{c+1} = cd[c] * H_c + S_c;   hT = H_{nC}
//
// where cd[c] = exp(acs[C-1]) is the decay across chunk c and S_c its end
// state from zero.  This is the recurrence over T/C steps that the SSD
// decomposition leaves between chunks (Mamba-3-Lite docs, "SSD Theory" 4.5:
// the state entering chunk c is every earlier chunk's end state decayed across
// the chunks in between; "The Chunkwise Complex SSD Algorithm" 4.5 writes it as
// H_c = Phi_{c-1} H_{c-1} + S_{c-1}).  It is evaluated in exactly that
// sequential form: the einsum variant on the page aligns the decay one chunk
// late when chunk totals differ (its own "Pitfalls" section).
//
// The state buffer holds S_c on entry (MFMA-fragment order, see the
// chunk-state kernel) and is overwritten in place with H_c, the carry-in state
// the output kernel reads; the pass is elementwise, so it walks the buffer in
// that order.  Only h0 and hT use the caller's (B,H,N,D) layout.  Memory-bound:
// one thread owns four state elements of one (b, h) and walks the chunks,
// issuing the loads of U chunks before their dependent updates so that several
// loads are in flight per thread.
#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

// REV: the adjoint pass of the gradient computation, run from the last chunk
// back to the first:  R_nC = dhT (or 0);  R_c = Q_c + conj(cd[c]) R_{c+1}.  The
// buffer holds Q_c on entry and R_{c+1} (the gradient reaching the end of chunk
// c) on exit; the init/final pointers then carry dhT in and dh0 = R_0 out.
template <bool REV>
__global__ __launch_bounds__(256) void k_state_pass(float4* __restrict__ st_re,
                                                    float4* __restrict__ st_im,
                                                    const float* __restrict__ cd_re,
                                                    const float* __restrict__ cd_im,
                                                    const float* __restrict__ h0_re,
                                                    const float* __restrict__ h0_im,
                                                    float* __restrict__ hT_re,
                                                    float* __restrict__ hT_im, int64_t total,
                                                    int N, int D, int nC) {
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (tid >= total) return;
    const int nd4 = N * D / 4;
    const int64_t bh = tid / nd4;
    const int e = (int)(tid % nd4);
    // fragment coordinates of this float4: rows n = 16 nt + 4 g + q (q = 0..3), column p
    const int li = e & 15, g = (e >> 4) & 3, tile = e >> 6;
    const int PT = D / 16;
    const int nt = tile / PT, pt = tile % PT;
    const int64_t sbase = (bh * N + nt * 16 + 4 * g) * (int64_t)D + pt * 16 + li;

    float4 hr = make_float4(0.f, 0.f, 0.f, 0.f), hi = hr;
    if (h0_re != nullptr) {
        hr = make_float4(h0_re[sbase], h0_re[sbase + D], h0_re[sbase + 2 * D],
                         h0_re[sbase + 3 * D]);
        hi = make_float4(h0_im[sbase], h0_im[sbase + D], h0_im[sbase + 2 * D],
                         h0_im[sbase + 3 * D]);
    }
    const int64_t base = bh * (int64_t)nC * nd4 + e;
    constexpr int U = 8;
    for (int c0 = 0; c0 < nC; c0 += U) {
        float4 sr[U], si[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c0 + u < nC) {
                const int c = REV ? nC - 1 - (c0 + u) : c0 + u;
                sr[u] = nt_load4(&st_re[base + (int64_t)c * nd4]);
                si[u] = nt_load4(&st_im[base + (int64_t)c * nd4]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c0 + u < nC) {
                const int c = REV ? nC - 1 - (c0 + u) : c0 + u;
                st_re[base + (int64_t)c * nd4] = hr;
                st_im[base + (int64_t)c * nd4] = hi;
                const float dr = cd_re[bh * nC + c];
                const float di = REV ? -cd_im[bh * nC + c] : cd_im[bh * nC + c];
                float4 nr, ni;
                nr.x = dr * hr.x - di * hi.x + sr[u].x;
                nr.y = dr * hr.y - di * hi.y + sr[u].y;
                nr.z = dr * hr.z - di * hi.z + sr[u].z;
                nr.w = dr * hr.w - di * hi.w + sr[u].w;
                ni.x = dr * hi.x + di * hr.x + si[u].x;
                ni.y = dr * hi.y + di * hr.y + si[u].y;
                ni.z = dr * hi.z + di * hr.z + si[u].z;
                ni.w = dr * hi.w + di * hr.w + si[u].w;
                hr = nr;
                hi = ni;
            }
        }
    }
    if (hT_re != nullptr) {
        hT_re[sbase] = hr.x; hT_re[sbase + D] = hr.y;
        hT_re[sbase + 2 * D] = hr.z; hT_re[sbase + 3 * D] = hr.w;
        hT_im[sbase] = hi.x; hT_im[sbase + D] = hi.y;
        hT_im[sbase + 2 * D] = hi.z; hT_im[sbase + 3 * D] = hi.w;
    }
}

hipError_t launch_state_pass_adjoint(const FwdArgs& a, float* q_re, float* q_im,
                                     const float* dhT_re, const float* dhT_im, float* dh0_re,
                                     float* dh0_im, hipStream_t stream) {
    const int64_t total = a.B * a.H * (a.N * a.D / 4);
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    hipLaunchKernelGGL(k_state_pass<true>, grid, block, 0, stream, reinterpret_cast<float4*>(q_re),
                       reinterpret_cast<float4*>(q_im), a.cd_re, a.cd_im, dhT_re, dhT_im, dh0_re,
                       dh0_im, total, (int)a.N, (int)a.D, (int)a.nC);
    return hipGetLastError();
}

}  // namespace cssd
