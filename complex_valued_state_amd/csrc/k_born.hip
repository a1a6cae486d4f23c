// Causal Born attention of the phase-state paper ("Complex Phase-State Dynamics
// Reduce the Optimization Steps of Sequence Models", section 5.5, eq. 5, and
// Appendix A, Algorithm 3), per (batch, head):
//   s_ij  = |<q_i|k_j>|^2 / (D tau_i)  for j <= i,   <q|k> = sum_d conj(q_d) k_d
//   psi_i = (sum_{j<=i} s_ij v_j) / (sum_{j<=i} s_ij)
// in one pass over the key blocks with fp32 accumulation on the matrix cores.
//
// Both contractions are dense, so both run on v_mfma_f32_16x16x4_f32:
//  * the overlap, as real products over the 2D features [re | im]: with
//    q~ = q / sqrt(D tau) (which folds the page's 1/(D tau) into the query),
//      Re <q~|k> = [kr | ki] . [qr | qi],   Im <q~|k> = -[ki | kr] . [-qr | qi],
//    so the imaginary part reuses the real part's key registers, halves swapped;
//  * the weighted sum, S . [vr | vi], with the row sums of S formed alongside.
// Each wave computes the transposed score tile (keys x queries): the matrix
// core leaves key 4g + r of query q in register r of lane q + 16g, which is
// exactly the A-operand layout of S . V for a key order permuted within each
// 16-key tile, so the scores never leave registers.
//
// Work decomposition.  A workgroup (4 waves, 16 query rows each) takes the
// query blocks p and nqb - 1 - p of one (batch, head), so every workgroup
// visits nqb + 1 key blocks.  All workgroups of one (batch, head), and of the
// heads that share a 128-byte line of q/k/v, are sent to the same XCD
// (workgroups are dispatched round-robin over the 8 XCDs), so their key/value
// re-reads hit that XCD's L2.  Key and value blocks (64 rows, both planes) are
// staged through LDS, double-buffered, with a padded row stride (D + 4 floats)
// that keeps the operand reads free of bank conflicts.
#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

namespace {

constexpr int kBornBlock = 64;  // query rows per block = key rows per block
constexpr int kXcds = 8;

__device__ __forceinline__ float4 ld4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}

__device__ __forceinline__ float pick4(const float4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Work item of workgroup `wg`: (bh, pair p), or false when the slot is empty.
__device__ __forceinline__ bool born_item(const BornArgs& a, int64_t wg, int64_t& bh, int64_t& p) {
    const int64_t x = wg % kXcds, y = wg / kXcds;
    const int64_t per_group = a.hpl * a.npair;  // items of one line group
    const int64_t m = y / per_group, within = y % per_group;
    const int64_t lg = x + kXcds * m;
    bh = lg * a.hpl + within / a.npair;
    p = within % a.npair;
    return bh < a.B * a.H;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void k_born(BornArgs a) {
    constexpr int Q4 = D / 4;         // features of one plane per lane group
    constexpr int NS = D / 2;         // MFMA k-steps over the 2D features
    constexpr int LS = D + 4;         // LDS row stride (floats)
    constexpr int PL = kBornBlock * LS;
    constexpr int NCT = 2 * D / 16;   // 16-column tiles of [vr | vi]
    constexpr int NLD = D / 4;        // float4 staging loads per thread per block
    __shared__ __align__(16) float lds[2][4][PL];  // [buffer][kr, ki, vr, vi][row * LS + d]

    int64_t bh, pair;
    if (!born_item(a, blockIdx.x, bh, pair)) return;  // workgroup-uniform
    const int64_t b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int64_t rs = a.H * D;  // stride between consecutive time steps
    const float* planes[4] = {a.k_re, a.k_im, a.v_re, a.v_im};
    const int64_t base = (b * a.T * a.H + h) * D;  // (b, t = 0, h)

    const int nblk = pair == a.nqb - 1 - pair ? 1 : 2;  // the middle block of an odd count
    for (int which = 0; which < nblk; ++which) {
        const int64_t qb = which == 0 ? pair : a.nqb - 1 - pair;
        // this lane's query row (as the B operand) and its scaled features
        const int64_t qrow = qb * kBornBlock + 16 * w + lr;
        float bre[NS], bim[NS];
        {
            float4 qr[Q4 / 4], qi[Q4 / 4];
            float scale = 0.f;
            if (qrow < a.T) {
                const int64_t o = base + qrow * rs + lg * Q4;
#pragma unroll
                for (int c = 0; c < Q4 / 4; ++c) {
                    qr[c] = ld4(a.q_re + o + 4 * c);
                    qi[c] = ld4(a.q_im + o + 4 * c);
                }
                const float tq = a.tau != nullptr ? a.tau[(b * a.T + qrow) * a.H + h] : 1.f;
                scale = rsqrtf((float)D * tq);
            } else {
#pragma unroll
                for (int c = 0; c < Q4 / 4; ++c) qr[c] = qi[c] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int s = 0; s < Q4; ++s) {
                const float r = pick4(qr[s / 4], s % 4) * scale;
                const float i = pick4(qi[s / 4], s % 4) * scale;
                bre[s] = r;
                bre[s + Q4] = i;
                bim[s] = -r;
                bim[s + Q4] = i;
            }
        }
        floatx4 o[NCT];
#pragma unroll
        for (int c = 0; c < NCT; ++c) o[c] = floatx4{0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;

        // staging: a block is 4 planes x 64 rows x D/4 float4s; plane pl takes the
        // D/16 consecutive loads i = pl * D/16 ... of every thread
        float4 stage[NLD];
        auto fetch = [&](int64_t kb) {
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int pl = i / (D / 16), rem = (i % (D / 16)) * 256 + tid;
                const int row = rem / Q4, c4 = rem % Q4;
                const int64_t key = kb * kBornBlock + row;
                stage[i] = key < a.T ? ld4(planes[pl] + base + key * rs + 4 * c4)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        };
        auto commit = [&](int buf) {
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int pl = i / (D / 16), rem = (i % (D / 16)) * 256 + tid;
                const int row = rem / Q4, c4 = rem % Q4;
                *reinterpret_cast<float4*>(&lds[buf][pl][row * LS + 4 * c4]) = stage[i];
            }
        };

        fetch(0);
        __syncthreads();  // the previous query block's readers are done with both buffers
        commit(0);
        __syncthreads();
        for (int64_t kb = 0; kb <= qb; ++kb) {
            const int buf = kb & 1;
            if (kb < qb) fetch(kb + 1);
            const bool diag = kb == qb;
            const int ntile = diag ? w + 1 : 4;  // key tiles past this wave's rows are all masked
            for (int t = 0; t < ntile; ++t) {
                // A operand: key row 16t + lr, features of lane group lg
                const float* kr = &lds[buf][0][(16 * t + lr) * LS + lg * Q4];
                const float* ki = &lds[buf][1][(16 * t + lr) * LS + lg * Q4];
                float are[NS];
#pragma unroll
                for (int c = 0; c < Q4 / 4; ++c) {
                    const float4 x = ld4(kr + 4 * c), y = ld4(ki + 4 * c);
                    are[4 * c + 0] = x.x; are[4 * c + 1] = x.y; are[4 * c + 2] = x.z; are[4 * c + 3] = x.w;
                    are[Q4 + 4 * c + 0] = y.x; are[Q4 + 4 * c + 1] = y.y;
                    are[Q4 + 4 * c + 2] = y.z; are[Q4 + 4 * c + 3] = y.w;
                }
                floatx4 sre = {0.f, 0.f, 0.f, 0.f}, sim = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    sre = __builtin_amdgcn_mfma_f32_16x16x4f32(are[s], bre[s], sre, 0, 0, 0);
                    sim = __builtin_amdgcn_mfma_f32_16x16x4f32(are[(s + Q4) % NS], bim[s], sim, 0, 0, 0);
                }
                // scores of query lr, keys 16t + 4lg + r
                float sc[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = sre[r] * sre[r] + sim[r] * sim[r];
                    if (diag && 16 * t + 4 * lg + r > 16 * w + lr) v = 0.f;
                    sc[r] = v;
                    lsum += v;
                }
                // O += S . [vr | vi]: k-step r takes keys 16t + 4g + r
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int vrow = 16 * t + 4 * lg + r;
#pragma unroll
                    for (int c = 0; c < NCT; ++c) {
                        const int pl = 2 + (16 * c) / D, col = (16 * c) % D + lr;
                        const float bv = lds[buf][pl][vrow * LS + col];
                        o[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(sc[r], bv, o[c], 0, 0, 0);
                    }
                }
            }
            if (kb < qb) commit(buf ^ 1);
            __syncthreads();
        }
        // row sums: lanes lr, lr + 16, lr + 32, lr + 48 hold parts of query lr
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        // lane lr + 16g holds rows 4g + r of every column tile
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int qloc = 4 * lg + r;
            const float den = __shfl(lsum, qloc);
            const int64_t row = qb * kBornBlock + 16 * w + qloc;
            if (row >= a.T) continue;
            const float inv = den != 0.f ? 1.f / den : 0.f;
            const int64_t at = base + row * rs;
#pragma unroll
            for (int c = 0; c < NCT; ++c) {
                float* dst = (16 * c) < D ? a.out_re : a.out_im;
                dst[at + (16 * c) % D + lr] = o[c][r] * inv;
            }
        }
    }
}

hipError_t launch_born(const BornArgs& a, hipStream_t s) {
    const int64_t groups = (a.B * a.H + a.hpl - 1) / a.hpl;
    const int64_t per_xcd = (groups + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(kXcds * per_xcd * a.hpl * a.npair)), block(256);
    switch (a.D) {
        case 16: hipLaunchKernelGGL(k_born<16>, grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL(k_born<32>, grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL(k_born<64>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cssd
