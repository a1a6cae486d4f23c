// Causal Born attention of the phase-state paper ("Complex Phase-State Dynamics
// Reduce the Optimization Steps of Sequence Models", section 5.5, eq. 5, and
// Appendix A, Algorithm 3), per (batch, head):
//   s_ij  = |<q_i|k_j>|^2 / (D tau_i)  for j <= i,   <q|k> = sum_d conj(q_d) k_d
//   psi_i = (sum_{j<=i} s_ij v_j) / (sum_{j<=i} s_ij)
// in one pass over the key blocks with fp32 accumulation on the matrix cores.
//
// Both contractions are dense, so both run on v_mfma_f32_16x16x4_f32:
//  * the overlap in Gauss form, three real products over the D features: with
//    q~ = q / sqrt(D tau) (which folds the page's 1/(D tau) into the query),
//      P1 = kr . qr,  P2 = ki . qi,  P3 = (kr - ki) . (qr + qi),
//      Re <q~|k> = P1 + P2,   -Im <q~|k> = P3 - P1 + P2,
//    three quarters of the matrix work of the four products (kr - ki is formed
//    from the staged key operands, qr + qi once per query block);
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
        // B operands: the scaled query features [qr | qi] and the sums qr + qi
        float bre[NS], bsum[Q4];
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
                bsum[s] = r + i;
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
                // the overlap in Gauss form, three products over the D features:
                // P1 = kr . qr, P2 = ki . qi, P3 = (kr - ki) . (qr + qi); then
                // Re = P1 + P2 and P3 - P1 + P2 = -Im (the sign drops out of |.|^2)
                floatx4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = {0.f, 0.f, 0.f, 0.f};
                floatx4 p3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < Q4; ++s) {
                    p1 = __builtin_amdgcn_mfma_f32_16x16x4f32(are[s], bre[s], p1, 0, 0, 0);
                    p2 = __builtin_amdgcn_mfma_f32_16x16x4f32(are[Q4 + s], bre[Q4 + s], p2, 0, 0, 0);
                    p3 = __builtin_amdgcn_mfma_f32_16x16x4f32(are[s] - are[Q4 + s], bsum[s], p3, 0, 0, 0);
                }
                // scores of query lr, keys 16t + 4lg + r
                float sc[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float re = p1[r] + p2[r], im = p3[r] - p1[r] + p2[r];
                    float v = re * re + im * im;
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

// ----------------------------------------------------------------------------
// bf16 inputs (the page trains this attention in half precision with fp32
// accumulation): the same decomposition on v_mfma_f32_16x16x32_bf16, which
// takes A[i][k] from lane i + 16 (k / 8), slot k % 8, B[k][j] from lane
// j + 16 (k / 8), slot k % 8, and leaves D[4g + r][j] in register r of lane
// j + 16g.
//  * Overlap: MFMA step m covers features d in [16m, 16m + 16); lane group g
//    holds d in [16m + 4g, 16m + 4g + 4) of the real plane in slots 0-3 and of
//    the imaginary plane in slots 4-7.  Key rows sit in LDS in exactly that
//    order (real quad, imaginary quad, next quad ...), and a second time with
//    each pair of quads swapped, so one 16-byte read is the A operand of the
//    real part and one more that of the imaginary part.
//  * Weighted sum: the 32-key step s pairs key tiles 2s and 2s + 1: slot j < 4
//    is key 32s + 4g + j, slot j >= 4 is key 32s + 16 + 4g + j - 4, which is
//    where the score tiles leave them, so the scores are packed to bf16 in
//    place.  Values sit in LDS as rows ([key][vr | vi]) and reach the B operand
//    through two transposing LDS reads (ds_read_b64_tr_b16: within each group of
//    16 lanes, lane 4q + x receives element x of the 8-byte pieces that lanes q,
//    4 + q, 8 + q and 12 + q point at).  The normaliser sums the rounded weights (one more
//    product, against a column of ones), so the output is an exact convex
//    combination of the values with those weights.
// ----------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ bf16x4 bf4_of_bits(uint2 v) { return __builtin_bit_cast(bf16x4, v); }
__device__ __forceinline__ float bf_to_f(__bf16 v) {
    return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, v) << 16);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

}  // namespace

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// SMALL: every row a workgroup addresses (up to the end of the last 128-row query
// block, past T) lies within 2 GB of its (b, h)'s first row, so loads and stores go
// through buffer views with 32-bit offsets (the launcher checks it)
template <int D, bool SMALL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 16 ? 3 : 1))) void k_born_bf16(
    BornArgs a) {
    constexpr int NM = D / 16;          // MFMA steps over the features (per part)
    // LDS key row stride (bytes): D/4 quads of 16 B, padded.  At D = 16 a read takes
    // 16 rows at 4 quads; with 96-byte rows the bank-conflict counter reads none for
    // it, with 80-byte rows 4 cycles an instruction (measured in isolation)
    constexpr int KS = D == 16 ? 96 : 4 * D + 16;
    // LDS value row stride (bytes): [vr | vi] of one key, padded by 32 B so that the
    // four rows one transposing read takes (32 B each) fall in distinct banks
    constexpr int VS = 4 * D + 32;
    constexpr int NCT = 2 * D / 16;     // 16-column tiles of [vr | vi]
    constexpr int KQ = kBornBlock * D / 4 / 256;   // key quads staged per thread
    constexpr int VQ = kBornBlock * 2 * D / 8 / 256;  // 8-value chunks of V staged per thread
    // key blocks in flight in registers: a block's work shrinks with D, so small D
    // needs more of them to cover the global-load latency
    constexpr int RD = D == 16 ? 2 : 1;
    // key rows twice: quads [re, im] (A of the real part) and [im, re] (A of the imaginary part)
    __shared__ __align__(16) unsigned char lds_k[2][2][kBornBlock * KS];
    __shared__ __align__(16) unsigned char lds_v[2][kBornBlock * VS];

    int64_t bh, pair;
    if (!born_item(a, blockIdx.x, bh, pair)) return;  // workgroup-uniform
    const int64_t b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int64_t rs = a.H * D;
    const int64_t base = (b * a.T * a.H + h) * D;
    const uint16_t* qr_p = reinterpret_cast<const uint16_t*>(a.q_re);
    const uint16_t* qi_p = reinterpret_cast<const uint16_t*>(a.q_im);
    const uint16_t* kr_p = reinterpret_cast<const uint16_t*>(a.k_re);
    const uint16_t* ki_p = reinterpret_cast<const uint16_t*>(a.k_im);
    const uint16_t* vr_p = reinterpret_cast<const uint16_t*>(a.v_re);
    const uint16_t* vi_p = reinterpret_cast<const uint16_t*>(a.v_im);
    // SMALL: views of this (b, h)'s key and value rows, ending at its last row
    const uint32_t ext_bh = SMALL ? (uint32_t)(((a.T - 1) * rs + D) * 2) : 0u;
    const BufRes vkr = make_buf(kr_p + base, ext_bh), vki = make_buf(ki_p + base, ext_bh);
    const BufRes vvr = make_buf(vr_p + base, ext_bh), vvi = make_buf(vi_p + base, ext_bh);

    // query blocks of 128 rows: wave w owns query tiles u = 0, 1 (rows 32w + 16u of
    // the block), so every key and value operand read from LDS serves two score tiles
    constexpr int QBR = 2 * kBornBlock;
    const int nblk = pair == a.nqb - 1 - pair ? 1 : 2;
    for (int which = 0; which < nblk; ++which) {
        const int qb = (int)(which == 0 ? pair : a.nqb - 1 - pair);
        // B operands: [qr quad, qi quad] and [-qr quad, qi quad], scaled by 1/sqrt(D tau)
        bf16x8 bre[2][NM], bim[2][NM];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t qrow = qb * QBR + 32 * w + 16 * u + lr;
            float scale = 0.f;
            int64_t o = 0;
            if (qrow < a.T) {
                o = base + qrow * rs;
                const float tq = a.tau != nullptr ? a.tau[(b * a.T + qrow) * a.H + h] : 1.f;
                scale = rsqrtf((float)D * tq);
            }
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                bf16x4 r4 = {}, i4 = {};
                if (qrow < a.T) {
                    r4 = bf4_of_bits(*reinterpret_cast<const uint2*>(qr_p + o + 16 * m + 4 * lg));
                    i4 = bf4_of_bits(*reinterpret_cast<const uint2*>(qi_p + o + 16 * m + 4 * lg));
                }
                bf16x4 sr, si, nr;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float fr = bf_to_f(r4[j]) * scale, fi = bf_to_f(i4[j]) * scale;
                    sr[j] = (__bf16)fr;
                    si[j] = (__bf16)fi;
                    nr[j] = (__bf16)(-fr);
                }
                bre[u][m] = cat8(sr, si);
                bim[u][m] = cat8(nr, si);
            }
        }
        floatx4 o[2][NCT];
        // row sums of the rounded weights, as one more product with a column of ones:
        // register r of lane j + 16g ends up with the sum for query 4g + r of the tile
        floatx4 den4[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            den4[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NCT; ++c) o[u][c] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        const __bf16 one = (__bf16)1.0f;
        const bf16x8 ones = {one, one, one, one, one, one, one, one};

        // staging registers, RD sets (blocks kb + 1 .. kb + RD in flight while block kb
        // is used): KQ key quads (real 8 B + imaginary 8 B) and VQ value chunks (16 B)
        uint2 skr[RD][KQ], ski[RD][KQ];
        uint4 sv[RD][VQ];
        auto fetch = [&](int kb, int set) {
            if constexpr (SMALL) {
                // through the views of this (b, h)'s rows: the block's offset joins
                // the lane's constant one, rows past the sequence read as zero
                const uint32_t boff = (uint32_t)kb * (uint32_t)(kBornBlock * rs * 2);
#pragma unroll
                for (int i = 0; i < KQ; ++i) {
                    const int idx = i * 256 + tid, row = idx / (D / 4), q = idx % (D / 4);
                    const uint32_t vo = (uint32_t)((row * rs + 4 * q) * 2) + boff;
                    skr[set][i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vkr, vo, 0, 0));
                    ski[set][i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vki, vo, 0, 0));
                }
#pragma unroll
                for (int i = 0; i < VQ; ++i) {
                    // a plane is a multiple of 64 chunks, so the plane is the wave's
                    const int idx = i * 256 + tid;
                    const int pl = (i * 256 + 64 * w) / (kBornBlock * D / 8);
                    const int rem = idx % (kBornBlock * D / 8), row = rem / (D / 8), c8 = rem % (D / 8);
                    const uint32_t vo = (uint32_t)((row * rs + 8 * c8) * 2) + boff;
                    sv[set][i] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(pl == 0 ? vvr : vvi, vo, 0, 0));
                }
                return;
            }
#pragma unroll
            for (int i = 0; i < KQ; ++i) {
                const int idx = i * 256 + tid, row = idx / (D / 4), q = idx % (D / 4);
                const int64_t key = kb * kBornBlock + row;
                if (key < a.T) {
                    skr[set][i] = *reinterpret_cast<const uint2*>(kr_p + base + key * rs + 4 * q);
                    ski[set][i] = *reinterpret_cast<const uint2*>(ki_p + base + key * rs + 4 * q);
                } else {
                    skr[set][i] = make_uint2(0u, 0u);
                    ski[set][i] = make_uint2(0u, 0u);
                }
            }
#pragma unroll
            for (int i = 0; i < VQ; ++i) {
                // chunk idx: plane (re, im), key row, 8 consecutive columns
                const int idx = i * 256 + tid;
                const int pl = idx / (kBornBlock * D / 8), rem = idx % (kBornBlock * D / 8);
                const int row = rem / (D / 8), c8 = rem % (D / 8);
                const int64_t key = kb * kBornBlock + row;
                const uint16_t* src = pl == 0 ? vr_p : vi_p;
                sv[set][i] = key < a.T ? *reinterpret_cast<const uint4*>(src + base + key * rs + 8 * c8)
                                       : make_uint4(0u, 0u, 0u, 0u);
            }
        };
        auto commit = [&](int buf, int set) {
#pragma unroll
            for (int i = 0; i < KQ; ++i) {
                const int idx = i * 256 + tid, row = idx / (D / 4), q = idx % (D / 4);
                *reinterpret_cast<uint4*>(&lds_k[buf][0][row * KS + 16 * q]) =
                    make_uint4(skr[set][i].x, skr[set][i].y, ski[set][i].x, ski[set][i].y);
                *reinterpret_cast<uint4*>(&lds_k[buf][1][row * KS + 16 * q]) =
                    make_uint4(ski[set][i].x, ski[set][i].y, skr[set][i].x, skr[set][i].y);
            }
#pragma unroll
            for (int i = 0; i < VQ; ++i) {
                const int idx = i * 256 + tid;
                const int pl = idx / (kBornBlock * D / 8), rem = idx % (kBornBlock * D / 8);
                const int row = rem / (D / 8), c8 = rem % (D / 8);
                *reinterpret_cast<uint4*>(&lds_v[buf][row * VS + 2 * (pl * D + 8 * c8)]) = sv[set][i];
            }
        };

        // key blocks of 64 up to the end of this query block; block b's loads go to
        // register set b % RD and are written to LDS buffer b % 2 at the end of block
        // b - 1, after which the set takes block b + RD
        const int nkb = 2 * qb + 2;
        fetch(0, 0);
        __syncthreads();  // the previous query block is done with the LDS buffers
        commit(0, 0);
#pragma unroll
        for (int j = 1; j <= RD; ++j)
            if (j < nkb) fetch(j, j % RD);
        __syncthreads();
        // a block wholly before the query block (kb < 2 qb) has no masked or empty
        // score tile for any wave; only the two blocks on the diagonal need the checks
        auto step = [&](int kb, int set_next, auto full_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
            const int buf = kb & 1;
            // key tile t of this block starts kd = 64 kb + 16 t - (128 qb + 32 w + 16 u)
            // rows after query tile u: kd < 0 unmasked, kd = 0 the diagonal tile, kd > 0 empty
            const int kd0 = 64 * kb - QBR * qb - 32 * w;
            // per 32-key step s2 (key tiles 2 s2, 2 s2 + 1): the scores of both query
            // tiles, packed to bf16 where the matrix core leaves them, then
            // O += P . [vr | vi] and the row sums
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if (!FULL && kd0 + 32 * s2 - 16 > 0) continue;  // both query tiles empty (wave-uniform)
                bf16x8 are[2][NM], aim[2][NM];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int m = 0; m < NM; ++m) {
                        const int ko = (16 * (2 * s2 + tt) + lr) * KS + 16 * (4 * m + lg);
                        are[tt][m] = *reinterpret_cast<const bf16x8*>(&lds_k[buf][0][ko]);
                        aim[tt][m] = *reinterpret_cast<const bf16x8*>(&lds_k[buf][1][ko]);
                    }
                bf16x8 pa[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        const int kd = kd0 + 16 * (2 * s2 + tt) - 16 * u;
                        float v[4] = {0.f, 0.f, 0.f, 0.f};
                        if (FULL || kd <= 0) {  // wave-uniform
                            floatx4 sre = {0.f, 0.f, 0.f, 0.f}, sim = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int m = 0; m < NM; ++m) {
                                sre = __builtin_amdgcn_mfma_f32_16x16x32_bf16(are[tt][m], bre[u][m], sre, 0, 0, 0);
                                sim = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aim[tt][m], bim[u][m], sim, 0, 0, 0);
                            }
#pragma unroll
                            for (int r = 0; r < 4; ++r) v[r] = sre[r] * sre[r] + sim[r] * sim[r];
                            if (!FULL && kd == 0) {  // the diagonal tile: keys after the query drop
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (4 * lg + r > lr) v[r] = 0.f;
                            }
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) pa[u][4 * tt + r] = (__bf16)v[r];
                    }
                }
                const bool act1 = FULL || kd0 + 32 * s2 - 16 <= 0;  // query tile 1 sees this step
                const bool act0 = FULL || kd0 + 32 * s2 <= 0;
                if (act0) den4[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[0], ones, den4[0], 0, 0, 0);
                if (act1) den4[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[1], ones, den4[1], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < NCT; ++c) {
                    // lane 4 r + q of group lg points at key 32 s2 + 4 lg + r (and + 16),
                    // columns 16 c + 4 q .. + 3; the transpose read hands lane 4 q + x
                    // column 16 c + 4 q + x of those four keys
                    const int vo = (32 * s2 + 4 * lg + (lr >> 2)) * VS + 2 * (16 * c + 4 * (lr & 3));
                    const v4i16 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16*)(&lds_v[buf][vo]));
                    const v4i16 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16*)(&lds_v[buf][vo + 16 * VS]));
                    const bf16x8 vb = cat8(__builtin_bit_cast(bf16x4, v0), __builtin_bit_cast(bf16x4, v1));
                    if (act0) o[0][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[0], vb, o[0][c], 0, 0, 0);
                    if (act1) o[1][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[1], vb, o[1][c], 0, 0, 0);
                }
            }
            if (kb + 1 < nkb) commit(buf ^ 1, set_next);
            if (kb + 1 + RD < nkb) fetch(kb + 1 + RD, set_next);
            __syncthreads();
        };
        static_assert(RD == 1 || RD == 2, "2 qb must be a multiple of RD");
        for (int kb0 = 0; kb0 < 2 * qb; kb0 += RD) {
#pragma unroll
            for (int j = 0; j < RD; ++j) step(kb0 + j, (j + 1) % RD, BoolTag<true>());
        }
        step(2 * qb, 1 % RD, BoolTag<false>());
        step(2 * qb + 1, 0, BoolTag<false>());
        if constexpr (SMALL) {
            // through views of this (b, h)'s rows: 32-bit offsets, rows past the
            // sequence dropped by the extent
            const uint32_t ext = (uint32_t)(((a.T - 1) * rs + D) * 4);
            const BufRes vre = make_buf(a.out_re + base, ext), vim = make_buf(a.out_im + base, ext);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                uint32_t vo = (uint32_t)(((int64_t)(qb * QBR + 32 * w + 16 * u + 4 * lg) * rs + lr) * 4);
                asm volatile("" : "+v"(vo));
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float den = den4[u][r];
                    const float inv = den != 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;  // about 1 ulp
#pragma unroll
                    for (int c = 0; c < NCT; ++c)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            __float_as_uint(o[u][c][r] * inv), (16 * c) < D ? vre : vim,
                            vo + (uint32_t)(r * rs + (16 * c) % D) * 4, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qloc = 4 * lg + r;
                    const float den = den4[u][r];
                    const int64_t row = (int64_t)qb * QBR + 32 * w + 16 * u + qloc;
                    if (row >= a.T) continue;
                    const float inv = den != 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;  // about 1 ulp
                    const int64_t at = base + row * rs;
#pragma unroll
                    for (int c = 0; c < NCT; ++c) {
                        float* dst = (16 * c) < D ? a.out_re : a.out_im;
                        dst[at + (16 * c) % D + lr] = o[u][c][r] * inv;
                    }
                }
            }
        }
    }
}

hipError_t launch_born(const BornArgs& a, hipStream_t s) {
    const int64_t groups = (a.B * a.H + a.hpl - 1) / a.hpl;
    const int64_t per_xcd = (groups + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(kXcds * per_xcd * a.hpl * a.npair)), block(256);
    if (a.in_dtype == 1) {
        // the rows one workgroup can address, up to the end of its last 128-row
        // query block, within 2 GB of its (b, h)'s first row
        const bool small = ((a.T + 2 * kBornBlock) * a.H * a.D + a.D) * 4 < ((int64_t)1 << 31);
        switch (a.D * 2 + (small ? 1 : 0)) {
            case 33: hipLaunchKernelGGL((k_born_bf16<16, true>), grid, block, 0, s, a); break;
            case 32: hipLaunchKernelGGL((k_born_bf16<16, false>), grid, block, 0, s, a); break;
            case 65: hipLaunchKernelGGL((k_born_bf16<32, true>), grid, block, 0, s, a); break;
            case 64: hipLaunchKernelGGL((k_born_bf16<32, false>), grid, block, 0, s, a); break;
            case 129: hipLaunchKernelGGL((k_born_bf16<64, true>), grid, block, 0, s, a); break;
            case 128: hipLaunchKernelGGL((k_born_bf16<64, false>), grid, block, 0, s, a); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (a.D) {
        case 16: hipLaunchKernelGGL(k_born<16>, grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL(k_born<32>, grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL(k_born<64>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cssd
