// The whole chunkwise forward for bf16 inputs in one kernel: one workgroup per
// (b, h) walks that sequence's chunks in order and keeps the carried state in
// registers, so the carry-in states never reach memory and every input row is
// read once.  Chunk size, head dim and state dim are 64.
//
// For chunk c of sequence (b, h), rows l and columns s of the chunk:
//   y[l, :]  = sum_{s<=l} (G . L)[l, s] X[s, :] + exp(acs[l]) C[l, :] H_c + Dskip X[l, :]
//   G        = C B^T,  L[l, s] = exp(acs[l] - acs[s]) 1[l >= s]
//   H_{c+1}  = cd[c] H_c + (diag(w) B)^T X,  H_0 = h0,  hT = H_nC
// (Mamba-3-Lite docs, "SSD Theory" 4.3-4.5 and "The Chunkwise Complex SSD
// Algorithm" 4.2-4.5: the segment matrix, the intra-chunk term, the chunk
// states and the chunk-to-chunk recurrence taken in its sequential form; the
// skip term follows the burn-mamba step_constant readout).  The discretisation
// and the chunk-local cumsum (acs, e = exp(acs), w = exp(acs[C-1] - acs),
// cd = exp(acs[C-1])) are done here too, one chunk ahead, by wave 0 (which takes
// one score tile of the ten with four waves, none with eight).
//
// Every product runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  That
// instruction takes A[i][k] from lane i + 16 (k / 8), slot k % 8, B[k][j] from
// lane j + 16 (k / 8), slot k % 8, and leaves D[4g + r][j] in register r of lane
// j + 16 g.  Wave w (of four; with eight, waves w and w + 4, see the kernel) owns
// the 16 columns p = 16 w + (lane % 16) of y and of the state; its part of H sits
// in the accumulator layout of the chunk-state product: tile nt, register r of lane
// p + 16 g <-> n = 16 nt + 4 g + r.
//  * y is formed transposed, y^T = H_c^T C^T (scaled by exp(acs)) + X^T M^T, so
//    that register r of lane l + 16 g holds y[l][16 w + 4 g + r]: four adjacent
//    columns of one row, stored with one 16-byte store per plane.
//  * H_c^T C^T: A = H^T, B = C rows.  The 32-wide contraction over n takes state
//    tiles 2 ks and 2 ks + 1: slot j < 4 is n = 32 ks + 4 g + j and slot j >= 4
//    is n = 32 ks + 16 + 4 g + j - 4, which is where the accumulators hold them,
//    so H enters the product straight from its registers (rounded to bf16 as an
//    operand only); the C row is read as the two matching 8-byte pieces.
//  * G^T = B C^T: A = B rows, B = C rows, both 16-byte reads of staged rows;
//    register r of lane l + 16 g then holds G[l][s0 + 4 g + r], where
//    M = G . L (+ Dskip on the diagonal) is formed in fp32, rounded to bf16 and
//    written row-major into LDS for every wave to read.
//  * X^T M^T and (w B)^T X contract over time with 8 consecutive steps per lane
//    group: X and w B are staged row-major like C and B and their operands come
//    from transposing LDS reads (ds_read_b64_tr_b16: lane 4 q + x of a 16-lane
//    group receives element x of the 8-byte pieces that lanes q, 4 + q, 8 + q and
//    12 + q point at, so lanes 4 t + q pointing at step t, columns 4 q .. 4 q + 3,
//    hand lane 4 q + x column 4 q + x of four consecutive steps).  The X operand
//    of the wave's columns serves both products.
// Complex products are four real products (a sum of bf16 operands would round),
// the imaginary operand negated where the real part needs it.
//
// Staging: the next chunk's C, B and X rows are loaded into registers (16-byte
// pieces) while the current chunk is computed, then written to LDS with the
// pieces XOR-swizzled by the row; w B is formed from the same B pieces in fp32
// and rounded to bf16 on the way.  The M tiles overwrite the B rows once the
// scores are done.  69 KB of LDS with four waves, 84 KB for a half-width
// workgroup, 102 KB with eight.  Rows of a partial last chunk past the sequence
// read as zero through the buffer extents and their stores are dropped.
//
// Launch shapes by the number of sequences B H against the CU count: up to one a
// CU, one eight-wave workgroup each; up to two a CU, one four-wave workgroup for
// each of the first (CU count), and two half-width workgroups for each of the
// rest on a second stream, so every CU holds one whole sequence and one half;
// beyond that, four-wave workgroups in rounds.
#include <mutex>
#include <type_traits>

#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRow = 128;  // bytes of a staged bf16 row of 64 values (C, B, M, X, w B)

// physical 16-byte piece of logical piece `ch` of staged row `row`:
// ch ^ ((row >> 1) & 7).  Measured with the LDS bank-conflict counter on this chip,
// in isolation: the 16-byte operand reads (rows r0 + li, pieces 4 k + g) and the
// 8-byte C reads (two half pieces per row) are both free of conflicts with it; with
// row & 7 the 8-byte reads take 2 conflict cycles an instruction, and with a row
// bit 3 term XOR-ed in as well the 16-byte reads take 4.  The 8-byte M tile writes
// take 4 with every row swizzle tried.
__device__ __forceinline__ int swz(int row, int ch) { return ch ^ ((row >> 1) & 7); }

// the same for the rows read by transposing reads (X, w B): ch ^ f(row),
// f(i) = 2 bit1(i) + 4 bit3(i).  Such a read covers rows r0 + {0..3} (r0 a
// multiple of 4) per 16-lane group and r0 + {0..3, 8..11} per 32 lanes, 32
// bytes (pieces ch, ch + 1 of an even ch) of each; rows of one parity then take
// disjoint piece pairs, so the 16 pieces are distinct modulo 256 bytes (the LDS
// bank-conflict counter reads none for these reads)
__device__ __forceinline__ int swt(int row, int ch) { return ch ^ ((row & 2) | ((row >> 1) & 4)); }

// four bf16 at 8-byte LDS piece `at`, transposed across each 16-lane group
__device__ __forceinline__ bf16x4 ld_tr(const unsigned char* base, int at) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(base + at));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ floatx4 mfma_bf(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 bneg(bf16x8 v) {
    u32x4 u = __builtin_bit_cast(u32x4, v);
    u ^= 0x80008000u;
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ uint32_t bf16_bits(float v) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}

__device__ __forceinline__ float lo_f(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_f(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

struct FusedArgs {
    const uint16_t *x_re, *x_im, *b_re, *b_im, *c_re, *c_im;
    const float *dt, *a_re, *a_im, *dskip;
    const float *h0_re, *h0_im;
    float *y_re, *y_im, *hT_re, *hT_im;
    int64_t T;
    int H, nC;
    // workgroups from `late` on are dispatched onto CUs that already hold one
    // (late = CU count when there are more sequences than CUs, but no more than
    // twice as many; otherwise no workgroup is late and priorities stay default)
    int late;
    // the chunk at which late workgroups give up their priority (and, in the same
    // launch, the others take it)
    int swap_at;
    // the half-width launch: sequences hbase .. hbase + hcount - 1, two workgroups each
    int64_t hbase, hcount;
};

// one chunk's inputs in flight in registers: KP 16-byte pieces a thread of each
// plane of the C, B and X rows
template <int KP>
struct Pre {
    u32x4 c[2][KP], b[2][KP], x[2][KP];  // [plane][piece]
};

}  // namespace

// WAVES = 4: wave w owns the 16 columns 16 w .. of y and of the state and does all
// of that column block's work.  WAVES = 8: waves w and w + 4 share the column block;
// half hv = wave / 4 computes the row tiles {0, 3} (hv = 0) or {1, 2} of y (equal
// shares of the causal product) and the state tiles {2 hv, 2 hv + 1} of S_c and of
// the update, and both keep the whole carried state of their columns: each half's
// updated tiles pass to the other through LDS, read after the next chunk's first
// barrier.  One eight-wave workgroup per CU (101 KB of LDS); its per-chunk time is
// about half that of a four-wave workgroup alone.
// HALF (four waves): two workgroups share one sequence, each taking two of the four
// column blocks (the columns of y and of the state are independent), split between
// its waves as the eight-wave form splits one: wave v takes column block
// 2 half + (v & 1) and half hv = v / 2, and the partner wave v ^ 2 holds the other
// half's tiles.  Each repeats the scores G.  84 KB of LDS, so a CU holds one such
// workgroup next to one whole four-wave one (69 KB) and never two of them.
template <int WAVES, bool HALF>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2))) void k_scan_fused_bf16(
    FusedArgs a) {
    static_assert(WAVES == 4 || WAVES == 8, "four or eight waves");
    static_assert(!HALF || WAVES == 4, "half-width workgroups have four waves");
    constexpr int C = 64, N = 64, D = 64;
    constexpr int NT = 64 * WAVES;       // threads
    constexpr int KP = 512 / NT;         // 16-byte pieces a thread of each staged plane
    constexpr bool W8 = WAVES == 8;
    constexpr bool SPL = W8 || HALF;  // row and state tiles split between two halves
    // C rows (re, im).  The planes are 16 bytes more than a multiple of the bank
    // window apart: 8-byte reads of the two planes at one offset, which the compiler
    // merges into one two-address read, then fall in different banks (0 instead of 8
    // conflict cycles an instruction, measured).
    __shared__ __align__(16) unsigned char l_c[2][C * kRow + 16];
    __shared__ __align__(16) unsigned char l_b[2][C * kRow];    // B rows, then the M rows
    __shared__ __align__(16) unsigned char l_x[2][C * kRow];    // X rows [s][p]
    __shared__ __align__(16) unsigned char l_wb[2][C * kRow];   // w B rows [s][n]
    // per chunk, in two slots (chunk parity): the real part of the cumsums in log2
    // units, the unit phasors u = exp(i Im acs) (cos and sin of the imaginary part,
    // taken in turns and reduced to its fractional part in fp64 first), exp(acs),
    // exp(acs[C-1] - acs) and the chunk decay exp(acs[C-1])
    __shared__ __align__(16) float l_acs[2][C];
    __shared__ __align__(16) float l_u[2][2][C];
    __shared__ __align__(16) float l_e[2][2][C];
    __shared__ __align__(16) float l_w[2][2][C];
    __shared__ float l_cd[2][2];
    // split forms: each wave's two updated state tiles, [wave][4 floats][lane] x 4
    __shared__ __align__(16) float l_hx[SPL ? WAVES : 1][4][64][4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int li = lane & 15, g = lane >> 4;
    const int wv = wave_id();
    int64_t bh = blockIdx.x;
    int cg = 0;  // HALF: which two column blocks
    if constexpr (HALF) {
        // both workgroups of a sequence on one XCD (dispatch is round-robin over 8),
        // so its B and C rows are fetched into one L2
        const int64_t e = blockIdx.x, k = e / 16, x8 = e % 8;
        cg = (int)((e / 8) & 1);
        if (8 * k + x8 >= a.hcount) return;  // workgroup-uniform, before any barrier
        bh = a.hbase + 8 * k + x8;
    }
    // column block, half (split forms), and the wave holding the other half's tiles
    const int w = HALF ? 2 * cg + (wv & 1) : (wv & 3);
    const int hv = HALF ? wv >> 1 : wv >> 2;
    const int partner = HALF ? wv ^ 2 : wv ^ 4;
    const int h = (int)(bh % a.H);
    const int64_t b = bh / a.H;
    const uint32_t sN = (uint32_t)a.H * N, sD = (uint32_t)a.H * D;
    const float dk = a.dskip != nullptr ? a.dskip[h] : 0.f;
    const int pcol = 16 * w + li;  // this lane's column of y and of the state

    // the carried state, tile nt register r <-> (n = 16 nt + 4 g + r, p = pcol);
    // the state planes are addressed through buffer views of this (b, h)'s N x D
    // block, so one lane offset serves all 16 elements (the rest is immediate)
    float hr[4][4], hi[4][4];
    const uint32_t soff = (uint32_t)(4 * g) * D + pcol;
    if (a.h0_re != nullptr) {
        const BufRes r0 = make_buf(a.h0_re + bh * (int64_t)N * D, N * D * 4);
        const BufRes i0 = make_buf(a.h0_im + bh * (int64_t)N * D, N * D * 4);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hr[nt][r] = buf_f32(r0, soff + (16 * nt + r) * D);
                hi[nt][r] = buf_f32(i0, soff + (16 * nt + r) * D);
            }
    } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) hr[nt][r] = hi[nt][r] = 0.f;
    }

    // staging roles: C, B and X pieces u = tid + NT k (row u / 8, piece u % 8);
    // N = D, so one offset serves the three
    auto load = [&](int c, Pre<KP>& P) {
        const int64_t t0 = (int64_t)c * C;
        const int valid = (int)min<int64_t>((int64_t)C, a.T - t0);
        const int64_t row0 = (b * a.T + t0) * a.H + h;
        const uint32_t extN = ((uint32_t)(valid - 1) * sN + N) * 2u;
        const uint32_t extD = ((uint32_t)(valid - 1) * sD + D) * 2u;
        const BufRes rc[2] = {make_buf(a.c_re + row0 * N, extN), make_buf(a.c_im + row0 * N, extN)};
        const BufRes rb[2] = {make_buf(a.b_re + row0 * N, extN), make_buf(a.b_im + row0 * N, extN)};
        const BufRes rx[2] = {make_buf(a.x_re + row0 * D, extD), make_buf(a.x_im + row0 * D, extD)};
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                const int u = tid + NT * k;
                const uint32_t off = ((uint32_t)(u >> 3) * sN + 8 * (u & 7)) * 2u;
                P.c[pl][k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc[pl], off, 0, 0));
                P.b[pl][k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb[pl], off, 0, 0));
                P.x[pl][k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx[pl], off, 0, 0));
            }
    };
    // the staged rows of chunk slot `slot`, and w B from the B pieces and w of
    // that chunk (formed in fp32, rounded to bf16)
    auto stage = [&](const Pre<KP>& P, int slot) {
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int u = tid + NT * k, row = u >> 3;
            const int at = row * kRow + 16 * swz(row, u & 7);
            const int atx = row * kRow + 16 * swt(row, u & 7);
#pragma unroll
            for (int pl = 0; pl < 2; ++pl) {
                *reinterpret_cast<u32x4*>(&l_c[pl][at]) = P.c[pl][k];
                *reinterpret_cast<u32x4*>(&l_b[pl][at]) = P.b[pl][k];
                *reinterpret_cast<u32x4*>(&l_x[pl][atx]) = P.x[pl][k];
            }
            const float wr = l_w[slot][0][row], wi = l_w[slot][1][row];
            u32x4 pr, pi;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t vr = P.b[0][k][j], vi = P.b[1][k][j];
                const float br[2] = {lo_f(vr), hi_f(vr)}, bi[2] = {lo_f(vi), hi_f(vi)};
                uint32_t ur[2], ui[2];
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    ur[f] = bf16_bits(wr * br[f] - wi * bi[f]);
                    ui[f] = bf16_bits(wr * bi[f] + wi * br[f]);
                }
                pr[j] = ur[0] | (ur[1] << 16);
                pi[j] = ui[0] | (ui[1] << 16);
            }
            *reinterpret_cast<u32x4*>(&l_wb[0][atx]) = pr;
            *reinterpret_cast<u32x4*>(&l_wb[1][atx]) = pi;
        }
    };
    // the discretisation and chunk-local cumsum of chunk c (wave 0, lane l holds
    // position l), from its raw steps dtv, into slot c & 1:
    //   A_log[l] = softplus(dt) A (0 past the sequence), acs = inclusive cumsum,
    //   e = exp(acs), w = exp(acs[C-1] - acs), cd = exp(acs[C-1])
    // ("The Chunkwise Complex SSD Algorithm" 4.2, "SSD Theory" 4.3 and 4.5).  The
    // sums stay fp64; the exponentials take the fp64 arguments reduced to log2
    // units and to half a turn, then the fp32 hardware exp2 / sin / cos, as the
    // segment matrix does.
    const float are_f = a.a_re[h], aim_f = a.a_im[h];
    auto cumsum = [&](int c, float dtv) {
        float fr = are_f, fi = aim_f;
        asm volatile("" : "+s"(fr), "+s"(fi));  // widened here, not kept live as fp64
        const double are = fr, aim = fi;
        // an opaque copy of the lane index: the addresses below are recomputed
        // here rather than kept live across the loop
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const int slot = c & 1;
        const int64_t t = (int64_t)c * C + lane;
        double vr = 0.0, vi = 0.0;
        if (t < a.T) {
            // softplus in fp32 (log1pf / expf of the device library, about one ulp):
            // this path's operands are bf16, whose rounding is 2^15 times coarser
            const double sp = (double)(fmaxf(dtv, 0.f) + log1pf(expf(-fabsf(dtv))));
            vr = sp * are;
            vi = sp * aim;
        }
        wave_inclusive_scan(vr);
        wave_inclusive_scan(vi);
        const double tr = lane_value(vr, 63), ti = lane_value(vi, 63);
        const double ar2 = vr * kLog2e, at2 = vi * kInvTwoPi;  // log2 units, turns
        l_acs[slot][lane] = (float)ar2;
        const float turn = (float)(at2 - rint(at2));
        const float ur = __builtin_amdgcn_cosf(turn), ui = __builtin_amdgcn_sinf(turn);
        l_u[slot][0][lane] = ur;
        l_u[slot][1][lane] = ui;
        const float mag = __builtin_amdgcn_exp2f((float)ar2);
        const float er = mag * ur, ei = mag * ui;
        float wr, wi;
        const double wr2 = (tr - vr) * kLog2e, wt2 = (ti - vi) * kInvTwoPi;
        cexp_scaled((float)wr2, (float)(wt2 - rint(wt2)), wr, wi);
        l_e[slot][0][lane] = er;
        l_e[slot][1][lane] = ei;
        l_w[slot][0][lane] = wr;
        l_w[slot][1][lane] = wi;
        if (lane == 63) {  // acs[C-1] is the chunk total
            l_cd[slot][0] = er;
            l_cd[slot][1] = ei;
        }
    };
    auto load_dt = [&](int c) {
        const int64_t t = (int64_t)c * C + lane;
        return t < a.T ? a.dt[(b * a.T + t) * a.H + h] : 0.f;
    };

    // Memory operations are issued in the same order and number on every wave and
    // every pass: per chunk c, the next chunk's rows (load), the raw steps of chunk
    // c + 2 (every wave loads them; wave 0 uses them), then the output stores (two
    // a row tile).  The prologue mirrors that with as many stores through a view of
    // extent 0 (all dropped).  The compiler's waits for a prefetch then count the operations
    // issued after it exactly, also across the loop's back edge, instead of
    // waiting for the output stores or for the loads just issued.
    constexpr int NLT = SPL ? 2 : 4;  // row tiles of y a wave
    Pre<KP> P;
    load(0, P);
    const float dt0 = load_dt(0);
    float dtn = a.nC > 1 ? load_dt(1) : 0.f;  // the raw steps of the chunk after next
    {
        const BufRes none = make_buf(a.y_re, 0);
#pragma unroll
        for (int i = 0; i < 2 * NLT; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, none, 16u * i, 0, 0);
    }
    if (wv == 0) cumsum(0, dt0);
    // Wave priority.  Of two workgroups on one CU, the one dispatched first wins
    // instruction arbitration and the other falls behind (measured: 14.1K against
    // 17.2K clocks a chunk), and the kernel waits for the one behind.  So a late
    // workgroup (a.late) takes priority up to chunk a.swap_at and, where the
    // early ones are in the same launch, gives it to them from there (two whole
    // workgroups on a CU, measured at B 8, T 2048, H 48: 0.292 ms with default
    // priorities, 0.281 switching at one half, 0.277 at 9/16 and at 5/8; the
    // launcher now splits that case into whole and half-width workgroups).
    const bool late = (int)blockIdx.x >= a.late;  // wave-uniform
    if (late) __builtin_amdgcn_s_setprio(1);
    for (int c = 0; c < a.nC; ++c) {
        if (c == a.swap_at && a.late < (1 << 30)) {
            if (late) __builtin_amdgcn_s_setprio(0);
            else __builtin_amdgcn_s_setprio(1);
        }
        const int64_t t0 = (int64_t)c * C;
        const int valid = (int)min<int64_t>((int64_t)C, a.T - t0);
        const int64_t row0 = (b * a.T + t0) * a.H + h;
        const int slot = c & 1;
        const float* const acs_r = l_acs[slot];
        const float* const u_r = l_u[slot][0];
        const float* const u_i = l_u[slot][1];
        const float* const le_r = l_e[slot][0];
        const float* const le_i = l_e[slot][1];

        __syncthreads();  // every wave is done with the previous chunk's LDS
        if (SPL && c > 0) {
            // the other half's two updated state tiles (2 (1 - hv), 2 (1 - hv) + 1)
            const float4* src = reinterpret_cast<const float4*>(&l_hx[SPL ? partner : 0][0][lane][0]);
            auto take = [&](auto nt0) {
                constexpr int T0 = decltype(nt0)::value;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float4 vr = src[(2 * j) * 64], vi = src[(2 * j + 1) * 64];
                    hr[T0 + j][0] = vr.x; hr[T0 + j][1] = vr.y; hr[T0 + j][2] = vr.z; hr[T0 + j][3] = vr.w;
                    hi[T0 + j][0] = vi.x; hi[T0 + j][1] = vi.y; hi[T0 + j][2] = vi.z; hi[T0 + j][3] = vi.w;
                }
            };
            if (hv == 0) take(std::integral_constant<int, 2>());
            else take(std::integral_constant<int, 0>());
        }
        stage(P, slot);
        if (c + 1 < a.nC) load(c + 1, P);
        __syncthreads();

        // ---- wave 0 has the fewest score tiles: it discretises the next chunk first
        // (into the other slot, last read in the previous chunk)
        if (wv == 0 && c + 1 < a.nC) cumsum(c + 1, dtn);
        if (c + 2 < a.nC) dtn = load_dt(c + 2);

        // ---- score tiles q in [q0, q0 + nq) of the 10 lt-major causal tiles:
        // M = G . L (+ Dskip).  Wave 0, which also discretises the next chunk, takes
        // the first diagonal tile alone; waves 1-3 take three tiles each, one of
        // them diagonal.
        // WAVES = 8: wave 0 only discretises; waves 1-3 take two tiles (q 0-5),
        // waves 4-7 one (q 6-9)
        constexpr int MQ = W8 ? 2 : 3;
        const int q0 = W8 ? (wv <= 3 ? 2 * (wv - 1) : wv + 2) : (wv == 0 ? 0 : 3 * wv - 2);
        const int nq = W8 ? (wv == 0 ? 0 : (wv <= 3 ? 2 : 1)) : (wv == 0 ? 1 : 3);  // wave-uniform
        const bool full = W8 ? false : wv != 0;  // four waves: three tiles, unconditional
        bf16x4 m_r[MQ], m_i[MQ];
        int m_lt[MQ], m_st[MQ];
        {
            int lt = 0, st = W8 && wv == 0 ? 0 : q0;
            while (st > lt) {
                st -= lt + 1;
                ++lt;
            }
#pragma unroll
            for (int jq = 0; jq < MQ; ++jq) {
                m_lt[jq] = lt;
                m_st[jq] = st;
                if ((!W8 && (jq == 0 || full)) || (W8 && jq < nq)) {  // wave-uniform
                    // register r <-> (l = 16 lt + li, s = 16 st + 4 g + r)
                    const int lrow = 16 * lt + li, s0 = 16 * st + 4 * g;
                    const float alr = acs_r[lrow], ulr = u_r[lrow], uli = u_i[lrow];
                    const floatx4 asr = *reinterpret_cast<const floatx4*>(&acs_r[s0]);
                    const floatx4 usr = *reinterpret_cast<const floatx4*>(&u_r[s0]);
                    const floatx4 usi = *reinterpret_cast<const floatx4*>(&u_i[s0]);
                    floatx4 gr = {0.f, 0.f, 0.f, 0.f}, gi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const int ch = 4 * ks + g;
                        const int sb = 16 * st + li;
                        const bf16x8 br = *reinterpret_cast<const bf16x8*>(&l_b[0][sb * kRow + 16 * swz(sb, ch)]);
                        const bf16x8 bi = *reinterpret_cast<const bf16x8*>(&l_b[1][sb * kRow + 16 * swz(sb, ch)]);
                        const bf16x8 cr = *reinterpret_cast<const bf16x8*>(&l_c[0][lrow * kRow + 16 * swz(lrow, ch)]);
                        const bf16x8 ci = *reinterpret_cast<const bf16x8*>(&l_c[1][lrow * kRow + 16 * swz(lrow, ch)]);
                        gr = mfma_bf(br, cr, gr);
                        gr = mfma_bf(bneg(bi), ci, gr);
                        gi = mfma_bf(br, ci, gi);
                        gi = mfma_bf(bi, cr, gi);
                    }
                    // L = exp2(Re acs[l] - Re acs[s]) u[l] conj(u[s]): the magnitude
                    // from an fp32 difference of log2 cumsums (they differ by a chunk's
                    // log-decay at most), the phase as a product of unit phasors.
                    // Computed for every element and selected (not branched on), so
                    // the four overlap; above the diagonal the magnitude may overflow
                    // and is dropped.
                    const bool diag = (lt == st);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float mag = __builtin_amdgcn_exp2f(alr - asr[r]);
                        const float pr = ulr * usr[r] + uli * usi[r];
                        const float pim = uli * usr[r] - ulr * usi[r];
                        const bool keep = !diag || s0 + r <= lrow;
                        const float lr = keep ? mag * pr : 0.f;
                        const float lim = keep ? mag * pim : 0.f;
                        m_r[jq][r] = (__bf16)(gr[r] * lr - gi[r] * lim + ((diag && s0 + r == lrow) ? dk : 0.f));
                        m_i[jq][r] = (__bf16)(gr[r] * lim + gi[r] * lr);
                    }
                    if (++st > lt) {
                        st = 0;
                        ++lt;
                    }
                }
            }
        }
        __syncthreads();  // the B rows are free: every wave's scores are done

        // ---- the M rows [l][s] over the B rows; the two non-causal tiles that a
        // 32-step product reads, (0, 1) and (2, 3), are zero
#pragma unroll
        for (int jq = 0; jq < MQ; ++jq) {
            if ((!W8 && (jq == 0 || full)) || (W8 && jq < nq)) {
                const int l = 16 * m_lt[jq] + li, s0 = 16 * m_st[jq] + 4 * g;
                const int at = l * kRow + 16 * swz(l, s0 >> 3) + 2 * (s0 & 7);
                *reinterpret_cast<bf16x4*>(&l_b[0][at]) = m_r[jq];
                *reinterpret_cast<bf16x4*>(&l_b[1][at]) = m_i[jq];
            }
        }
        if (wv == 0) {
            int zl = threadIdx.x & 63;  // opaque copy of the lane index (see cumsum)
            asm volatile("" : "+v"(zl));
#pragma unroll
            for (int zt = 0; zt < 2; ++zt) {
                const int l = 32 * zt + (zl & 15), s0 = 32 * zt + 16 + 4 * (zl >> 4);
                const int at = l * kRow + 16 * swz(l, s0 >> 3) + 2 * (s0 & 7);
                *reinterpret_cast<u32x2*>(&l_b[0][at]) = u32x2{0u, 0u};
                *reinterpret_cast<u32x2*>(&l_b[1][at]) = u32x2{0u, 0u};
            }
        }
        __syncthreads();

        // ---- the X operand of this wave's columns: slot j <-> s = 32 k2 + 8 g + j.
        // Lane 4 t + q (of li) points at step 8 g + t (+ 4 for slots 4-7, + 32 k2),
        // columns 16 c16 + 4 q .. + 3; the read hands lane li column 16 c16 + li.
        // The swizzle depends on bits 1 and 3 of the step only, so the + 4 and
        // + 32 k2 steps are immediate offsets (512 and 4096 k2 bytes), and column
        // group c16 sits at tr_base(c16) = tr_base(0) ^ 32 c16.
        auto tr_base = [&](int c16) {
            int s = 8 * g + (li >> 2);
            asm volatile("" : "+v"(s));  // recomputed where used, not kept live
            return (s * kRow + 16 * swt(s, (li & 3) >> 1) + 8 * (li & 1)) ^ (32 * c16);
        };
        bf16x8 xr[2], xi[2], xni[2];
        {
            const int ax = tr_base(w);
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int a0 = ax + 4096 * k2, a1 = a0 + 512;
                xr[k2] = cat8(ld_tr(l_x[0], a0), ld_tr(l_x[0], a1));
                xi[k2] = cat8(ld_tr(l_x[1], a0), ld_tr(l_x[1], a1));
                xni[k2] = bneg(xi[k2]);
            }
        }
        // ---- per row tile lt: y^T = (C H_c)^T diag(exp(acs)) + X^T M^T, then stored
        // (register r of lane li + 16 g <-> row 16 lt + li, column 16 w + 4 g + r;
        // rows past the sequence are dropped by the extent)
        {
            // H_c^T as the A operand: slot j <-> n = 32 ks + 4 g + j (j < 4),
            // 32 ks + 16 + 4 g + j - 4 (j >= 4), the accumulator registers themselves
            bf16x8 hb_r[2], hb_i[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    hb_r[ks][j] = (__bf16)hr[2 * ks][j];
                    hb_r[ks][j + 4] = (__bf16)hr[2 * ks + 1][j];
                    hb_i[ks][j] = (__bf16)hi[2 * ks][j];
                    hb_i[ks][j + 4] = (__bf16)hi[2 * ks + 1][j];
                }
            const uint32_t extD = (uint32_t)(valid - 1) * sD + D;
            const BufRes ry_r = make_buf(a.y_re + row0 * D, extD * 4);
            const BufRes ry_i = make_buf(a.y_im + row0 * D, extD * 4);
#pragma unroll
            for (int jt = 0; jt < NLT; ++jt) {
                const int lt = SPL ? (hv == 0 ? 3 * jt : 1 + jt) : jt;  // wave-uniform
                floatx4 yr = {0.f, 0.f, 0.f, 0.f}, yi = {0.f, 0.f, 0.f, 0.f};
                const int l = 16 * lt + li;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    // C[l][32 ks + 4 g + 0..3] and C[l][32 ks + 16 + 4 g + 0..3]
                    const int ch = 4 * ks + (g >> 1), o8 = 8 * (g & 1);
                    const int a0 = l * kRow + 16 * swz(l, ch) + o8;
                    const int a1 = l * kRow + 16 * swz(l, ch + 2) + o8;
                    const u32x2 r0 = *reinterpret_cast<const u32x2*>(&l_c[0][a0]);
                    const u32x2 r1 = *reinterpret_cast<const u32x2*>(&l_c[0][a1]);
                    const u32x2 i0 = *reinterpret_cast<const u32x2*>(&l_c[1][a0]);
                    const u32x2 i1 = *reinterpret_cast<const u32x2*>(&l_c[1][a1]);
                    const bf16x8 cr = __builtin_bit_cast(bf16x8, u32x4{r0[0], r0[1], r1[0], r1[1]});
                    const bf16x8 ci = __builtin_bit_cast(bf16x8, u32x4{i0[0], i0[1], i1[0], i1[1]});
                    yr = mfma_bf(hb_r[ks], cr, yr);
                    yr = mfma_bf(bneg(hb_i[ks]), ci, yr);
                    yi = mfma_bf(hb_i[ks], cr, yi);
                    yi = mfma_bf(hb_r[ks], ci, yi);
                }
                {
                    const float er = le_r[l], ei = le_i[l];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float re = yr[r], im = yi[r];
                        yr[r] = er * re - ei * im;
                        yi[r] = er * im + ei * re;
                    }
                }
                // X^T M^T over s in 32-steps (the second only for rows 32 and up)
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    if (k2 == 1 && lt < 2) continue;
                    const int ch = 4 * k2 + g;
                    const bf16x8 mr = *reinterpret_cast<const bf16x8*>(&l_b[0][l * kRow + 16 * swz(l, ch)]);
                    const bf16x8 mi = *reinterpret_cast<const bf16x8*>(&l_b[1][l * kRow + 16 * swz(l, ch)]);
                    yr = mfma_bf(xr[k2], mr, yr);
                    yr = mfma_bf(xni[k2], mi, yr);
                    yi = mfma_bf(xi[k2], mr, yi);
                    yi = mfma_bf(xr[k2], mi, yi);
                }
                const uint32_t off = ((uint32_t)l * sD + 16 * w + 4 * g) * 4u;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, yr), ry_r, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, yi), ry_i, off, 0, 0);
            }
        }
        // ---- S_c = (w B)^T X on this wave's columns, then H_{c+1} = cd H_c + S_c
        const float dr = l_cd[slot][0], di = l_cd[slot][1];
        auto update = [&](auto nt_c) {
            constexpr int nt = decltype(nt_c)::value;
            floatx4 sr = {0.f, 0.f, 0.f, 0.f}, si = {0.f, 0.f, 0.f, 0.f};
            const int an = tr_base(nt);
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                // (w B)^T[16 nt + li][32 k2 + 8 g + j] in slot j
                const int a0 = an + 4096 * k2, a1 = a0 + 512;
                const bf16x8 ar = cat8(ld_tr(l_wb[0], a0), ld_tr(l_wb[0], a1));
                const bf16x8 ai = cat8(ld_tr(l_wb[1], a0), ld_tr(l_wb[1], a1));
                sr = mfma_bf(ar, xr[k2], sr);
                sr = mfma_bf(ai, xni[k2], sr);
                si = mfma_bf(ar, xi[k2], si);
                si = mfma_bf(ai, xr[k2], si);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float nr = dr * hr[nt][r] - di * hi[nt][r] + sr[r];
                const float ni = dr * hi[nt][r] + di * hr[nt][r] + si[r];
                hr[nt][r] = nr;
                hi[nt][r] = ni;
            }
        };
        // split forms: this half's two tiles, handed to the other half through LDS
        auto give = [&](auto nt0) {
            constexpr int T0 = decltype(nt0)::value;
            float4* dst = reinterpret_cast<float4*>(&l_hx[SPL ? wv : 0][0][lane][0]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                dst[(2 * j) * 64] = float4{hr[T0 + j][0], hr[T0 + j][1], hr[T0 + j][2], hr[T0 + j][3]};
                dst[(2 * j + 1) * 64] = float4{hi[T0 + j][0], hi[T0 + j][1], hi[T0 + j][2], hi[T0 + j][3]};
            }
        };
        if (!SPL) {
            update(std::integral_constant<int, 0>());
            update(std::integral_constant<int, 1>());
            update(std::integral_constant<int, 2>());
            update(std::integral_constant<int, 3>());
        } else if (hv == 0) {
            update(std::integral_constant<int, 0>());
            update(std::integral_constant<int, 1>());
            if (c + 1 < a.nC) give(std::integral_constant<int, 0>());
        } else {
            update(std::integral_constant<int, 2>());
            update(std::integral_constant<int, 3>());
            if (c + 1 < a.nC) give(std::integral_constant<int, 2>());
        }
    }
    if (a.hT_re != nullptr) {
        // split forms: each half stores the tiles it updated last
        const BufRes r1 = make_buf(a.hT_re + bh * (int64_t)N * D, N * D * 4);
        const BufRes i1 = make_buf(a.hT_im + bh * (int64_t)N * D, N * D * 4);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            if (SPL && (nt >> 1) != hv) continue;  // wave-uniform
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                buf_store_f32(hr[nt][r], r1, soff + (16 * nt + r) * D);
                buf_store_f32(hi[nt][r], i1, soff + (16 * nt + r) * D);
            }
        }
    }
}

namespace {

// The second stream of the split launch and its fork and join events, one set per
// device, created on the first split launch on that device (default priority,
// timing off) and kept until the process ends.  The launcher enqueues under the
// set's lock, so each wait binds to the record of the same call also when several
// host threads launch at once.
struct SideSet {
    std::mutex m;
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};

hipError_t side_set(SideSet** out) {
    static SideSet sets[64];
    static std::mutex init;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    SideSet& ss = sets[dev];
    std::lock_guard<std::mutex> lock(init);
    if (ss.s == nullptr) {
        hipStream_t st = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
        if (e != hipSuccess) {
            if (j != nullptr) (void)hipEventDestroy(j);
            if (f != nullptr) (void)hipEventDestroy(f);
            if (st != nullptr) (void)hipStreamDestroy(st);
            return e;
        }
        ss.fork = f;
        ss.join = j;
        ss.s = st;
    }
    *out = &ss;
    return hipSuccess;
}

}  // namespace

bool scan_fused(const FwdArgs& f) {
    return f.in_dtype == 1 && f.C == 64 && f.N == 64 && f.D == 64;
}

hipError_t launch_scan_fused(const FwdArgs& f, hipStream_t s) {
    if (!scan_fused(f)) return hipErrorNotSupported;
    FusedArgs a;
    a.x_re = static_cast<const uint16_t*>(f.x_re);
    a.x_im = static_cast<const uint16_t*>(f.x_im);
    a.b_re = static_cast<const uint16_t*>(f.b_re);
    a.b_im = static_cast<const uint16_t*>(f.b_im);
    a.c_re = static_cast<const uint16_t*>(f.c_re);
    a.c_im = static_cast<const uint16_t*>(f.c_im);
    a.dt = f.dt; a.a_re = f.a_re; a.a_im = f.a_im; a.dskip = f.dskip;
    a.h0_re = f.h0_re; a.h0_im = f.h0_im;
    a.y_re = f.y_re; a.y_im = f.y_im; a.hT_re = f.hT_re; a.hT_im = f.hT_im;
    a.T = f.T; a.H = (int)f.H; a.nC = (int)f.nC;
    a.hbase = 0;
    a.hcount = 0;
    const int64_t nseq = f.B * f.H;
    int cus = 0;
    if (device_cu_count(&cus) != hipSuccess) cus = 0;
    a.late = 1 << 30;
    a.swap_at = a.nC;
    // eight waves when every sequence gets a CU of its own (T 2048, H 48, B 1:
    // 0.126 ms against 0.159 with four; B 4: 0.166 against 0.194)
    if (cus > 0 && nseq <= cus) {
        hipLaunchKernelGGL((k_scan_fused_bf16<8, false>), dim3((unsigned)nseq), dim3(512), 0, s, a);
        return hipGetLastError();
    }
    if (cus > 0 && nseq <= 2 * (int64_t)cus) {
        // more sequences than CUs, at most twice as many: the first `cus` run whole,
        // one four-wave workgroup each, and the rest as two half-width workgroups
        // each, launched beside them on a second stream.  LDS admits one whole and
        // one half on a CU, never two halves, so the work spreads over every CU
        // instead of two whole sequences on half of them (a half costs nearly a
        // whole's vector work: 0.257-0.260 ms against 0.277 at B 8, T 2048, H 48).
        SideSet* ss = nullptr;
        hipError_t e = side_set(&ss);
        if (e != hipSuccess) return e;
        FusedArgs hb = a;
        hb.hbase = cus;
        hb.hcount = nseq - cus;
        // the halves are dispatched after the whole workgroups they share CUs with,
        // which then win instruction arbitration (the halves took 0.246 ms, the
        // wholes 0.216, at B 8, T 2048, H 48): the halves take wave priority for
        // the first 9/16 of their chunks (measured with the switch at 0, 6, 8, 10,
        // 12 and 16 sixteenths: 0.269, 0.263, 0.260, 0.261, 0.265 and 0.272 ms)
        hb.late = 0;
        hb.swap_at = (9 * a.nC) / 16;
        const int64_t hblocks = 16 * ((hb.hcount + 7) / 8);
        std::lock_guard<std::mutex> lock(ss->m);
        e = hipEventRecord(ss->fork, s);
        if (e == hipSuccess) e = hipStreamWaitEvent(ss->s, ss->fork, 0);
        if (e == hipSuccess) {
            hipLaunchKernelGGL((k_scan_fused_bf16<4, false>), dim3((unsigned)cus), dim3(256), 0, s, a);
            e = hipGetLastError();
        }
        if (e == hipSuccess) {
            hipLaunchKernelGGL((k_scan_fused_bf16<4, true>), dim3((unsigned)hblocks), dim3(256), 0,
                               ss->s, hb);
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipEventRecord(ss->join, ss->s);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, ss->join, 0);
        return e;
    }
    // more than twice as many sequences as CUs (or no CU count): four waves, in
    // rounds of two workgroups a CU
    hipLaunchKernelGGL((k_scan_fused_bf16<4, false>), dim3((unsigned)nseq), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace cssd
