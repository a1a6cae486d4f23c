// K2 for fp32 inputs at C = 128, N = 128, D = 64 (the long-sequence shape,
// whose 128-row chunks hold 256 KB of C and B rows): the same output as
// k_chunk_scan (see k_chunk_scan.h for the formulas and passages), with every
// input row of a chunk read from memory once.
//
// One persistent workgroup of eight waves per CU walks the chunks
// blockIdx.x, blockIdx.x + gridDim.x, ...  Wave w owns the 16 output columns
// [16 (w % 4), 16 (w % 4) + 16) of the four row tiles {h, 2 + h, 5 - h, 7 - h},
// h = w / 4: both halves carry 18 causal tile products.  The state dimension n
// is taken in eight blocks of 16.  For each block the chunk's C and B rows
// restricted to it (32 KB) and the block's rows of H_c (8 KB) are staged in LDS
// by direct-to-LDS buffer loads (row pieces XOR-swizzled) into three buffers,
// block k + 2 issued while block k is used (the third buffer is the start of the
// M region, free until the last block).  Per block:
//   Y_off += C[:, blk] H_c[blk, cols]            (the wave's four row tiles)
//   G^T   += B[s tile, blk] C[l tile, blk]^T     (the wave's score tiles: 36
//                                                 causal tiles, five for waves
//                                                 0-3 and four for 4-7, so the
//                                                 two waves of a SIMD hold nine)
// After the last block: Y_off times exp(acs[l]) per row, M = G . L (+ Dskip on
// the diagonal) in registers and into a 72 KB LDS region, the wave's columns of
// X into registers (half of them issued with the last block), Y_diag = M X.  The
// next chunk's first two blocks are staged while the M X products run, and this
// chunk's outputs are stored during the next chunk's first block.  156 KB of
// LDS: one workgroup per CU.
#pragma once

#include "k_chunk_scan_lds.h"

namespace cssd {

// s_waitcnt immediate for at most `vm` vector-memory and `lgkm` LDS/scalar
// operations outstanding (gfx9 encoding; expcnt not waited on)
constexpr int waitcnt_vm_lgkm(int vm, int lgkm) {
    return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

// A workgroup barrier without the workgroup-scope release/acquire fences of
// __syncthreads(): those would also wait for every direct-to-LDS load still in
// flight, which is what the staging ahead must not do.  The caller first waits
// for exactly what the other waves will read (its own staged loads, vmcnt; its
// LDS writes, lgkmcnt); the memory clobber keeps the compiler from moving LDS
// accesses across.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

template <int C, int N, int D>
__global__ __launch_bounds__(512) void k_chunk_scan_wide(ScanArgs a) {
    constexpr int NB = 16;                   // n per staged block
    constexpr int NBLK = N / NB;             // blocks per chunk
    constexpr int NLT = C / 16;              // row tiles per chunk
    constexpr int NP = NLT * (NLT + 1) / 2;  // causal tiles, lt-major
    constexpr int MQ = 5;                    // most score tiles one wave owns
    constexpr int PL = C * NB;               // floats of one staged C or B plane
    constexpr int HP = NB * D;               // floats of one staged H plane
    constexpr int BUF = 4 * PL + 2 * HP;     // floats of one block buffer
    // direct-to-LDS loads per wave for one block: four C/B pieces and one H piece
    constexpr int LPB = 5;
    static_assert(C == 128 && N == 128 && D == 64, "built for C = N = 128, D = 64");
    static_assert(PL == 8 * 256 && HP == 4 * 256, "one 1 KB load per wave and plane");
    static_assert(NP == 36 && 4 * 5 + 4 * 4 == NP, "score tiles: five for waves 0-3, four for 4-7");
    static_assert(BUF <= NP * 512, "the third block buffer must fit in the M region");
    // separate LDS objects, so that the compiler's wait for pending direct-to-LDS
    // writes before an LDS read covers only the object read
    __shared__ floatx4 lds_s0[BUF / 4];       // block buffer 0: C re, C im, B re, B im, H re, H im
    __shared__ floatx4 lds_s1[BUF / 4];       // block buffer 1
    __shared__ floatx4 lds_m4[NP * 512 / 4];  // the M tiles (re, im planes of 1 KB); buffer 2
    __shared__ floatx4 lds_a4[4 * 256 / 4];   // acs re, acs im (fp64), e re, e im
    float* const ls0 = reinterpret_cast<float*>(lds_s0);
    float* const ls1 = reinterpret_cast<float*>(lds_s1);
    float* const ldm = reinterpret_cast<float*>(lds_m4);
    float* const lda = reinterpret_cast<float*>(lds_a4);
    const double* const lacs_r = reinterpret_cast<const double*>(lda);
    const double* const lacs_i = reinterpret_cast<const double*>(lda + 256);
    const float* const le_r = lda + 512;
    const float* const le_i = lda + 768;
    // block k of a chunk lives in buffer k % 3
    auto buf_of = [&](int k) -> float* { return k % 3 == 0 ? ls0 : (k % 3 == 1 ? ls1 : ldm); };

    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int w = wave_id();
    const int ct = w & 3, hf = w >> 2;
    const uint32_t sN = (uint32_t)a.H * N, sD = (uint32_t)a.H * D;

    // the four row tiles of this wave
    int rows[4];
    rows[0] = hf;
    rows[1] = 2 + hf;
    rows[2] = 5 - hf;
    rows[3] = 7 - hf;
    // the score tiles of this wave: q in [q0, q0 + nq), lt-major
    const int q0 = w < 4 ? 5 * w : 20 + 4 * (w - 4);
    const int nq = w < 4 ? 5 : 4;
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

    // per-chunk views; rows past the chunk's last real row lie past the extents
    struct Ctx {
        int64_t row0, pbase, chunk;
        uint32_t extN, extD;
        int h;
    };
    auto ctx_of = [&](int64_t chunk) {
        Ctx x;
        const int c = (int)(chunk % a.nC);
        const int64_t bh = chunk / a.nC;
        x.h = (int)(bh % a.H);
        const int64_t b = bh / a.H;
        const int64_t t0 = (int64_t)c * C;
        const int valid = (int)min<int64_t>((int64_t)C, a.T - t0);
        x.row0 = (b * a.T + t0) * a.H + x.h;
        x.pbase = bh * (int64_t)a.nC * C + t0;
        x.chunk = chunk;
        x.extN = (uint32_t)(valid - 1) * sN + N;
        x.extD = (uint32_t)(valid - 1) * sD + D;
        return x;
    };
    // 16-byte piece swizzle of a staged 64-byte row: logical piece c of row `row`
    // sits at physical piece c ^ f(row & 15), f(i) = ((i >> 2) ^ (i >> 1)) & 3.
    // The MFMA operand reads take piece g of rows 16 t + i, i = 0..15: any 8
    // consecutive lanes then cover 128 distinct bytes modulo 128 and any 16 cover
    // 256 distinct bytes modulo 256, so the reads are free of bank conflicts
    // whether a pass serves 8 or 16 lanes.
    auto swz = [](int row, int c) { return c ^ ((((row & 15) >> 2) ^ ((row & 15) >> 1)) & 3); };
    // block blk of a chunk: wave w loads 1 KB piece-block w of each of the four C/B
    // planes, and piece w % 4 of H plane w / 4 (H_c is stored in MFMA-fragment
    // order, tile (n tile, column tile) at (n tile * D/16 + column tile) * 1 KB, so
    // block blk's 16 rows of H_c are 4 KB per plane).  Lane i's 16 bytes land at
    // the instruction's base + 16 i.  The per-lane byte offsets are one VGPR each;
    // the block and piece parts, which never move a read past the row or tile it
    // starts in, go in the instructions' scalar offsets.
    const uint32_t stage_voff = [&] {
        const int u = w * 64 + lane;  // physical 16-byte piece within a plane
        const int row = u >> 2, pc = u & 3;
        return ((uint32_t)row * sN + 4 * swz(row, pc)) * 4;
    }();
    auto stage = [&](const Ctx& x, int blk, float* dst) {
        const void* const src[4] = {a.c_re, a.c_im, a.b_re, a.b_im};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const BufRes r = make_buf(static_cast<const float*>(src[p]) + x.row0 * N, x.extN * 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(dst + p * PL + w * 256), 16,
                                                     stage_voff, NB * blk * 4, 0, 0);
        }
        const float* const hsrc = (w >> 2) ? a.hc_im : a.hc_re;
        const BufRes rh = make_buf(hsrc + x.chunk * (int64_t)N * D, N * D * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rh, (LdsPtr)(dst + 4 * PL + (w >> 2) * HP + (w & 3) * 256), 16, 16 * lane,
            (blk * HP + (w & 3) * 256) * 4, 0, 0);
    };
    // the chunk's fp64 cumsums and exp(acs): waves 0-3 one 1 KB slot each
    auto stage_aux = [&](const Ctx& x) {
        if (w < 4) {
            const void* src = w == 0 ? (const void*)(a.acs_re + x.pbase)
                              : w == 1 ? (const void*)(a.acs_im + x.pbase)
                              : w == 2 ? (const void*)(a.e_re + x.pbase)
                                       : (const void*)(a.e_im + x.pbase);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_buf(src, (w < 2 ? 8 : 4) * C),
                                                     (LdsPtr)(lda + 256 * w), 16, 16 * lane, 0, 0, 0);
        }
    };
    // operand rows 16 t + li of a staged plane, this lane's 16-byte piece g; the
    // swizzle depends on the row only through li, so one lane offset serves every
    // tile (kept opaque per block, so that the compiler forms the few addresses
    // a block needs instead of holding all of them across the chunk loop)
    const int lane_off = li * NB + 4 * swz(li, g);
    auto row4 = [&](const float* plane, int t, int lo) -> floatx4 {
        return *reinterpret_cast<const floatx4*>(plane + t * 16 * NB + lo);
    };
    // the skip weight through the scalar cache (uniform, read-only)
    auto skip_of = [&](int h) -> float {
        typedef const __attribute__((address_space(4))) float* ConstF;
        return a.dskip != nullptr ? ((ConstF)a.dskip)[h] : 0.f;
    };
    // per-lane byte offset of (row 4 g, column 16 ct + li) in a [row][D] plane
    const uint32_t dvo = ((uint32_t)(4 * g) * sD + 16 * ct + li) * 4;

    int64_t chunk = blockIdx.x;
    if (chunk >= a.nchunks) return;  // workgroup-uniform
    Ctx cur = ctx_of(chunk);
    stage(cur, 0, ls0);
    stage(cur, 1, ls1);
    // the previous chunk's outputs, stored during the next chunk's first block:
    // register r <-> row 16 rows[i] + 4 g + r, column 16 ct + li
    float yp_r[4][4], yp_i[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) yp_r[i][r] = yp_i[i][r] = 0.f;
    Ctx prev = cur;
    bool first = true;
    // the stores of the previous chunk's outputs (before the first chunk, the same
    // 32 stores per wave go through views of extent 0 and are dropped, so that the
    // count of memory operations in flight is the same on every pass; padded rows
    // of a partial chunk are dropped likewise)
    auto store_prev = [&]() {
        const uint32_t ext = first ? 0u : prev.extD * 4;
        const BufRes ry_r = make_buf(a.y_re + prev.row0 * D, ext);
        const BufRes ry_i = make_buf(a.y_im + prev.row0 * D, ext);
        uint32_t vo0 = dvo;
        asm volatile("" : "+v"(vo0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t vo = vo0 + (uint32_t)(rows[i] * 16 + r) * sD * 4;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yp_r[i][r]), ry_r, vo, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yp_i[i][r]), ry_i, vo, 0, 0);
            }
        }
    };

    for (;;) {
        CTile acc[4];  // Y_off, then y
#pragma unroll
        for (int i = 0; i < 4; ++i) ctile_zero(acc[i]);
        CTile gt[MQ];  // G^T of the owned score tiles
#pragma unroll
        for (int j = 0; j < MQ; ++j) ctile_zero(gt[j]);
        float xr[NLT][4], xi[NLT][4];  // the wave's columns of X (loaded from block 7 on)
        // X[16 st + 4 g + r][16 ct + li] for st in [st0, st1)
        auto load_x = [&](int st0, int st1) {
            const BufRes rx_r = make_buf(static_cast<const float*>(a.x_re) + cur.row0 * D, cur.extD * 4);
            const BufRes rx_i = make_buf(static_cast<const float*>(a.x_im) + cur.row0 * D, cur.extD * 4);
            uint32_t vo0 = dvo;
            asm volatile("" : "+v"(vo0));
#pragma unroll
            for (int st = st0; st < st1; ++st)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t vo = vo0 + (uint32_t)(st * 16 + r) * sD * 4;
                    xr[st][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx_r, vo, 0, 0));
                    xi[st][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx_i, vo, 0, 0));
                }
        };

        // Vector-memory operations of this wave in flight at the top of block k, in
        // issue order, after block k's staged loads:
        //   k = 0: block 1 (LPB)
        //   k = 1: the cumsum tables (waves 0-3, one), block 2 (LPB), the previous
        //          chunk's 32 stores
        //   k = 2: the stores, block 3 (LPB)
        //   k = 3..6: block k + 1 (LPB)
        //   k = 7: nothing
        // Waiting down to that count completes block k (every wave's part of it,
        // after the barrier).
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
            if (blk == 1 || blk == 2)
                __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(LPB + 32, 0));
            else if (blk + 1 < NBLK)
                __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(LPB, 0));
            else
                __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(0, 0));
            barrier_no_fence();  // block blk is in; every wave is done with block blk - 1
            const float* const bc = buf_of(blk);
            int lo = lane_off;
            asm volatile("" : "+v"(lo));
            if (blk == 0) stage_aux(cur);
            if (blk + 2 < NBLK) stage(cur, blk + 2, buf_of(blk + 2));
            if (blk == 0) store_prev();
            if (blk == NBLK - 1) load_x(0, NLT / 2);
            // Y_off += C[:, blk] H_c[blk, cols]
            {
                const floatx4 hr = *reinterpret_cast<const floatx4*>(bc + 4 * PL + ct * 256 + 4 * lane);
                const floatx4 hi =
                    *reinterpret_cast<const floatx4*>(bc + 4 * PL + HP + ct * 256 + 4 * lane);
                const floatx4 hs = hr + hi;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const floatx4 cr = row4(bc, rows[i], lo), ci = row4(bc + PL, rows[i], lo);
                    const floatx4 cs = cr + ci;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ctile_mac(acc[i], cr[e], ci[e], cs[e], hr[e], hi[e], hs[e]);
                }
            }
            // G^T += B[s tile, blk] C[l tile, blk]^T
#pragma unroll
            for (int j = 0; j < MQ; ++j) {
                if (j < nq) {  // wave-uniform
                    const int lt = own_lt[j], st = own_st[j];
                    const floatx4 br = row4(bc + 2 * PL, st, lo), bi = row4(bc + 3 * PL, st, lo);
                    const floatx4 cr = row4(bc, lt, lo), ci = row4(bc + PL, lt, lo);
                    const floatx4 bs = br + bi, cs = cr + ci;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ctile_mac(gt[j], br[e], bi[e], bs[e], cr[e], ci[e], cs[e]);
                }
            }
        }

        // ---- chunk epilogue
        // accumulator register r <-> row l = 16 lt + 4 g + r: times exp(acs[l]), back
        // in Gauss form (t1 = re, t2 = 0, t3 = re + im)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const floatx4 er = *reinterpret_cast<const floatx4*>(le_r + rows[i] * 16 + 4 * g);
            const floatx4 ei = *reinterpret_cast<const floatx4*>(le_i + rows[i] * 16 + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float re = ctile_re(acc[i], r), im = ctile_im(acc[i], r);
                const float nr = er[r] * re - ei[r] * im;
                const float ni = er[r] * im + ei[r] * re;
                acc[i].t1[r] = nr;
                acc[i].t2[r] = 0.f;
                acc[i].t3[r] = nr + ni;
            }
        }
        // M = G . L (+ Dskip on the diagonal) into LDS; register r <-> (l = l0 + li,
        // s = s0 + 4 g + r).  The M region was last read as block 5's buffer.
        const float dk = skip_of(cur.h);
#pragma unroll
        for (int j = 0; j < MQ; ++j) {
            if (j < nq) {
                const int lt = own_lt[j], st = own_st[j];
                const int lrow = lt * 16 + li;
                const bool diag = (lt == st);
                const double alr = lacs_r[lrow], ali = lacs_i[lrow];
                floatx4 mr, mi;
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
                    mr[r] = gr * lr - gi * lim + ((diag && s == lrow) ? dk : 0.f);
                    mi[r] = gr * lim + gi * lr;
                }
                const int q = q0 + j;
                *reinterpret_cast<floatx4*>(ldm + (2 * q) * 256 + 4 * lane) = mr;
                *reinterpret_cast<floatx4*>(ldm + (2 * q + 1) * 256 + 4 * lane) = mi;
            }
        }
        load_x(NLT / 2, NLT);
        // the next chunk's first two blocks, while the products below run (block 0
        // goes to buffer 0, block 6's; block 1 to buffer 1 once every wave is done
        // with block 7)
        const int64_t next = chunk + gridDim.x;
        const bool more = next < a.nchunks;  // workgroup-uniform
        Ctx nx = cur;
        if (more) {
            nx = ctx_of(next);
            stage(nx, 0, ls0);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(63, 0));
        barrier_no_fence();  // the M tiles are in
        if (more) stage(nx, 1, ls1);
        // Y_diag: y[lt] += M(lt, st) X[st rows, this wave's columns]
#pragma unroll
        for (int st = 0; st < NLT; ++st) {
            float xs[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) xs[r] = xr[st][r] + xi[st][r];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int lt = rows[i];
                if (st <= lt) {  // wave-uniform
                    const int q = lt * (lt + 1) / 2 + st;
                    const floatx4 mr = *reinterpret_cast<const floatx4*>(ldm + (2 * q) * 256 + 4 * lane);
                    const floatx4 mi =
                        *reinterpret_cast<const floatx4*>(ldm + (2 * q + 1) * 256 + 4 * lane);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        ctile_mac(acc[i], mr[r], mi[r], mr[r] + mi[r], xr[st][r], xi[st][r], xs[r]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                yp_r[i][r] = ctile_re(acc[i], r);
                yp_i[i][r] = ctile_im(acc[i], r);
            }
        prev = cur;
        first = false;
        if (!more) break;
        chunk = next;
        cur = nx;
    }
    store_prev();  // the last chunk's outputs
}

template <int C, int N, int D>
hipError_t launch_chunk_scan_wide(const FwdArgs& f, hipStream_t s) {
    ScanArgs a;
    a.x_re = f.x_re; a.x_im = f.x_im; a.b_re = f.b_re; a.b_im = f.b_im;
    a.c_re = f.c_re; a.c_im = f.c_im; a.dskip = f.dskip;
    a.acs_re = f.acs_re; a.acs_im = f.acs_im; a.e_re = f.e_re; a.e_im = f.e_im;
    a.hc_re = f.st_re; a.hc_im = f.st_im; a.y_re = f.y_re; a.y_im = f.y_im;
    a.T = f.T; a.H = (int)f.H; a.nC = (int)f.nC;
    a.nchunks = f.B * f.H * f.nC;
    int cus = 0;
    const hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
    const int64_t grid = a.nchunks < cus ? a.nchunks : cus;
    hipLaunchKernelGGL((k_chunk_scan_wide<C, N, D>), dim3((unsigned)grid), dim3(512), 0, s, a);
    return hipGetLastError();
}

}  // namespace cssd
