// The chunk end states and the chunk-to-chunk pass of the forward, fused:
//
//   S_c = (diag(w) B)^T X   over the rows of chunk c   (the chunk-state kernel)
//   H_0 = h0 (or 0);  H_{c+1} = cd[c] H_c + S_c;  hT = H_{nC}
//
// (Mamba-3-Lite docs, "SSD Theory" 4.5, and "The Chunkwise Complex SSD
// Algorithm" 4.5: the per-chunk states einsum, then the recurrence over the
// T/C chunk boundaries, evaluated in that sequential form).  The separate
// kernels write every S_c to memory and read it back to form H_c; here one wave
// owns one 16 x 16 tile (n, p) of the state of one (b, h) and walks the chunks
// in order, so S_c lives only in the wave's accumulator and H in its
// registers (a wave owns up to two tiles p of one n).  What is written is
// exactly what the output kernel reads: the
// carry-in state H_c of every chunk (MFMA-fragment order, the accumulator
// layout itself, one contiguous 1 KB float4 store per tile), and hT.
//
// Mapping as in the chunk-state kernel: step j of the 16x16x4 MFMA contracts
// time l = (C/4) g + j (g = lane/16); B and X are read with lane%16 along their
// contiguous axis through per-chunk buffer views whose extent ends at the
// chunk's last real row (padded rows read as zero).  For bf16 inputs with two
// p tiles per wave a lane reads two adjacent X columns in one 4-byte load, so
// a wave's X row segment is one 64-byte piece instead of two 32-byte ones;
// tile q then holds the columns p = 16 pt0 + 2 (lane%16) + q, and each store
// puts the values back in their fragment slots (measured at B8 T2048 H48 N64
// D64 C64, before that shape moved to k_state_scan_mm: 0.45 -> 0.42 ms, with 8
// k-steps in flight).  For fp32 inputs the
// paired 8-byte load measured slower (0.38 -> 0.41 ms) and is off.  The
// operands (B and X) of the next DIST k-steps are kept in flight in a register
// ring that runs on across chunk boundaries.  All workgroups of one (b, h) go to
// the same XCD (dispatch is round-robin over the 8 XCDs), so the B and X rows
// that several waves of that (b, h) read are fetched into one L2.
#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

namespace {

constexpr int kScanXcds = 8;

// k-steps whose operands are in flight (a divisor of C/4), and whether a lane
// reads two adjacent X columns in one load, per input type
template <typename In>
struct ScanTune {
    static constexpr int dist = 4;
    static constexpr bool pair = false;
};
template <>
struct ScanTune<InBF16> {
    static constexpr int dist = 8;
    static constexpr bool pair = true;
};

}  // namespace

// A wave owns PW consecutive 16-column tiles p of one 16-row tile n (operand
// reuse: the B row segment serves all PW tiles).  The weights w of the current
// chunk sit in a wave-private LDS slot (16 lanes read the same weight: a
// broadcast), refilled once per chunk from registers loaded a chunk ahead.
template <typename In, int C, int PW>
__global__ __launch_bounds__(256) void k_state_scan(
    const typename In::T* __restrict__ x_re, const typename In::T* __restrict__ x_im,
    const typename In::T* __restrict__ b_re, const typename In::T* __restrict__ b_im,
    const float* __restrict__ w_re, const float* __restrict__ w_im,
    const float* __restrict__ cd_re, const float* __restrict__ cd_im,
    const float* __restrict__ h0_re, const float* __restrict__ h0_im, float* __restrict__ st_re,
    float* __restrict__ st_im, float* __restrict__ hT_re, float* __restrict__ hT_im, int64_t T,
    int H, int N, int D, int nC, int64_t nbh) {
    constexpr int KJ = C / 4;  // MFMA k-steps per chunk
    constexpr int DIST = ScanTune<In>::dist;
    constexpr bool PAIR = PW == 2 && ScanTune<In>::pair;
    constexpr int RING = DIST < KJ ? DIST : KJ;
    constexpr int WPL = (C + 63) / 64;  // weights per lane and plane when loading a chunk's w
    // per wave: w re, w im of the current chunk, each in four groups of KJ steps (the
    // k-steps of lane group g) padded to KJ + 1, so that the four addresses a step
    // reads fall in distinct banks at C = 128 too
    __shared__ float lds_w[4][2 * 4 * (C / 4 + 1)];
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int wv = wave_id();
    const int NK = N / 16, PT = D / 16, units = NK * (PT / PW);
    // work item: (b, h, unit).  With at least 4 units per (b, h) a workgroup
    // takes 4 units of one (b, h), and the workgroups of one (b, h) share an XCD.
    int64_t bh;
    int unit;
    if (units >= 4) {
        const int per = units / 4;  // workgroups per (b, h)
        const int64_t x = blockIdx.x % kScanXcds, y = blockIdx.x / kScanXcds;
        bh = (y / per) * kScanXcds + x;
        unit = (int)(y % per) * 4 + wv;
    } else {
        const int64_t u = (int64_t)blockIdx.x * 4 + wv;
        bh = u / units;
        unit = (int)(u % units);
    }
    if (bh >= nbh) return;  // wave-uniform; the kernel has no barriers
    const int nt = unit / (PT / PW), pt0 = (unit % (PT / PW)) * PW;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const uint32_t sN = (uint32_t)H * N, sD = (uint32_t)H * D;
    float* const lw = lds_w[wv];

    // carried state, tile q register r <-> (n = 16 nt + 4g + r, p = pcol(q))
    auto pcol = [&](int q) { return PAIR ? 16 * pt0 + 2 * li + q : 16 * (pt0 + q) + li; };
    const int64_t sbase = (bh * N + nt * 16 + 4 * g) * (int64_t)D;
    float hr[PW][4], hi[PW][4];
#pragma unroll
    for (int q = 0; q < PW; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hr[q][r] = h0_re != nullptr ? h0_re[sbase + r * D + pcol(q)] : 0.f;
            hi[q][r] = h0_im != nullptr ? h0_im[sbase + r * D + pcol(q)] : 0.f;
        }

    struct Ops {
        float br, bi, xr[PW], xi[PW];
    };
    // operands of k-step j of chunk c (c < nC)
    auto load = [&](int c, int j, Ops& o) {
        const int64_t t0 = (int64_t)c * C;
        const int valid = (int)min<int64_t>((int64_t)C, T - t0);
        const int64_t row0 = (b * T + t0) * H + h;
        const uint32_t extN = (uint32_t)(valid - 1) * sN + N, extD = (uint32_t)(valid - 1) * sD + D;
        const BufRes rb_r = make_buf(b_re + row0 * N, extN * sizeof(typename In::T));
        const BufRes rb_i = make_buf(b_im + row0 * N, extN * sizeof(typename In::T));
        const BufRes rx_r = make_buf(x_re + row0 * D, extD * sizeof(typename In::T));
        const BufRes rx_i = make_buf(x_im + row0 * D, extD * sizeof(typename In::T));
        const uint32_t l = (uint32_t)(KJ * g + j);
        o.br = In::bload1(rb_r, l * sN + nt * 16 + li);
        o.bi = In::bload1(rb_i, l * sN + nt * 16 + li);
        if constexpr (PAIR) {
            const float2 vr = In::bload2(rx_r, l * sD + pt0 * 16 + 2 * li);
            const float2 vi = In::bload2(rx_i, l * sD + pt0 * 16 + 2 * li);
            o.xr[0] = vr.x;
            o.xr[1] = vr.y;
            o.xi[0] = vi.x;
            o.xi[1] = vi.y;
        } else {
#pragma unroll
            for (int q = 0; q < PW; ++q) {
                o.xr[q] = In::bload1(rx_r, l * sD + (pt0 + q) * 16 + li);
                o.xi[q] = In::bload1(rx_i, l * sD + (pt0 + q) * 16 + li);
            }
        }
    };
    // the weights of chunk c: lane takes positions lane + 64 k
    float wn_r[WPL], wn_i[WPL];
    auto load_w = [&](int c) {
#pragma unroll
        for (int k = 0; k < WPL; ++k) {
            const int pos = lane + 64 * k;
            const int64_t at = bh * (int64_t)nC * C + (int64_t)c * C + pos;
            wn_r[k] = pos < C ? w_re[at] : 0.f;
            wn_i[k] = pos < C ? w_im[at] : 0.f;
        }
    };

    Ops ring[RING];
#pragma unroll
    for (int j = 0; j < RING; ++j) load(0, j, ring[j]);
    load_w(0);

    // tile q's place within one chunk's N x D block: fragment (nt, p/16), lane p%16 + 16g
    // (with paired columns a tile's store covers every other 16-byte slot of two fragments)
    int64_t slot[PW];
#pragma unroll
    for (int q = 0; q < PW; ++q)
        slot[q] = ((int64_t)nt * PT + pcol(q) / 16) * 256 + 4 * (pcol(q) % 16 + 16 * g);
    for (int c = 0; c < nC; ++c) {
        // carry-in state of chunk c
        {
            const int64_t off = (bh * nC + c) * (int64_t)N * D;
#pragma unroll
            for (int q = 0; q < PW; ++q) {
                *reinterpret_cast<floatx4*>(st_re + off + slot[q]) =
                    floatx4{hr[q][0], hr[q][1], hr[q][2], hr[q][3]};
                *reinterpret_cast<floatx4*>(st_im + off + slot[q]) =
                    floatx4{hi[q][0], hi[q][1], hi[q][2], hi[q][3]};
            }
        }
        // this chunk's weights into the wave's LDS slot, the next chunk's into registers
#pragma unroll
        for (int k = 0; k < WPL; ++k) {
            const int pos = lane + 64 * k;
            if (pos < C) {
                lw[pos + pos / KJ] = wn_r[k];
                lw[4 * (KJ + 1) + pos + pos / KJ] = wn_i[k];
            }
        }
        if (c + 1 < nC) load_w(c + 1);
        const float dr = cd_re[bh * nC + c], di = cd_im[bh * nC + c];
        CTile acc[PW];
#pragma unroll
        for (int q = 0; q < PW; ++q) ctile_zero(acc[q]);
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const Ops o = ring[j % RING];
            // refill this slot with the operands RING steps ahead
            const int jn = j + RING;
            if (jn < KJ)
                load(c, jn, ring[j % RING]);
            else if (c + 1 < nC)  // wave-uniform
                load(c + 1, jn - KJ, ring[j % RING]);
            __builtin_amdgcn_sched_barrier(0);
            const float wr = lw[(KJ + 1) * g + j], wi = lw[4 * (KJ + 1) + (KJ + 1) * g + j];
            const float pr = wr * o.br - wi * o.bi;  // (w B)[l, n]
            const float pi = wr * o.bi + wi * o.br;
            const float ps = pr + pi;
#pragma unroll
            for (int q = 0; q < PW; ++q) ctile_mac(acc[q], pr, pi, ps, o.xr[q], o.xi[q], o.xr[q] + o.xi[q]);
        }
        // H_{c+1} = cd[c] H_c + S_c
#pragma unroll
        for (int q = 0; q < PW; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float nr = dr * hr[q][r] - di * hi[q][r] + ctile_re(acc[q], r);
                const float ni = dr * hi[q][r] + di * hr[q][r] + ctile_im(acc[q], r);
                hr[q][r] = nr;
                hi[q][r] = ni;
            }
    }
    if (hT_re != nullptr) {
#pragma unroll
        for (int q = 0; q < PW; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hT_re[sbase + r * D + pcol(q)] = hr[q][r];
                hT_im[sbase + r * D + pcol(q)] = hi[q][r];
            }
    }
}

// The same scan with the chunks dealt to four waves, for problems whose (b, h)
// count leaves the plain form with about one wave per SIMD or fewer (each wave
// there waits on its own operand stream with nothing to overlap).  A workgroup
// of four waves owns one unit (PW tiles) of one (b, h).  In round r wave k
// forms S_c of chunk c = 4 r + k with the plain form's k-step loop (operands in
// a register ring that runs on to chunk c + 4); the four S_c meet in LDS, and
// every wave then runs the round's four steps H_{c+1} = cd[c] H_c + S_c on its
// copy of the carried state, storing the carry-in of its own chunk.  The state
// stays in registers and the four copies stay identical (the same operations
// in the same order).  The workgroups of one (b, h) share an XCD as above.
template <typename In, int C, int PW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_state_scan_cp(
    const typename In::T* __restrict__ x_re, const typename In::T* __restrict__ x_im,
    const typename In::T* __restrict__ b_re, const typename In::T* __restrict__ b_im,
    const float* __restrict__ w_re, const float* __restrict__ w_im,
    const float* __restrict__ cd_re, const float* __restrict__ cd_im,
    const float* __restrict__ h0_re, const float* __restrict__ h0_im, float* __restrict__ st_re,
    float* __restrict__ st_im, float* __restrict__ hT_re, float* __restrict__ hT_im, int64_t T,
    int H, int N, int D, int nC, int64_t nbh) {
    constexpr int KJ = C / 4;  // MFMA k-steps per chunk
    constexpr int DIST = ScanTune<In>::dist;
    constexpr int RING = DIST < KJ ? DIST : KJ;
    constexpr int WPL = (C + 63) / 64;
    constexpr int SPLIT = 4;  // chunks per round = waves per workgroup
    static_assert(!(PW == 2 && ScanTune<In>::pair), "paired X columns are not used here");
    __shared__ float lds_w[SPLIT][2 * 4 * (C / 4 + 1)];  // per wave: w of its current chunk (padded as above)
    __shared__ floatx4 lds_s[2][SPLIT][2 * PW][64];      // [round parity][wave][tile re/im][lane]
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int wv = wave_id();
    const int NK = N / 16, PT = D / 16, units = NK * (PT / PW);
    const int64_t xcd = blockIdx.x % kScanXcds, y = blockIdx.x / kScanXcds;
    const int64_t bh = (y / units) * kScanXcds + xcd;
    const int unit = (int)(y % units);
    if (bh >= nbh) return;  // workgroup-uniform
    const int nt = unit / (PT / PW), pt0 = (unit % (PT / PW)) * PW;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const uint32_t sN = (uint32_t)H * N, sD = (uint32_t)H * D;
    float* const lw = lds_w[wv];

    // carried state, tile q register r <-> (n = 16 nt + 4g + r, p = 16 (pt0 + q) + li)
    const int64_t sbase = (bh * N + nt * 16 + 4 * g) * (int64_t)D;
    float hr[PW][4], hi[PW][4];
#pragma unroll
    for (int q = 0; q < PW; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hr[q][r] = h0_re != nullptr ? h0_re[sbase + r * D + 16 * (pt0 + q) + li] : 0.f;
            hi[q][r] = h0_im != nullptr ? h0_im[sbase + r * D + 16 * (pt0 + q) + li] : 0.f;
        }

    struct Ops {
        float br, bi, xr[PW], xi[PW];
    };
    const uint32_t lane_b = (uint32_t)(KJ * g) * sN + nt * 16 + li;
    const uint32_t lane_x = (uint32_t)(KJ * g) * sD + pt0 * 16 + li;
    auto load = [&](int c, int j, Ops& o) {
        const int64_t t0 = (int64_t)c * C;
        const int valid = (int)min<int64_t>((int64_t)C, T - t0);
        const int64_t row0 = (b * T + t0) * H + h;
        const uint32_t extN = (uint32_t)(valid - 1) * sN + N, extD = (uint32_t)(valid - 1) * sD + D;
        const BufRes rb_r = make_buf(b_re + row0 * N, extN * sizeof(typename In::T));
        const BufRes rb_i = make_buf(b_im + row0 * N, extN * sizeof(typename In::T));
        const BufRes rx_r = make_buf(x_re + row0 * D, extD * sizeof(typename In::T));
        const BufRes rx_i = make_buf(x_im + row0 * D, extD * sizeof(typename In::T));
        // time l = KJ g + j: the lane parts of the offsets are opaque per call, so
        // that the compiler adds the step's row offset here instead of holding
        // every step's offsets in registers across the unrolled loop
        uint32_t eb = lane_b, ex = lane_x;
        asm volatile("" : "+v"(eb), "+v"(ex));
        const uint32_t db = (uint32_t)j * sN, dx = (uint32_t)j * sD;
        o.br = In::bload1(rb_r, eb + db);
        o.bi = In::bload1(rb_i, eb + db);
#pragma unroll
        for (int q = 0; q < PW; ++q) {
            o.xr[q] = In::bload1(rx_r, ex + dx + q * 16);
            o.xi[q] = In::bload1(rx_i, ex + dx + q * 16);
        }
    };
    float wn_r[WPL], wn_i[WPL];
    auto load_w = [&](int c) {
#pragma unroll
        for (int k = 0; k < WPL; ++k) {
            const int pos = lane + 64 * k;
            const int64_t at = bh * (int64_t)nC * C + (int64_t)c * C + pos;
            wn_r[k] = pos < C ? w_re[at] : 0.f;
            wn_i[k] = pos < C ? w_im[at] : 0.f;
        }
    };

    Ops ring[RING];
    if (wv < nC) {
#pragma unroll
        for (int j = 0; j < RING; ++j) load(wv, j, ring[j]);
        load_w(wv);
    }
    int64_t slot[PW];
#pragma unroll
    for (int q = 0; q < PW; ++q) slot[q] = ((int64_t)nt * PT + pt0 + q) * 256 + 4 * lane;

    for (int r0 = 0; r0 < nC; r0 += SPLIT) {
        const int par = (r0 / SPLIT) & 1;
        const int c = r0 + wv;  // this wave's chunk
        CTile acc[PW];
#pragma unroll
        for (int q = 0; q < PW; ++q) ctile_zero(acc[q]);
        if (c < nC) {  // wave-uniform
#pragma unroll
            for (int k = 0; k < WPL; ++k) {
                const int pos = lane + 64 * k;
                if (pos < C) {
                    lw[pos + pos / KJ] = wn_r[k];
                    lw[4 * (KJ + 1) + pos + pos / KJ] = wn_i[k];
                }
            }
            const int cn = c + SPLIT;  // this wave's next chunk
            if (cn < nC) load_w(cn);
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                const Ops o = ring[j % RING];
                const int jn = j + RING;
                if (jn < KJ)
                    load(c, jn, ring[j % RING]);
                else if (cn < nC)  // wave-uniform
                    load(cn, jn - KJ, ring[j % RING]);
                __builtin_amdgcn_sched_barrier(0);
                const float wr = lw[(KJ + 1) * g + j], wi = lw[4 * (KJ + 1) + (KJ + 1) * g + j];
                const float pr = wr * o.br - wi * o.bi;  // (w B)[l, n]
                const float pi = wr * o.bi + wi * o.br;
                const float ps = pr + pi;
#pragma unroll
                for (int q = 0; q < PW; ++q)
                    ctile_mac(acc[q], pr, pi, ps, o.xr[q], o.xi[q], o.xr[q] + o.xi[q]);
            }
        }
#pragma unroll
        for (int q = 0; q < PW; ++q) {
            floatx4 sr, si;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sr[r] = ctile_re(acc[q], r);
                si[r] = ctile_im(acc[q], r);
            }
            lds_s[par][wv][2 * q][lane] = sr;
            lds_s[par][wv][2 * q + 1][lane] = si;
        }
        __syncthreads();  // the round's S_c are in (and the other parity's are read)
        // the round's chunk-to-chunk steps, the same on every wave
        for (int k = 0; k < SPLIT; ++k) {
            const int ck = r0 + k;
            if (ck >= nC) break;  // workgroup-uniform
            if (k == wv) {  // carry-in state of this wave's chunk
                const int64_t off = (bh * nC + ck) * (int64_t)N * D;
#pragma unroll
                for (int q = 0; q < PW; ++q) {
                    *reinterpret_cast<floatx4*>(st_re + off + slot[q]) =
                        floatx4{hr[q][0], hr[q][1], hr[q][2], hr[q][3]};
                    *reinterpret_cast<floatx4*>(st_im + off + slot[q]) =
                        floatx4{hi[q][0], hi[q][1], hi[q][2], hi[q][3]};
                }
            }
            const float dr = cd_re[bh * nC + ck], di = cd_im[bh * nC + ck];
#pragma unroll
            for (int q = 0; q < PW; ++q) {
                const floatx4 sr = lds_s[par][k][2 * q][lane], si = lds_s[par][k][2 * q + 1][lane];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float nr = dr * hr[q][r] - di * hi[q][r] + sr[r];
                    const float ni = dr * hi[q][r] + di * hr[q][r] + si[r];
                    hr[q][r] = nr;
                    hi[q][r] = ni;
                }
            }
        }
    }
    if (hT_re != nullptr && wv == 0) {
#pragma unroll
        for (int q = 0; q < PW; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hT_re[sbase + r * D + 16 * (pt0 + q) + li] = hr[q][r];
                hT_im[sbase + r * D + 16 * (pt0 + q) + li] = hi[q][r];
            }
    }
}

// The same scan for fp32 inputs at N = D = 64, C = 64, with the B and X rows
// staged through LDS.  A workgroup (4 waves) owns half of one (b, h)'s state:
// rows n in [32 h2, 32 h2 + 32) and every column p; wave w owns the tiles
// (n tile w / 2 of the half, p tiles 2 (w % 2) and 2 (w % 2) + 1).  The rows
// of each half chunk (a stage of 32 time steps) are fetched once per
// workgroup with 16-byte loads (whole 128-byte lines) into registers, written
// to one of two LDS buffers, and read from there as MFMA operands, while the
// next two stages' loads are in flight.  Without staging the four waves
// fetched the same rows separately in 64-byte pieces: twice the L2 requests,
// and the kernel waited on L1 misses in flight (measured at B8 T2048 H48:
// 0.38 ms unstaged, 0.31 ms staged).  Within a stage, MFMA k-step j and lane group g take time
// step 4 j + g.  Rows are XOR-swizzled in 16-byte units so that the four rows
// one operand read touches fall in distinct banks.
namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kSR = 32;  // time steps per stage
__device__ __forceinline__ int swz_b(int r) { return 4 * (((r >> 1) ^ r) & 1); }  // B rows: 8 units
__device__ __forceinline__ int swz_x(int r) { return 4 * (r & 3); }               // X rows: 16 units
}  // namespace

// The adjoint mode (ADJ) serves the gradient pass: with B -> C, X -> dY and
// w -> e it walks the chunks from the last to the first,
//   R_nC = dhT (or 0);  Q_c = C^H diag(conj e) dY;  R_c = Q_c + conj(cd[c]) R_{c+1},
// stores R_{c+1} in slot c and R_0 = dh0, and with R_{c+1} in registers also
// forms the log-decay gradient's boundary term <R_{c+1}, H_{c+1}> (the forward
// state entering chunk c + 1, or hT after the last chunk), one fp64 partial per
// workgroup (half of the n rows) and chunk.
struct AdjExtra {
    const float *hs_re, *hs_im;  // forward carry-in states H_c, fragment order
    const float *hT_re, *hT_im;  // forward final state (caller's layout), or NULL
    double *z_re, *z_im;         // [(b, h, c) * 2 + half]
};

template <bool ADJ, int C, int N>
__global__ __launch_bounds__(256) void k_state_scan_lds(
    const float* __restrict__ x_re, const float* __restrict__ x_im,
    const float* __restrict__ b_re, const float* __restrict__ b_im,
    const float* __restrict__ w_re, const float* __restrict__ w_im,
    const float* __restrict__ cd_re, const float* __restrict__ cd_im,
    const float* __restrict__ h0_re, const float* __restrict__ h0_im, float* __restrict__ st_re,
    float* __restrict__ st_im, float* __restrict__ hT_re, float* __restrict__ hT_im, int64_t T,
    int H, int nC, int64_t nbh, AdjExtra adj) {
    constexpr int D = 64, PT = D / 16;
    constexpr int NQ = N / 32;   // workgroups per (b, h): 32 rows n each
    constexpr int NS = C / kSR;  // stages per chunk
    constexpr int KS = kSR / 4;  // k-steps per stage
    constexpr int WPL = C / 64;  // weights per lane when a chunk's w is loaded
    static_assert(!ADJ || (C == 64 && N == 64), "the adjoint mode is built for N = C = 64");
    __shared__ floatx4 sb[2][2][kSR * 8];   // [buffer][plane][row * 8 + unit]: 32 B columns per row
    __shared__ floatx4 sx[2][2][kSR * 16];  // [buffer][plane][row * 16 + unit]: all 64 X columns
    __shared__ float lds_w[4][2 * C];
    __shared__ double lds_z[4][2];  // ADJ: per-wave partials of the boundary term
    const int tid = threadIdx.x, lane = tid & 63;
    const int li = lane & 15, g = lane >> 4;
    const int wv = wave_id();
    const int64_t xcd = blockIdx.x % kScanXcds, y = blockIdx.x / kScanXcds;
    // each XCD takes a run of consecutive (b, h): the rows of neighbouring heads
    // are adjacent in memory (measured slightly faster than interleaving them)
    const int64_t bh = xcd * (int64_t)(gridDim.x / (NQ * kScanXcds)) + y / NQ;
    const int h2 = (int)(y % NQ);
    if (bh >= nbh) return;  // uniform over the workgroup
    const int ntl = wv >> 1, pt0 = (wv & 1) * 2, nt = 2 * h2 + ntl;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const uint32_t sN = (uint32_t)H * N, sD = (uint32_t)H * D;
    float* const lw = lds_w[wv];

    const int64_t sbase = (bh * N + nt * 16 + 4 * g) * (int64_t)D + pt0 * 16 + li;
    float hr[2][4], hi[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hr[q][r] = h0_re != nullptr ? h0_re[sbase + r * D + 16 * q] : 0.f;
            hi[q][r] = h0_im != nullptr ? h0_im[sbase + r * D + 16 * q] : 0.f;
        }

    // one stage in registers: B (this half's 32 columns) and X (64 columns), both planes
    struct StageIn {
        floatx4 b[2], x[2][2];
    };
    // B row rb, 16-byte unit ub of each plane; X rows idx / 16, units idx % 16
    const int rb = tid >> 3, ub = tid & 7;
    // the chunk of stage qs (the adjoint walks the chunks backwards)
    auto chunk_of = [&](int qs) { return ADJ ? nC - 1 - qs / NS : qs / NS; };
    auto gload = [&](int qs, StageIn& R) {
        const int c = chunk_of(qs), s = qs % NS;
        const int64_t t0 = (int64_t)c * C;
        const int valid = (int)min<int64_t>((int64_t)C, T - t0);
        const int64_t row0 = (b * T + t0) * H + h;
        const uint32_t extN = (uint32_t)(valid - 1) * sN + N, extD = (uint32_t)(valid - 1) * sD + D;
        const BufRes vb_r = make_buf(b_re + row0 * N, extN * 4u), vb_i = make_buf(b_im + row0 * N, extN * 4u);
        const BufRes vx_r = make_buf(x_re + row0 * D, extD * 4u), vx_i = make_buf(x_im + row0 * D, extD * 4u);
        const uint32_t eb = (uint32_t)(s * kSR + rb) * sN + 32 * h2 + 4 * ub;
        R.b[0] = buf_f32x4(vb_r, eb);
        R.b[1] = buf_f32x4(vb_i, eb);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int idx = tid + 256 * k, rx = idx >> 4, ux = idx & 15;
            const uint32_t ex = (uint32_t)(s * kSR + rx) * sD + 4 * ux;
            R.x[0][k] = buf_f32x4(vx_r, ex);
            R.x[1][k] = buf_f32x4(vx_i, ex);
        }
    };
    auto lstore = [&](int buf, const StageIn& R) {
        sb[buf][0][rb * 8 + (ub ^ swz_b(rb))] = R.b[0];
        sb[buf][1][rb * 8 + (ub ^ swz_b(rb))] = R.b[1];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int idx = tid + 256 * k, rx = idx >> 4, ux = idx & 15;
            sx[buf][0][rx * 16 + (ux ^ swz_x(rx))] = R.x[0][k];
            sx[buf][1][rx * 16 + (ux ^ swz_x(rx))] = R.x[1][k];
        }
    };
    float wn_r[WPL], wn_i[WPL];  // the next chunk's weights, positions lane + 64 k
    auto load_w = [&](int c) {
#pragma unroll
        for (int k = 0; k < WPL; ++k) {
            const int64_t at = (bh * nC + c) * (int64_t)C + lane + 64 * k;
            wn_r[k] = w_re[at];
            wn_i[k] = w_im[at];
        }
    };
    // per-lane operand offsets (floats) within a stage buffer; row 4 j + g adds 4 j rows
    const int offb = g * 32 + (((4 * ntl + (li >> 2)) ^ swz_b(g)) << 2) + (li & 3);
    int offx[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) offx[q] = g * 64 + (((4 * (pt0 + q) + (li >> 2)) ^ swz_x(g)) << 2) + (li & 3);

    const int total = nC * NS;  // even
    const int64_t slot = ((int64_t)nt * PT + pt0) * 256 + 4 * lane;
    CTile acc[2];
    // stage qs: Rx holds stage qs + 1, and its registers are then refilled with
    // stage qs + 3 (two stages are in flight in registers, one in each set)
    auto body = [&](int qs, StageIn& Rx) {
        const int c = chunk_of(qs), s = qs % NS, buf = qs & 1;
        __syncthreads();  // stage qs is in LDS; nobody reads the other buffer any more
        if (qs + 1 < total) lstore(buf ^ 1, Rx);
        if (qs + 3 < total) gload(qs + 3, Rx);
        if constexpr (ADJ) {
            // the partials written at this chunk's first stage are visible now
            if (s == 1 && tid == 0) {
                const int64_t zi = (bh * nC + c) * 2 + h2;
                adj.z_re[zi] = (lds_z[0][0] + lds_z[1][0]) + (lds_z[2][0] + lds_z[3][0]);
                adj.z_im[zi] = (lds_z[0][1] + lds_z[1][1]) + (lds_z[2][1] + lds_z[3][1]);
            }
        }
        if (s == 0) {
            const int64_t off = (bh * nC + c) * (int64_t)N * D + slot;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                *reinterpret_cast<floatx4*>(st_re + off + 256 * q) =
                    floatx4{hr[q][0], hr[q][1], hr[q][2], hr[q][3]};
                *reinterpret_cast<floatx4*>(st_im + off + 256 * q) =
                    floatx4{hi[q][0], hi[q][1], hi[q][2], hi[q][3]};
            }
            if constexpr (ADJ) {
                // <R_{c+1}, H_{c+1}> over this wave's two tiles, in fp64
                float vr[2][4], vi[2][4];
                if (c + 1 < nC) {
                    const int64_t hoff = (bh * nC + c + 1) * (int64_t)N * D + slot;
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const floatx4 ur = *reinterpret_cast<const floatx4*>(adj.hs_re + hoff + 256 * q);
                        const floatx4 ui = *reinterpret_cast<const floatx4*>(adj.hs_im + hoff + 256 * q);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            vr[q][r] = ur[r];
                            vi[q][r] = ui[r];
                        }
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const bool has = adj.hT_re != nullptr && h0_re != nullptr;
                            vr[q][r] = has ? adj.hT_re[sbase + r * D + 16 * q] : 0.f;
                            vi[q][r] = has ? adj.hT_im[sbase + r * D + 16 * q] : 0.f;
                        }
                }
                double zr = 0.0, zi = 0.0;
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        zr += (double)hr[q][r] * vr[q][r] + (double)hi[q][r] * vi[q][r];
                        zi += (double)hi[q][r] * vr[q][r] - (double)hr[q][r] * vi[q][r];
                    }
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) {
                    zr += __shfl_xor(zr, off, 64);
                    zi += __shfl_xor(zi, off, 64);
                }
                if (lane == 0) {
                    lds_z[wv][0] = zr;
                    lds_z[wv][1] = zi;
                }
            }
#pragma unroll
            for (int k = 0; k < WPL; ++k) {
                lw[lane + 64 * k] = wn_r[k];
                lw[C + lane + 64 * k] = wn_i[k];
            }
            if (ADJ ? c > 0 : c + 1 < nC) load_w(ADJ ? c - 1 : c + 1);
#pragma unroll
            for (int q = 0; q < 2; ++q) ctile_zero(acc[q]);
        }
        const float* const pb_r = reinterpret_cast<const float*>(sb[buf][0]) + offb;
        const float* const pb_i = reinterpret_cast<const float*>(sb[buf][1]) + offb;
        const float* const px_r = reinterpret_cast<const float*>(sx[buf][0]);
        const float* const px_i = reinterpret_cast<const float*>(sx[buf][1]);
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int l = s * kSR + 4 * j + g;
            const float wr = lw[l], wi = lw[C + l];
            const float br = pb_r[128 * j], bi = pb_i[128 * j];
            const float pr = wr * br - wi * bi;  // (w B)[l, n], conjugated in the adjoint
            const float pi = ADJ ? -(wr * bi + wi * br) : wr * bi + wi * br;
            const float ps = pr + pi;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const float xr = px_r[offx[q] + 256 * j], xi = px_i[offx[q] + 256 * j];
                ctile_mac(acc[q], pr, pi, ps, xr, xi, xr + xi);
            }
        }
        if (s == NS - 1) {
            const float dr = cd_re[bh * nC + c], di = ADJ ? -cd_im[bh * nC + c] : cd_im[bh * nC + c];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float nr = dr * hr[q][r] - di * hi[q][r] + ctile_re(acc[q], r);
                    const float ni = dr * hi[q][r] + di * hr[q][r] + ctile_im(acc[q], r);
                    hr[q][r] = nr;
                    hi[q][r] = ni;
                }
        }
    };
    load_w(ADJ ? nC - 1 : 0);
    StageIn R0, R1;
    gload(0, R0);
    lstore(0, R0);
    gload(1, R1);
    if (total > 2) gload(2, R0);
    for (int qs = 0; qs < total; qs += 2) {
        body(qs, R1);
        body(qs + 1, R0);
    }
    if (hT_re != nullptr) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hT_re[sbase + r * D + 16 * q] = hr[q][r];
                hT_im[sbase + r * D + 16 * q] = hi[q][r];
            }
    }
}

template <int C, int N>
static hipError_t launch_scan_lds(const FwdArgs& a, hipStream_t s) {
    const int64_t nbh = a.B * a.H;
    const int64_t blocks = kScanXcds * ((nbh + kScanXcds - 1) / kScanXcds) * (N / 32);
    typedef const float* P;
    const AdjExtra none = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    hipLaunchKernelGGL((k_state_scan_lds<false, C, N>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<P>(a.x_re), static_cast<P>(a.x_im), static_cast<P>(a.b_re),
                       static_cast<P>(a.b_im),
                       a.w_re, a.w_im, a.cd_re, a.cd_im, a.h0_re, a.h0_im, a.st_re, a.st_im,
                       a.hT_re, a.hT_im, a.T, (int)a.H, (int)a.nC, nbh, none);
    return hipGetLastError();
}

bool state_scan_adjoint_fused(const FwdArgs& a) {
    return a.in_dtype == 0 && a.C == 64 && a.N == 64 && a.D == 64;
}

hipError_t launch_state_scan_adjoint(const FwdArgs& a, const float* dy_re, const float* dy_im,
                                     const float* dhT_re, const float* dhT_im, float* r_re,
                                     float* r_im, float* dh0_re, float* dh0_im,
                                     const float* hT_re, const float* hT_im, double* z_re,
                                     double* z_im, hipStream_t s) {
    if (!state_scan_adjoint_fused(a)) return hipErrorNotSupported;
    const int64_t nbh = a.B * a.H;
    const int64_t blocks = kScanXcds * ((nbh + kScanXcds - 1) / kScanXcds) * 2;
    const AdjExtra adj = {a.st_re, a.st_im, hT_re, hT_im, z_re, z_im};
    hipLaunchKernelGGL((k_state_scan_lds<true, 64, 64>), dim3((unsigned)blocks), dim3(256), 0, s,
                       dy_re, dy_im, static_cast<const float*>(a.c_re),
                       static_cast<const float*>(a.c_im), a.e_re, a.e_im, a.cd_re, a.cd_im,
                       dhT_re, dhT_im, r_re, r_im, dh0_re, dh0_im, a.T, (int)a.H, (int)a.nC, nbh,
                       adj);
    return hipGetLastError();
}

// bf16 inputs at N = D = C = 64: the same scan with the chunk-state contraction
// on the bf16 matrix cores.  v_mfma_f32_16x16x32_bf16 contracts 32 time steps in
// one instruction, with lane i + 16 g holding the 8 consecutive steps 8g .. 8g+7
// of row i of each operand, so both operands are staged transposed: a row per
// feature (n of w B, p of X) over the 32 steps of a half chunk.  The weights w
// are applied while staging, in fp32, and w B is then rounded to bf16 as an
// operand (B and X are bf16 already); the products accumulate in fp32 and the
// carried state stays fp32.  A complex product is four real products with the
// imaginary A operand negated for the real part (a sum of bf16 operands would
// round).  Workgroup and wave mapping, carry-in stores and the chunk-to-chunk
// update are those of k_state_scan_lds.
namespace {
typedef __bf16 bf16x8_s __attribute__((ext_vector_type(8)));
constexpr int kRowB = 80;  // bytes per staged feature row: 32 bf16 + 16 B (distinct banks)
__device__ __forceinline__ bf16x8_s neg8(bf16x8_s v) {
    u32x4 u = __builtin_bit_cast(u32x4, v);
    u ^= 0x80008000u;
    return __builtin_bit_cast(bf16x8_s, u);
}
__device__ __forceinline__ uint32_t bf16_bits(float v) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}
}  // namespace

__global__ __launch_bounds__(256) void k_state_scan_mm(
    const uint16_t* __restrict__ x_re, const uint16_t* __restrict__ x_im,
    const uint16_t* __restrict__ b_re, const uint16_t* __restrict__ b_im,
    const float* __restrict__ w_re, const float* __restrict__ w_im,
    const float* __restrict__ cd_re, const float* __restrict__ cd_im,
    const float* __restrict__ h0_re, const float* __restrict__ h0_im, float* __restrict__ st_re,
    float* __restrict__ st_im, float* __restrict__ hT_re, float* __restrict__ hT_im, int64_t T,
    int H, int nC, int64_t nbh) {
    constexpr int C = 64, N = 64, D = 64, PT = D / 16;
    constexpr int NS = C / kSR;  // stages (of 32 steps) per chunk
    // [buffer][plane][feature row]: w B for this half's 32 n, X for all 64 p
    __shared__ __align__(16) unsigned char lds_wb[2][2][32 * kRowB];
    __shared__ __align__(16) unsigned char lds_xt[2][2][64 * kRowB];
    const int tid = threadIdx.x, lane = tid & 63;
    const int li = lane & 15, g = lane >> 4;
    const int wv = wave_id();
    const int64_t xcd = blockIdx.x % kScanXcds, y = blockIdx.x / kScanXcds;
    const int64_t bh = xcd * (int64_t)(gridDim.x / (2 * kScanXcds)) + y / 2;
    const int h2 = (int)(y % 2);
    if (bh >= nbh) return;  // uniform over the workgroup
    const int ntl = wv >> 1, pt0 = (wv & 1) * 2, nt = 2 * h2 + ntl;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const uint32_t sN = (uint32_t)H * N, sD = (uint32_t)H * D;

    const int64_t sbase = (bh * N + nt * 16 + 4 * g) * (int64_t)D + pt0 * 16 + li;
    float hr[2][4], hi[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hr[q][r] = h0_re != nullptr ? h0_re[sbase + r * D + 16 * q] : 0.f;
            hi[q][r] = h0_im != nullptr ? h0_im[sbase + r * D + 16 * q] : 0.f;
        }

    // staging items: threads 0-127 take X features 2 pp, 2 pp + 1 over the 8
    // steps 8 rg .. 8 rg + 7 (pp = tid % 32, rg = tid / 32); threads 128-191
    // take B features 32 h2 + 2 np, + 1 (np = tid % 16, rg = (tid - 128) / 16)
    const bool is_x = tid < 128, is_b = tid >= 128 && tid < 192;
    const int pp = tid & 31, np = (tid - 128) & 15;
    const int rg = is_x ? tid >> 5 : ((tid - 128) >> 4) & 3;
    struct Raw {
        uint32_t re[8], im[8];  // two features (low, high half) at 8 steps
        float wr[8], wi[8];     // B items: the weights of those steps
    };
    auto gload = [&](int qs, Raw& R) {
        const int c = qs / NS, s = qs % NS;
        const int64_t t0 = (int64_t)c * C;
        const int valid = (int)min<int64_t>((int64_t)C, T - t0);
        const int64_t row0 = (b * T + t0) * H + h;
        if (is_x) {
            const uint32_t ext = ((uint32_t)(valid - 1) * sD + D) * 2u;
            const BufRes vr = make_buf(x_re + row0 * D, ext), vi = make_buf(x_im + row0 * D, ext);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const uint32_t e = (uint32_t)(s * kSR + 8 * rg + r) * sD + 2 * pp;
                R.re[r] = __builtin_amdgcn_raw_buffer_load_b32(vr, e * 2u, 0, 0);
                R.im[r] = __builtin_amdgcn_raw_buffer_load_b32(vi, e * 2u, 0, 0);
            }
        } else if (is_b) {
            const uint32_t ext = ((uint32_t)(valid - 1) * sN + N) * 2u;
            const BufRes vr = make_buf(b_re + row0 * N, ext), vi = make_buf(b_im + row0 * N, ext);
            const int64_t wbase = (bh * nC + c) * (int64_t)C + s * kSR + 8 * rg;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const uint32_t e = (uint32_t)(s * kSR + 8 * rg + r) * sN + 32 * h2 + 2 * np;
                R.re[r] = __builtin_amdgcn_raw_buffer_load_b32(vr, e * 2u, 0, 0);
                R.im[r] = __builtin_amdgcn_raw_buffer_load_b32(vi, e * 2u, 0, 0);
                R.wr[r] = w_re[wbase + r];
                R.wi[r] = w_im[wbase + r];
            }
        }
    };
    auto lstore = [&](int buf, const Raw& R) {
        if (is_x) {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                uint32_t pr[4], pi[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t a0 = (R.re[2 * k] >> (16 * f)) & 0xffffu;
                    const uint32_t a1 = (R.re[2 * k + 1] >> (16 * f)) & 0xffffu;
                    const uint32_t b0 = (R.im[2 * k] >> (16 * f)) & 0xffffu;
                    const uint32_t b1 = (R.im[2 * k + 1] >> (16 * f)) & 0xffffu;
                    pr[k] = a0 | (a1 << 16);
                    pi[k] = b0 | (b1 << 16);
                }
                const int off = (2 * pp + f) * kRowB + 16 * rg;
                *reinterpret_cast<uint4*>(&lds_xt[buf][0][off]) = make_uint4(pr[0], pr[1], pr[2], pr[3]);
                *reinterpret_cast<uint4*>(&lds_xt[buf][1][off]) = make_uint4(pi[0], pi[1], pi[2], pi[3]);
            }
        } else if (is_b) {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                uint32_t pr[4], pi[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t ur[2], ui[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int r = 2 * k + e;
                        const float br = __uint_as_float(((R.re[r] >> (16 * f)) & 0xffffu) << 16);
                        const float bi = __uint_as_float(((R.im[r] >> (16 * f)) & 0xffffu) << 16);
                        ur[e] = bf16_bits(R.wr[r] * br - R.wi[r] * bi);  // (w B)[l, n]
                        ui[e] = bf16_bits(R.wr[r] * bi + R.wi[r] * br);
                    }
                    pr[k] = ur[0] | (ur[1] << 16);
                    pi[k] = ui[0] | (ui[1] << 16);
                }
                const int off = (2 * np + f) * kRowB + 16 * rg;
                *reinterpret_cast<uint4*>(&lds_wb[buf][0][off]) = make_uint4(pr[0], pr[1], pr[2], pr[3]);
                *reinterpret_cast<uint4*>(&lds_wb[buf][1][off]) = make_uint4(pi[0], pi[1], pi[2], pi[3]);
            }
        }
    };

    const int total = nC * NS;
    const int64_t slot = ((int64_t)nt * PT + pt0) * 256 + 4 * lane;
    floatx4 sre[2], sim[2];
    Raw R;
    gload(0, R);
    lstore(0, R);
    if (total > 1) gload(1, R);
    for (int qs = 0; qs < total; ++qs) {
        const int c = qs / NS, s = qs % NS, buf = qs & 1;
        __syncthreads();  // stage qs is in LDS; nobody reads the other buffer any more
        if (qs + 1 < total) lstore(buf ^ 1, R);
        if (qs + 2 < total) gload(qs + 2, R);
        if (s == 0) {
            const int64_t off = (bh * nC + c) * (int64_t)N * D + slot;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                *reinterpret_cast<floatx4*>(st_re + off + 256 * q) =
                    floatx4{hr[q][0], hr[q][1], hr[q][2], hr[q][3]};
                *reinterpret_cast<floatx4*>(st_im + off + 256 * q) =
                    floatx4{hi[q][0], hi[q][1], hi[q][2], hi[q][3]};
                sre[q] = floatx4{0.f, 0.f, 0.f, 0.f};
                sim[q] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
        }
        // A: (w B)^T rows n = 16 ntl + li, steps 8g .. 8g + 7; B: X^T rows p
        const int ao = (16 * ntl + li) * kRowB + 16 * g;
        const bf16x8_s ar = *reinterpret_cast<const bf16x8_s*>(&lds_wb[buf][0][ao]);
        const bf16x8_s ai = *reinterpret_cast<const bf16x8_s*>(&lds_wb[buf][1][ao]);
        const bf16x8_s nai = neg8(ai);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int xo = (16 * (pt0 + q) + li) * kRowB + 16 * g;
            const bf16x8_s xr = *reinterpret_cast<const bf16x8_s*>(&lds_xt[buf][0][xo]);
            const bf16x8_s xi = *reinterpret_cast<const bf16x8_s*>(&lds_xt[buf][1][xo]);
            sre[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar, xr, sre[q], 0, 0, 0);
            sre[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nai, xi, sre[q], 0, 0, 0);
            sim[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar, xi, sim[q], 0, 0, 0);
            sim[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ai, xr, sim[q], 0, 0, 0);
        }
        if (s == NS - 1) {
            const float dr = cd_re[bh * nC + c], di = cd_im[bh * nC + c];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float nr = dr * hr[q][r] - di * hi[q][r] + sre[q][r];
                    const float ni = dr * hi[q][r] + di * hr[q][r] + sim[q][r];
                    hr[q][r] = nr;
                    hi[q][r] = ni;
                }
        }
    }
    if (hT_re != nullptr) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hT_re[sbase + r * D + 16 * q] = hr[q][r];
                hT_im[sbase + r * D + 16 * q] = hi[q][r];
            }
    }
}

static hipError_t launch_scan_mm(const FwdArgs& a, hipStream_t s) {
    const int64_t nbh = a.B * a.H;
    const int64_t blocks = kScanXcds * ((nbh + kScanXcds - 1) / kScanXcds) * 2;
    typedef const uint16_t* P;
    hipLaunchKernelGGL(k_state_scan_mm, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<P>(a.x_re), static_cast<P>(a.x_im), static_cast<P>(a.b_re),
                       static_cast<P>(a.b_im), a.w_re, a.w_im, a.cd_re, a.cd_im, a.h0_re, a.h0_im,
                       a.st_re, a.st_im, a.hT_re, a.hT_im, a.T, (int)a.H, (int)a.nC, nbh);
    return hipGetLastError();
}

template <typename In, int C, int PW>
static hipError_t launch_scan_pw(const FwdArgs& a, hipStream_t s) {
    const int units = (int)((a.N / 16) * (a.D / 16 / PW));
    const int64_t nbh = a.B * a.H;
    int64_t blocks;
    if (units >= 4)
        blocks = kScanXcds * ((nbh + kScanXcds - 1) / kScanXcds) * (units / 4);
    else
        blocks = (nbh * units + 3) / 4;
    hipLaunchKernelGGL((k_state_scan<In, C, PW>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const typename In::T*>(a.x_re),
                       static_cast<const typename In::T*>(a.x_im),
                       static_cast<const typename In::T*>(a.b_re),
                       static_cast<const typename In::T*>(a.b_im), a.w_re, a.w_im, a.cd_re,
                       a.cd_im, a.h0_re, a.h0_im, a.st_re, a.st_im, a.hT_re, a.hT_im, a.T,
                       (int)a.H, (int)a.N, (int)a.D, (int)a.nC, nbh);
    return hipGetLastError();
}

template <int C>
static hipError_t launch_scan_cp(const FwdArgs& a, hipStream_t s) {
    const int units = (int)((a.N / 16) * (a.D / 16 / 2));
    const int64_t nbh = a.B * a.H;
    const int64_t blocks = kScanXcds * ((nbh + kScanXcds - 1) / kScanXcds) * units;
    hipLaunchKernelGGL((k_state_scan_cp<InF32, C, 2>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const float*>(a.x_re), static_cast<const float*>(a.x_im),
                       static_cast<const float*>(a.b_re), static_cast<const float*>(a.b_im),
                       a.w_re, a.w_im, a.cd_re, a.cd_im, a.h0_re, a.h0_im, a.st_re, a.st_im,
                       a.hT_re, a.hT_im, a.T, (int)a.H, (int)a.N, (int)a.D, (int)a.nC, nbh);
    return hipGetLastError();
}

// Two tiles per wave where D allows (measured at B8 T2048 H48 N64 D64 C64: one
// tile per wave 0.52 ms, two 0.38 ms, against 0.41 ms for the separate
// chunk-state and state-pass kernels).
template <typename In, int C>
static hipError_t launch_scan_c(const FwdArgs& a, hipStream_t s) {
    return a.D >= 32 ? launch_scan_pw<In, C, 2>(a, s) : launch_scan_pw<In, C, 1>(a, s);
}

template <typename In>
static hipError_t launch_scan_in(const FwdArgs& a, hipStream_t s) {
    switch (a.C) {
        case 16: return launch_scan_c<In, 16>(a, s);
        case 32: return launch_scan_c<In, 32>(a, s);
        case 64: return launch_scan_c<In, 64>(a, s);
        default: return launch_scan_c<In, 128>(a, s);
    }
}

hipError_t launch_state_scan(const FwdArgs& a, hipStream_t s) {
    if (a.C == 64 && a.N == 64 && a.D == 64)
        return a.in_dtype == 1 ? launch_scan_mm(a, s) : launch_scan_lds<64, 64>(a, s);
    // staged through LDS at N = 128, C = 64 (four workgroups per (b, h)) where the
    // problem has a workgroup for every CU: with fewer the one wave per SIMD of the
    // staged form loses to the plain scan's (measured at B1 T16384 H48 C128:
    // 0.82 ms staged against 0.71 ms)
    if (a.in_dtype == 0 && a.D == 64 && a.N == 128 && a.C == 64 && a.B * a.H * 4 >= 256)
        return launch_scan_lds<64, 128>(a, s);
    // the chunks dealt to four waves where the plain form would have fewer waves
    // than the chip has SIMDs and each sequence has several rounds of chunks
    if (a.in_dtype == 0 && a.D >= 32 && a.C == 128 && a.nC >= 8 &&
        a.B * a.H * (a.N / 16) * (a.D / 32) < 1024)
        return launch_scan_cp<128>(a, s);
    return a.in_dtype == 1 ? launch_scan_in<InBF16>(a, s) : launch_scan_in<InF32>(a, s);
}

}  // namespace cssd
