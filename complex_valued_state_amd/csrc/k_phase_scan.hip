// The per-coordinate complex scan of the phase-state paper ("Complex Phase-State
// Dynamics Reduce the Optimization Steps of Sequence Models", section 5.2,
// eq. 2-3):
//   lambda_t = (1 + i phi_t) / (1 - i phi_t),  alpha_t = sigmoid(u_t),
//   psi_t    = alpha_t lambda_t psi_{t-1} + b_t       for every coordinate
// Each coordinate has its own transition, so there is no matrix product to map
// onto the matrix cores: this is a memory-bound scan over independent
// coordinates, 16 bytes read and 8 written per coordinate and step.
//
// Evaluation.  Time is cut into segments of L steps (section 5.3 evaluates the
// same trajectory chunk by chunk, each chunk's end state seeding the next):
//  1. k_phase_summary: per (b, segment, coordinate), the segment's total factor
//     P = prod a_t and its end state from zero S;
//  2. k_phase_carry: per (b, coordinate), the segment-entry states
//     psi_in[c+1] = P_c psi_in[c] + S_c from psi_0, and psi_T;
//  3. k_phase_out: per (b, segment, coordinate), the recurrence from psi_in[c],
//     writing every state.
// With one segment (L >= T) only k_phase_out runs, straight from psi_0, and it
// writes psi_T itself: the inputs are read once.  That is the choice whenever
// batch x coordinates alone fill the chip; shorter segments buy parallelism for
// small batches at the cost of a second read of the inputs.
//
// Within a segment the recurrence runs forward step by step in fp32, so no
// reciprocal of a cumulative product is formed and the page's clamp of the
// log-cumsum (which only guards that reciprocal) has nothing to guard: the result
// is the exact trajectory up to rounding.  Threads of a wave take consecutive
// coordinates of one (b, segment), so each load or store of a wave is one
// contiguous 256-byte run; each thread keeps the next 8 steps' inputs in flight
// while it computes the current 8 (double-buffered registers), which is what
// hides HBM latency at one wave per SIMD (deeper blocks of 12 to 32 steps
// measured no faster).
#include "cssd_device.h"
#include "cssd_launch.h"

namespace cssd {

namespace {

constexpr int kPhaseU = 8;  // steps per prefetch block

// Every input is read once and every state written once per launch: streaming
// (non-temporal) loads and stores keep them from displacing other lines in the
// caches.  Measured on the 256 x 1024 x 16 x 16 layer: 5.0 TB/s with ordinary
// accesses, 5.6 TB/s with these.
__device__ __forceinline__ float get(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void put(float* p, float v) { __builtin_nontemporal_store(v, p); }

// a = sigmoid(u) (1 + i phi) / (1 - i phi).  With q = phi (|phi| <= 1) or 1/phi
// (|phi| > 1): lambda = (+-(1 - q^2) + 2 i q) / (1 + q^2), the sign + for
// |phi| <= 1, which stays finite for every finite phi.
__device__ __forceinline__ void phase_coeff(float phi, float u, float& ar, float& ai) {
    const bool big = fabsf(phi) > 1.f;
    const float q = big ? __builtin_amdgcn_rcpf(phi) : phi;
    const float alpha = __builtin_amdgcn_rcpf(1.f + __expf(-u));
    const float s = alpha * __builtin_amdgcn_rcpf(1.f + q * q);
    const float re = s * (1.f - q * q);
    ar = big ? -re : re;
    ai = s * (2.f * q);
}

// Inputs of kPhaseU consecutive steps of one coordinate.
struct Block {
    float phi[kPhaseU], u[kPhaseU], br[kPhaseU], bi[kPhaseU];
};

// Loads steps [t, t + kPhaseU) at offset `at` (of step t), stride `hn`.  The
// caller clamps `at` to a block that lies inside the segment.
__device__ __forceinline__ void load_block(Block& k, const PhaseArgs& a, int64_t at) {
#pragma unroll
    for (int j = 0; j < kPhaseU; ++j) {
        const int64_t o = at + j * a.HN;
        k.phi[j] = get(a.phi + o);
        k.u[j] = get(a.u + o);
        k.br[j] = get(a.b_re + o);
        k.bi[j] = get(a.b_im + o);
    }
}

// Runs the recurrence over steps [t0, t1) of coordinate (b, k) from (hr, hi).
// WRITE: store each state to psi.  PROD: also accumulate the product of the
// coefficients in (pr, pi).
template <bool WRITE, bool PROD>
__device__ __forceinline__ void scan_segment(const PhaseArgs& a, int64_t base, int64_t n,
                                             float& hr, float& hi, float& pr, float& pi) {
    const int64_t nblk = n / kPhaseU;
    int64_t at = base;
    if (nblk > 0) {
        Block cur, nxt;
        load_block(cur, a, at);
        for (int64_t i = 0; i < nblk; ++i) {
            // prefetch the next block, or reload this one on the last pass
            const int64_t nat = i + 1 < nblk ? at + kPhaseU * a.HN : at;
            load_block(nxt, a, nat);
#pragma unroll
            for (int j = 0; j < kPhaseU; ++j) {
                float cr, ci;
                phase_coeff(cur.phi[j], cur.u[j], cr, ci);
                const float nr = cr * hr - ci * hi + cur.br[j];
                const float ni = cr * hi + ci * hr + cur.bi[j];
                hr = nr;
                hi = ni;
                if (WRITE) {
                    put(a.psi_re + at + j * a.HN, hr);
                    put(a.psi_im + at + j * a.HN, hi);
                }
                if (PROD) {
                    const float qr = cr * pr - ci * pi;
                    const float qi = cr * pi + ci * pr;
                    pr = qr;
                    pi = qi;
                }
            }
            cur = nxt;
            at = nat;
        }
        at = base + nblk * kPhaseU * a.HN;
    }
    for (int64_t j = nblk * kPhaseU; j < n; ++j, at += a.HN) {
        float cr, ci;
        phase_coeff(get(a.phi + at), get(a.u + at), cr, ci);
        const float nr = cr * hr - ci * hi + get(a.b_re + at);
        const float ni = cr * hi + ci * hr + get(a.b_im + at);
        hr = nr;
        hi = ni;
        if (WRITE) {
            put(a.psi_re + at, hr);
            put(a.psi_im + at, hi);
        }
        if (PROD) {
            const float qr = cr * pr - ci * pi;
            const float qi = cr * pi + ci * pr;
            pr = qr;
            pi = qi;
        }
    }
}

}  // namespace

__global__ __launch_bounds__(256) void k_phase_summary(PhaseArgs a) {
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (tid >= a.B * a.nch * a.HN) return;
    const int64_t k = tid % a.HN;
    const int64_t c = (tid / a.HN) % a.nch;
    const int64_t b = tid / (a.HN * a.nch);
    const int64_t t0 = c * a.L;
    const int64_t n = min<int64_t>(a.L, a.T - t0);
    float sr = 0.f, si = 0.f, pr = 1.f, pi = 0.f;
    scan_segment<false, true>(a, (b * a.T + t0) * a.HN + k, n, sr, si, pr, pi);
    a.p_re[tid] = pr;  // tid = (b * nch + c) * HN + k
    a.p_im[tid] = pi;
    a.s_re[tid] = sr;
    a.s_im[tid] = si;
}

__global__ __launch_bounds__(256) void k_phase_carry(PhaseArgs a) {
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (tid >= a.B * a.HN) return;
    const int64_t k = tid % a.HN, b = tid / a.HN;
    float hr = a.psi0_re != nullptr ? a.psi0_re[tid] : 0.f;
    float hi = a.psi0_im != nullptr ? a.psi0_im[tid] : 0.f;
    int64_t w = b * a.nch * a.HN + k;
    for (int64_t c = 0; c < a.nch; ++c, w += a.HN) {
        a.in_re[w] = hr;
        a.in_im[w] = hi;
        const float pr = a.p_re[w], pi = a.p_im[w];
        const float nr = pr * hr - pi * hi + a.s_re[w];
        const float ni = pr * hi + pi * hr + a.s_im[w];
        hr = nr;
        hi = ni;
    }
    if (a.psiT_re != nullptr) {
        a.psiT_re[tid] = hr;
        a.psiT_im[tid] = hi;
    }
}

__global__ __launch_bounds__(256) void k_phase_out(PhaseArgs a) {
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (tid >= a.B * a.nch * a.HN) return;
    const int64_t k = tid % a.HN;
    const int64_t c = (tid / a.HN) % a.nch;
    const int64_t b = tid / (a.HN * a.nch);
    const int64_t t0 = c * a.L;
    const int64_t n = min<int64_t>(a.L, a.T - t0);
    float hr, hi;
    if (a.nch == 1) {  // one segment: start from psi_0 (tid = b * HN + k)
        hr = a.psi0_re != nullptr ? a.psi0_re[tid] : 0.f;
        hi = a.psi0_im != nullptr ? a.psi0_im[tid] : 0.f;
    } else {
        hr = a.in_re[tid];
        hi = a.in_im[tid];
    }
    float pr = 1.f, pi = 0.f;
    scan_segment<true, false>(a, (b * a.T + t0) * a.HN + k, n, hr, hi, pr, pi);
    if (a.nch == 1 && a.psiT_re != nullptr) {
        a.psiT_re[tid] = hr;
        a.psiT_im[tid] = hi;
    }
}

hipError_t launch_phase_summary(const PhaseArgs& a, hipStream_t s) {
    const int64_t units = a.B * a.nch * a.HN;
    hipLaunchKernelGGL(k_phase_summary, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_phase_carry(const PhaseArgs& a, hipStream_t s) {
    const int64_t units = a.B * a.HN;
    hipLaunchKernelGGL(k_phase_carry, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_phase_out(const PhaseArgs& a, hipStream_t s) {
    const int64_t units = a.B * a.nch * a.HN;
    hipLaunchKernelGGL(k_phase_out, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace cssd
