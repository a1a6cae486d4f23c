// C ABI of libcssd.so (declared in include/cssd.h): host-side validation,
// workspace layout, kernel sequencing and the optional per-kernel profiler.
// Nothing here allocates device memory, synchronises a stream or reads device
// memory; every kernel is enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <mutex>
#include <vector>

#include "cssd.h"
#include "cssd_launch.h"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool pow2_16_128(int64_t v) { return v == 16 || v == 32 || v == 64 || v == 128; }

bool aligned(const void* p, uintptr_t bytes) {
    return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0;
}

// ---------------------------------------------------------------- profiler
struct Pending {
    int kernel;
    hipEvent_t start, stop;
};

struct Profiler {
    std::mutex mu;
    bool on = false;
    std::vector<Pending> pending;
    std::vector<hipEvent_t> pool;
    double ms[cssd::K_COUNT] = {0};
    int64_t launches[cssd::K_COUNT] = {0};
};

Profiler& prof() {
    static Profiler p;
    return p;
}

hipEvent_t take_event(Profiler& p) {
    if (!p.pool.empty()) {
        hipEvent_t e = p.pool.back();
        p.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// CSSD_DEBUG_SYNC=1 in the environment (read once): after every launch the
// stream is synchronised and an asynchronous error of the kernel is returned as
// the launch's error, so a failing call names its kernel.  Off by default: the
// library otherwise never synchronises.  Streams being captured are left alone.
bool debug_sync() {
    static const bool on = [] {
        const char* v = std::getenv("CSSD_DEBUG_SYNC");
        return v != nullptr && v[0] != '\0' && v[0] != '0';
    }();
    return on;
}

hipError_t after_launch(hipStream_t stream, hipError_t err) {
    if (err != hipSuccess || !debug_sync()) return err;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
        return err;
    const hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

// Runs one launcher, bracketed by events while profiling is on.
template <typename F>
hipError_t timed(int kernel, hipStream_t stream, F&& launch_fn) {
    auto launch = [&] { return after_launch(stream, launch_fn()); };
    Profiler& p = prof();
    hipEvent_t e0 = nullptr, e1 = nullptr;
    bool on;
    {
        std::lock_guard<std::mutex> g(p.mu);
        on = p.on;
    }
    // a stream being captured into a graph gets no event brackets: they would
    // be captured with the kernels and never complete outside a replay
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (on && hipStreamIsCapturing(stream, &cap) == hipSuccess &&
        cap == hipStreamCaptureStatusNone) {
        std::lock_guard<std::mutex> g(p.mu);
        e0 = take_event(p);
        e1 = take_event(p);
    }
    // on every early return the events go back to the pool, so none is leaked
    auto give_back = [&](hipError_t err) {
        if (e0 || e1) {
            std::lock_guard<std::mutex> g(p.mu);
            if (e0) p.pool.push_back(e0);
            if (e1) p.pool.push_back(e1);
        }
        return err;
    };
    if (!(e0 && e1)) {
        give_back(hipSuccess);
        e0 = e1 = nullptr;
    }
    if (e0 && hipEventRecord(e0, stream) != hipSuccess) return give_back(hipGetLastError());
    hipError_t err = launch();
    if (err != hipSuccess) return give_back(err);
    if (e0) {
        if (hipEventRecord(e1, stream) != hipSuccess) return give_back(hipGetLastError());
        std::lock_guard<std::mutex> g(p.mu);
        p.pending.push_back(Pending{kernel, e0, e1});
    }
    return hipSuccess;
}

struct Layout {
    size_t acs_re, acs_im, e_re, e_im, w_re, w_im, cd_re, cd_im, st_re, st_im, total;
};

Layout layout(int64_t B, int64_t T, int64_t H, int64_t D, int64_t N, int64_t C) {
    const int64_t nC = (T + C - 1) / C;
    const size_t P = (size_t)(B * H * nC * C);
    const size_t S = (size_t)(B * H * nC) * (size_t)(N * D);
    Layout l;
    size_t off = 0;
    auto put = [&](size_t bytes) {
        const size_t at = off;
        off = round_up(off + bytes);
        return at;
    };
    l.acs_re = put(P * sizeof(double));
    l.acs_im = put(P * sizeof(double));
    l.e_re = put(P * sizeof(float));
    l.e_im = put(P * sizeof(float));
    l.w_re = put(P * sizeof(float));
    l.w_im = put(P * sizeof(float));
    l.cd_re = put((size_t)(B * H * nC) * sizeof(float));
    l.cd_im = put((size_t)(B * H * nC) * sizeof(float));
    l.st_re = put(S * sizeof(float));
    l.st_im = put(S * sizeof(float));
    l.total = off;
    return l;
}

// The gradient pass: the forward workspace, then its own regions.
struct BwdLayout {
    Layout fwd;
    size_t r_re, r_im, q1_re, q1_im, q2_re, q2_im, ddp, hT_re, hT_im, z_re, z_im, pa, total;
};

// bytes of the fp32 copies of bf16 x, B, C (two planes each) that cssd_backward
// widens into its workspace after the backward's own layout
size_t widen_bytes(int64_t B, int64_t T, int64_t H, int64_t D, int64_t N) {
    return 2 * round_up((size_t)(B * T * H * D) * sizeof(float)) +
           4 * round_up((size_t)(B * T * H * N) * sizeof(float));
}

BwdLayout bwd_layout(int64_t B, int64_t T, int64_t H, int64_t D, int64_t N, int64_t C) {
    BwdLayout l;
    l.fwd = layout(B, T, H, D, N, C);
    const int64_t nC = (T + C - 1) / C;
    const size_t P = (size_t)(B * H * nC * C);
    const size_t S = (size_t)(B * H * nC) * (size_t)(N * D);
    const size_t HS = (size_t)(B * H) * (size_t)(N * D);
    size_t off = l.fwd.total;
    auto put = [&](size_t bytes) {
        const size_t at = off;
        off = round_up(off + bytes);
        return at;
    };
    l.r_re = put(S * sizeof(float));
    l.r_im = put(S * sizeof(float));
    l.q1_re = put(P * sizeof(float));
    l.q1_im = put(P * sizeof(float));
    l.q2_re = put(P * sizeof(float));
    l.q2_im = put(P * sizeof(float));
    l.ddp = put(P * sizeof(float));
    l.hT_re = put(HS * sizeof(float));
    l.hT_im = put(HS * sizeof(float));
    // boundary terms of the log-decay gradient, two partials per chunk
    l.z_re = put((size_t)(B * H * nC) * 2 * sizeof(double));
    l.z_im = put((size_t)(B * H * nC) * 2 * sizeof(double));
    // dA / dDskip partials: one per span of max(C, 64) positions of each (b, h)
    const int64_t span = C > 64 ? C : 64;
    l.pa = put((size_t)(B * H * ((nC * C + span - 1) / span)) * 3 * sizeof(double));
    l.total = off;
    return l;
}

bool empty_problem(int64_t B, int64_t T, int64_t H) { return B == 0 || T == 0 || H == 0; }

int check_shape(int64_t B, int64_t T, int64_t H, int64_t D, int64_t N, int64_t C) {
    if (B < 0 || T < 0 || H < 0 || D <= 0 || N <= 0 || C <= 0) return CSSD_ERR_INVALID_ARG;
    if (!pow2_16_128(D) || !pow2_16_128(N) || !pow2_16_128(C)) return CSSD_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t)1 << 31;
    const int64_t m = D > N ? D : N;
    if (B > lim || T > lim || H > lim) return CSSD_ERR_UNSUPPORTED;
    if (B * H > lim / (N * D)) return CSSD_ERR_UNSUPPORTED;  // one [B,H,N,D] state plane
    if (empty_problem(B, T, H)) return CSSD_OK;
    const int64_t nC = (T + C - 1) / C;
    if (B * H > lim / (nC * C) || B * nC * C * H > lim / m) return CSSD_ERR_UNSUPPORTED;
    if (B * H * nC > lim / (N * D)) return CSSD_ERR_UNSUPPORTED;
    // the kernels address one chunk's rows of a plane through a buffer view whose
    // extent, (C - 1) H m + m elements of up to 4 bytes, must fit 32 bits
    if (C * H * m > lim / 2) return CSSD_ERR_UNSUPPORTED;
    return CSSD_OK;
}

cssd::FwdArgs fwd_args(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int64_t chunk, int32_t in_dtype, const void* x_re,
                       const void* x_im, const void* B_re, const void* B_im, const void* C_re,
                       const void* C_im, const float* dt, const float* A_re, const float* A_im,
                       const float* Dskip, const float* h0_re, const float* h0_im, float* y_re,
                       float* y_im, float* hT_re, float* hT_im, char* ws, const Layout& L) {
    cssd::FwdArgs a;
    a.B = batch;
    a.T = seqlen;
    a.H = nheads;
    a.D = headdim;
    a.N = dstate;
    a.C = chunk;
    a.nC = (seqlen + chunk - 1) / chunk;
    a.in_dtype = in_dtype;
    a.x_re = x_re; a.x_im = x_im;
    a.b_re = B_re; a.b_im = B_im;
    a.c_re = C_re; a.c_im = C_im;
    a.dt = dt; a.a_re = A_re; a.a_im = A_im; a.dskip = Dskip;
    a.h0_re = h0_re; a.h0_im = h0_im;
    a.y_re = y_re; a.y_im = y_im; a.hT_re = hT_re; a.hT_im = hT_im;
    a.acs_re = reinterpret_cast<double*>(ws + L.acs_re);
    a.acs_im = reinterpret_cast<double*>(ws + L.acs_im);
    a.e_re = reinterpret_cast<float*>(ws + L.e_re);
    a.e_im = reinterpret_cast<float*>(ws + L.e_im);
    a.w_re = reinterpret_cast<float*>(ws + L.w_re);
    a.w_im = reinterpret_cast<float*>(ws + L.w_im);
    a.cd_re = reinterpret_cast<float*>(ws + L.cd_re);
    a.cd_im = reinterpret_cast<float*>(ws + L.cd_im);
    a.st_re = reinterpret_cast<float*>(ws + L.st_re);
    a.st_im = reinterpret_cast<float*>(ws + L.st_im);
    return a;
}

// Both planes of one output: dst = src, or zeros when src is NULL.
hipError_t fill_planes(float* dst_re, float* dst_im, const float* src_re, const float* src_im,
                       int64_t n, hipStream_t s) {
    hipError_t e = timed(cssd::K_FILL, s, [&] { return cssd::launch_fill(dst_re, src_re, n, s); });
    if (e != hipSuccess) return e;
    return timed(cssd::K_FILL, s, [&] { return cssd::launch_fill(dst_im, src_im, n, s); });
}

// cssd_forward over zero time steps (or no batch rows or heads): nothing but
// hT is written, and hT = h0 (zero without h0).  n = elements of one state plane.
int empty_forward(int64_t n, const float* h0_re, const float* h0_im, float* hT_re, float* hT_im,
                  void* stream) {
    if ((h0_re == nullptr) != (h0_im == nullptr) || (hT_re == nullptr) != (hT_im == nullptr))
        return CSSD_ERR_INVALID_ARG;
    const void* st[] = {h0_re, h0_im, hT_re, hT_im};
    for (const void* p : st)
        if (!aligned(p, 16)) return CSSD_ERR_INVALID_ARG;
    if (hT_re == nullptr) return CSSD_OK;
    if (hT_re == hT_im || hT_re == h0_re || hT_re == h0_im || hT_im == h0_re || hT_im == h0_im)
        return CSSD_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return fill_planes(hT_re, hT_im, h0_re, h0_im, n, s) == hipSuccess ? CSSD_OK : CSSD_ERR_HIP;
}

// cssd_backward of an empty problem: dA and dDskip are empty sums (zero) and
// dh0 = dhT (zero without dhT).  H = heads, n = elements of one state plane.
int empty_backward(int64_t H, int64_t n, const float* dhT_re, const float* dhT_im, float* dA_re,
                   float* dA_im, float* dD, float* dh0_re, float* dh0_im, void* stream) {
    if (H > 0 && (dA_re == nullptr || dA_im == nullptr)) return CSSD_ERR_INVALID_ARG;
    if ((dhT_re == nullptr) != (dhT_im == nullptr) || (dh0_re == nullptr) != (dh0_im == nullptr))
        return CSSD_ERR_INVALID_ARG;
    if (!aligned(dA_re, 4) || !aligned(dA_im, 4) || !aligned(dD, 4) || !aligned(dhT_re, 16) ||
        !aligned(dhT_im, 16) || !aligned(dh0_re, 16) || !aligned(dh0_im, 16))
        return CSSD_ERR_INVALID_ARG;
    float* outs[] = {dA_re, dA_im, dD, dh0_re, dh0_im};
    for (int i = 0; i < 5; ++i) {
        if (outs[i] == nullptr) continue;
        if (outs[i] == dhT_re || outs[i] == dhT_im) return CSSD_ERR_INVALID_ARG;
        for (int j = 0; j < i; ++j)
            if (outs[i] == outs[j]) return CSSD_ERR_INVALID_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (H > 0) {
        if (fill_planes(dA_re, dA_im, nullptr, nullptr, H, s) != hipSuccess) return CSSD_ERR_HIP;
        if (dD != nullptr &&
            timed(cssd::K_FILL, s, [&] { return cssd::launch_fill(dD, nullptr, H, s); }) !=
                hipSuccess)
            return CSSD_ERR_HIP;
    }
    if (dh0_re != nullptr && fill_planes(dh0_re, dh0_im, dhT_re, dhT_im, n, s) != hipSuccess)
        return CSSD_ERR_HIP;
    return CSSD_OK;
}

}  // namespace

extern "C" {

int cssd_version(void) { return CSSD_VERSION; }

const char* cssd_status_string(int status) {
    switch (status) {
        case CSSD_OK: return "CSSD_OK";
        case CSSD_ERR_INVALID_ARG: return "CSSD_ERR_INVALID_ARG: bad pointer, size, alignment or aliasing";
        case CSSD_ERR_UNSUPPORTED: return "CSSD_ERR_UNSUPPORTED: sizes outside the supported set";
        case CSSD_ERR_WORKSPACE: return "CSSD_ERR_WORKSPACE: workspace missing, too small or misaligned";
        case CSSD_ERR_HIP: return "CSSD_ERR_HIP: a HIP launch or runtime call failed";
        case CSSD_ERR_TOO_LARGE:
            return "CSSD_ERR_TOO_LARGE: the problem's workspace exceeds the fixed device array "
                   "of cssd_forward_noalloc";
        default: return "unknown cssd status";
    }
}

int cssd_forward_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                int64_t dstate, int64_t chunk, size_t* bytes) {
    if (bytes == nullptr) return CSSD_ERR_INVALID_ARG;
    const int st = check_shape(batch, seqlen, nheads, headdim, dstate, chunk);
    if (st != CSSD_OK) return st;
    *bytes = empty_problem(batch, seqlen, nheads)
                 ? 0
                 : layout(batch, seqlen, nheads, headdim, dstate, chunk).total;
    return CSSD_OK;
}

int cssd_forward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                 int64_t chunk, int32_t in_dtype, const void* x_re, const void* x_im,
                 const void* B_re, const void* B_im, const void* C_re, const void* C_im,
                 const float* dt, const float* A_re, const float* A_im, const float* Dskip,
                 const float* h0_re, const float* h0_im, float* y_re, float* y_im, float* hT_re,
                 float* hT_im, void* workspace, size_t workspace_bytes, void* stream) {
    const int st = check_shape(batch, seqlen, nheads, headdim, dstate, chunk);
    if (st != CSSD_OK) return st;
    if (in_dtype != CSSD_F32 && in_dtype != CSSD_BF16) return CSSD_ERR_INVALID_ARG;
    if (empty_problem(batch, seqlen, nheads))
        return empty_forward(batch * nheads * dstate * headdim, h0_re, h0_im, hT_re, hT_im, stream);
    // B and C rows are read as 16-byte (f32) / 8-byte (bf16) vectors, states as
    // float4; everything else only needs its element alignment.
    const uintptr_t in_el = in_dtype == CSSD_BF16 ? 2 : 4, in_vec = 4 * in_el;
    const void* req[] = {x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, y_re, y_im};
    const uintptr_t req_al[] = {in_el, in_el, in_vec, in_vec, in_vec, in_vec, 4, 4, 4, 4, 4};
    for (int i = 0; i < 11; ++i)
        if (req[i] == nullptr || !aligned(req[i], req_al[i])) return CSSD_ERR_INVALID_ARG;
    if ((h0_re == nullptr) != (h0_im == nullptr)) return CSSD_ERR_INVALID_ARG;
    if ((hT_re == nullptr) != (hT_im == nullptr)) return CSSD_ERR_INVALID_ARG;
    const void* opt[] = {Dskip, h0_re, h0_im, hT_re, hT_im};
    const uintptr_t opt_al[] = {4, 16, 16, 16, 16};
    for (int i = 0; i < 5; ++i)
        if (opt[i] != nullptr && !aligned(opt[i], opt_al[i])) return CSSD_ERR_INVALID_ARG;
    const void* ins[] = {x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0_re, h0_im};
    const void* outs[] = {y_re, y_im, hT_re, hT_im};
    for (const void* o : outs) {
        if (o == nullptr) continue;
        for (const void* i : ins)
            if (o == i) return CSSD_ERR_INVALID_ARG;
    }
    if (y_re == y_im || (hT_re != nullptr && (hT_re == hT_im || hT_re == y_re || hT_re == y_im)))
        return CSSD_ERR_INVALID_ARG;

    const Layout L = layout(batch, seqlen, nheads, headdim, dstate, chunk);
    if (workspace == nullptr || workspace_bytes < L.total ||
        (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return CSSD_ERR_WORKSPACE;

    cssd::FwdArgs a = fwd_args(batch, seqlen, nheads, headdim, dstate, chunk, in_dtype, x_re, x_im,
                               B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0_re, h0_im, y_re,
                               y_im, hT_re, hT_im, static_cast<char*>(workspace), L);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (cssd::scan_fused(a)) {  // one kernel, the cumsum included
        if (timed(cssd::K_SCAN_FUSED, s, [&] { return cssd::launch_scan_fused(a, s); }) !=
            hipSuccess)
            return CSSD_ERR_HIP;
        return CSSD_OK;
    }
    if (timed(cssd::K_CUMSUM, s, [&] { return cssd::launch_cumsum(a, s); }) != hipSuccess)
        return CSSD_ERR_HIP;
    if (timed(cssd::K_STATE_SCAN, s, [&] { return cssd::launch_state_scan(a, s); }) != hipSuccess)
        return CSSD_ERR_HIP;
    if (timed(cssd::K_CHUNK_SCAN, s, [&] { return cssd::launch_chunk_scan(a, s); }) != hipSuccess)
        return CSSD_ERR_HIP;
    return CSSD_OK;
}

int cssd_backward_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                 int64_t dstate, int64_t chunk, size_t* bytes) {
    if (bytes == nullptr) return CSSD_ERR_INVALID_ARG;
    const int st = check_shape(batch, seqlen, nheads, headdim, dstate, chunk);
    if (st != CSSD_OK) return st;
    *bytes = empty_problem(batch, seqlen, nheads)
                 ? 0
                 : bwd_layout(batch, seqlen, nheads, headdim, dstate, chunk).total;
    return CSSD_OK;
}

int cssd_backward_workspace_size_dtype(int64_t batch, int64_t seqlen, int64_t nheads,
                                       int64_t headdim, int64_t dstate, int64_t chunk,
                                       int32_t in_dtype, size_t* bytes) {
    if (in_dtype != CSSD_F32 && in_dtype != CSSD_BF16) return CSSD_ERR_INVALID_ARG;
    const int st = cssd_backward_workspace_size(batch, seqlen, nheads, headdim, dstate, chunk,
                                                bytes);
    if (st != CSSD_OK || in_dtype == CSSD_F32 || *bytes == 0) return st;
    *bytes += widen_bytes(batch, seqlen, nheads, headdim, dstate);
    return CSSD_OK;
}

}  // extern "C"

namespace {

// cssd_backward and cssd_backward_saved.  saved: the workspace already holds the
// forward's cumsums and chunk states and fhT_* is the forward's final state (read
// only with dhT); else both are recomputed here.
int backward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
             int64_t chunk, int32_t in_dtype, const void* x_re, const void* x_im,
             const void* B_re, const void* B_im, const void* C_re, const void* C_im,
             const float* dt, const float* A_re, const float* A_im, const float* Dskip,
             const float* h0_re, const float* h0_im, const float* y_re, const float* y_im,
             const float* dy_re, const float* dy_im, const float* dhT_re, const float* dhT_im,
             float* dx_re, float* dx_im, float* dB_re, float* dB_im, float* dC_re, float* dC_im,
             float* ddt, float* dA_re, float* dA_im, float* dD, float* dh0_re, float* dh0_im,
             void* workspace, size_t workspace_bytes, void* stream, bool saved,
             const float* fhT_re, const float* fhT_im) {
    const int st = check_shape(batch, seqlen, nheads, headdim, dstate, chunk);
    if (st != CSSD_OK) return st;
    if (in_dtype != CSSD_F32 && in_dtype != CSSD_BF16) return CSSD_ERR_INVALID_ARG;
    // bf16 inputs: cssd_backward widens them (below); the saved form would need the
    // chunk states of a bf16 forward, which the one-kernel bf16 path never stores
    if (in_dtype == CSSD_BF16 && saved) return CSSD_ERR_UNSUPPORTED;
    if (empty_problem(batch, seqlen, nheads))
        return empty_backward(nheads, batch * nheads * dstate * headdim, dhT_re, dhT_im, dA_re,
                              dA_im, dD, dh0_re, dh0_im, stream);
    // y is not read (the log-decay gradient takes conj(C) . dC in its place), so
    // it is not checked either
    (void)y_re;
    (void)y_im;
    const bool wide = in_dtype == CSSD_BF16;
    // row-vector reads need 16 bytes; the gradients are written element-wise
    const void* req[] = {x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im,
                         dy_re, dy_im, dx_re, dx_im, dB_re, dB_im, dC_re, dC_im, ddt,
                         dA_re, dA_im};
    const uintptr_t req_al[] = {16, 16, 16, 16, 16, 16, 4, 4, 4,
                                16, 16, 4, 4, 4, 4, 4, 4, 4, 4, 4};
    for (int i = 0; i < 20; ++i)
        if (req[i] == nullptr || !aligned(req[i], req_al[i])) return CSSD_ERR_INVALID_ARG;
    if ((h0_re == nullptr) != (h0_im == nullptr) || (dhT_re == nullptr) != (dhT_im == nullptr) ||
        (dh0_re == nullptr) != (dh0_im == nullptr))
        return CSSD_ERR_INVALID_ARG;
    const void* opt[] = {Dskip, h0_re, h0_im, dhT_re, dhT_im, dD, dh0_re, dh0_im};
    const uintptr_t opt_al[] = {4, 16, 16, 16, 16, 4, 16, 16};
    for (int i = 0; i < 8; ++i)
        if (opt[i] != nullptr && !aligned(opt[i], opt_al[i])) return CSSD_ERR_INVALID_ARG;
    if (saved) {
        // the forward's final state enters only the term <dhT, hT>
        if ((fhT_re == nullptr) != (fhT_im == nullptr) || !aligned(fhT_re, 16) ||
            !aligned(fhT_im, 16) || (dhT_re != nullptr && fhT_re == nullptr))
            return CSSD_ERR_INVALID_ARG;
    } else {
        fhT_re = fhT_im = nullptr;
    }
    const void* ins[] = {x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0_re,
                         h0_im, dy_re, dy_im, dhT_re, dhT_im, fhT_re, fhT_im};
    const void* outs[] = {dx_re, dx_im, dB_re, dB_im, dC_re, dC_im, ddt, dA_re, dA_im, dD,
                          dh0_re, dh0_im};
    for (int i = 0; i < 12; ++i) {
        if (outs[i] == nullptr) continue;
        for (const void* in : ins)
            if (outs[i] == in) return CSSD_ERR_INVALID_ARG;
        for (int j = 0; j < i; ++j)
            if (outs[i] == outs[j]) return CSSD_ERR_INVALID_ARG;
    }

    const BwdLayout L = bwd_layout(batch, seqlen, nheads, headdim, dstate, chunk);
    const size_t extra = wide ? widen_bytes(batch, seqlen, nheads, headdim, dstate) : 0;
    if (workspace == nullptr || workspace_bytes < L.total + extra ||
        (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return CSSD_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (wide) {
        // the bf16 planes widened once, after the backward's own layout; the fp32
        // kernels then run on exactly the rounded values
        const int64_t nx = batch * seqlen * nheads * headdim, nb = batch * seqlen * nheads * dstate;
        const void* src[6] = {x_re, x_im, B_re, B_im, C_re, C_im};
        const void* dst[6];
        size_t off = L.total;
        for (int i = 0; i < 6; ++i) {
            const int64_t n = i < 2 ? nx : nb;
            float* d = reinterpret_cast<float*>(ws + off);
            if (timed(cssd::K_WIDEN, s, [&] {
                    return cssd::launch_widen(static_cast<const uint16_t*>(src[i]), d, n, s);
                }) != hipSuccess)
                return CSSD_ERR_HIP;
            dst[i] = d;
            off += round_up((size_t)n * 4);
        }
        x_re = dst[0]; x_im = dst[1]; B_re = dst[2]; B_im = dst[3]; C_re = dst[4]; C_im = dst[5];
        in_dtype = CSSD_F32;
    }
    cssd::BwdArgs a;
    // the recomputed forward writes its final state into the workspace, not y
    a.f = fwd_args(batch, seqlen, nheads, headdim, dstate, chunk, in_dtype, x_re, x_im, B_re,
                   B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0_re, h0_im, nullptr, nullptr,
                   reinterpret_cast<float*>(ws + L.hT_re), reinterpret_cast<float*>(ws + L.hT_im),
                   ws, L.fwd);
    a.dy_re = dy_re; a.dy_im = dy_im;
    a.dhT_re = dhT_re; a.dhT_im = dhT_im;
    a.dx_re = dx_re; a.dx_im = dx_im; a.db_re = dB_re; a.db_im = dB_im;
    a.dc_re = dC_re; a.dc_im = dC_im; a.ddt = ddt; a.da_re = dA_re; a.da_im = dA_im; a.dd = dD;
    a.dh0_re = dh0_re; a.dh0_im = dh0_im;
    a.r_re = reinterpret_cast<float*>(ws + L.r_re);
    a.r_im = reinterpret_cast<float*>(ws + L.r_im);
    a.q1_re = reinterpret_cast<float*>(ws + L.q1_re);
    a.q1_im = reinterpret_cast<float*>(ws + L.q1_im);
    a.q2_re = reinterpret_cast<float*>(ws + L.q2_re);
    a.q2_im = reinterpret_cast<float*>(ws + L.q2_im);
    a.ddp = reinterpret_cast<float*>(ws + L.ddp);
    a.hT_re = saved ? fhT_re : a.f.hT_re;
    a.hT_im = saved ? fhT_im : a.f.hT_im;
    a.z_re = reinterpret_cast<double*>(ws + L.z_re);
    a.z_im = reinterpret_cast<double*>(ws + L.z_im);
    a.pa = reinterpret_cast<double*>(ws + L.pa);

    // forward recomputation: cumsums, chunk states, carry-in states H_c and hT
    if (!saved) {
        if (timed(cssd::K_CUMSUM, s, [&] { return cssd::launch_cumsum(a.f, s); }) != hipSuccess)
            return CSSD_ERR_HIP;
        if (timed(cssd::K_STATE_SCAN, s, [&] { return cssd::launch_state_scan(a.f, s); }) !=
            hipSuccess)
            return CSSD_ERR_HIP;
    }
    // adjoint chunk states and the backward pass over chunks: R_{c+1}, dh0 (and,
    // where the two are fused, the boundary terms of the log-decay gradient)
    const bool fused_adj = cssd::state_scan_adjoint_fused(a.f);
    if (fused_adj) {
        if (timed(cssd::K_STATE_SCAN_ADJ, s, [&] {
                return cssd::launch_state_scan_adjoint(a.f, dy_re, dy_im, dhT_re, dhT_im, a.r_re,
                                                       a.r_im, dh0_re, dh0_im, a.hT_re, a.hT_im,
                                                       a.z_re, a.z_im, s);
            }) != hipSuccess)
            return CSSD_ERR_HIP;
    } else {
        if (timed(cssd::K_CHUNK_STATE, s, [&] {
                return cssd::launch_chunk_state_adjoint(a.f, dy_re, dy_im, a.r_re, a.r_im, s);
            }) != hipSuccess)
            return CSSD_ERR_HIP;
        if (timed(cssd::K_STATE_PASS, s, [&] {
                return cssd::launch_state_pass_adjoint(a.f, a.r_re, a.r_im, dhT_re, dhT_im,
                                                       dh0_re, dh0_im, s);
            }) != hipSuccess)
            return CSSD_ERR_HIP;
    }
    if (timed(cssd::K_BWD_DX, s, [&] { return cssd::launch_bwd_dx(a, s); }) != hipSuccess)
        return CSSD_ERR_HIP;
    if (timed(cssd::K_BWD_DB, s, [&] { return cssd::launch_bwd_db(a, s); }) != hipSuccess)
        return CSSD_ERR_HIP;
    if (timed(cssd::K_BWD_DC, s, [&] { return cssd::launch_bwd_dc(a, s); }) != hipSuccess)
        return CSSD_ERR_HIP;
    if (timed(cssd::K_BWD_DZ, s, [&] { return cssd::launch_bwd_dz(a, !fused_adj, s); }) !=
        hipSuccess)
        return CSSD_ERR_HIP;
    return CSSD_OK;
}

}  // namespace

extern "C" {

int cssd_backward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                  int64_t chunk, int32_t in_dtype, const void* x_re, const void* x_im,
                  const void* B_re, const void* B_im, const void* C_re, const void* C_im,
                  const float* dt, const float* A_re, const float* A_im, const float* Dskip,
                  const float* h0_re, const float* h0_im, const float* y_re, const float* y_im,
                  const float* dy_re, const float* dy_im, const float* dhT_re,
                  const float* dhT_im, float* dx_re, float* dx_im, float* dB_re, float* dB_im,
                  float* dC_re, float* dC_im, float* ddt, float* dA_re, float* dA_im, float* dD,
                  float* dh0_re, float* dh0_im, void* workspace, size_t workspace_bytes,
                  void* stream) {
    return backward(batch, seqlen, nheads, headdim, dstate, chunk, in_dtype, x_re, x_im, B_re,
                    B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0_re, h0_im, y_re, y_im, dy_re,
                    dy_im, dhT_re, dhT_im, dx_re, dx_im, dB_re, dB_im, dC_re, dC_im, ddt, dA_re,
                    dA_im, dD, dh0_re, dh0_im, workspace, workspace_bytes, stream, false, nullptr,
                    nullptr);
}

int cssd_backward_saved(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int64_t chunk, int32_t in_dtype, const void* x_re,
                        const void* x_im, const void* B_re, const void* B_im, const void* C_re,
                        const void* C_im, const float* dt, const float* A_re, const float* A_im,
                        const float* Dskip, const float* h0_re, const float* h0_im,
                        const float* y_re, const float* y_im, const float* hT_re,
                        const float* hT_im, const float* dy_re, const float* dy_im,
                        const float* dhT_re, const float* dhT_im, float* dx_re, float* dx_im,
                        float* dB_re, float* dB_im, float* dC_re, float* dC_im, float* ddt,
                        float* dA_re, float* dA_im, float* dD, float* dh0_re, float* dh0_im,
                        void* workspace, size_t workspace_bytes, void* stream) {
    return backward(batch, seqlen, nheads, headdim, dstate, chunk, in_dtype, x_re, x_im, B_re,
                    B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0_re, h0_im, y_re, y_im, dy_re,
                    dy_im, dhT_re, dhT_im, dx_re, dx_im, dB_re, dB_im, dC_re, dC_im, ddt, dA_re,
                    dA_im, dD, dh0_re, dh0_im, workspace, workspace_bytes, stream, true, hT_re,
                    hT_im);
}

namespace {

// Sizes of the decode entry points (batch or nheads 0: nothing to do).
int step_sizes(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate) {
    if (batch < 0 || nheads < 0 || headdim <= 0 || dstate <= 0) return CSSD_ERR_INVALID_ARG;
    if (!pow2_16_128(headdim) || !pow2_16_128(dstate)) return CSSD_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t)1 << 31;
    if (batch > lim || nheads > lim || batch * nheads > lim / (headdim * dstate))
        return CSSD_ERR_UNSUPPORTED;
    return CSSD_OK;
}

// Host-side checks shared by the decode entry points.  h_re/h_im may be NULL
// (the stationary-output entry point has no state).
int check_step(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate, const float* x_re,
               const float* x_im, const float* B_re, const float* B_im, const float* C_re,
               const float* C_im, const float* dt, const float* A_re, const float* A_im,
               const float* Dskip, const float* h_re, const float* h_im, const float* y_re,
               const float* y_im, bool with_state) {
    const int sz = step_sizes(batch, nheads, headdim, dstate);
    if (sz != CSSD_OK) return sz;
    // x, the state and y are accessed as float4; B, C, dt, A, Dskip as scalars
    const void* req[] = {x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, y_re, y_im};
    const uintptr_t req_al[] = {16, 16, 4, 4, 4, 4, 4, 4, 4, 16, 16};
    for (int i = 0; i < 11; ++i)
        if (req[i] == nullptr || !aligned(req[i], req_al[i])) return CSSD_ERR_INVALID_ARG;
    if (with_state && (h_re == nullptr || h_im == nullptr || !aligned(h_re, 16) || !aligned(h_im, 16)))
        return CSSD_ERR_INVALID_ARG;
    if (Dskip != nullptr && !aligned(Dskip, 4)) return CSSD_ERR_INVALID_ARG;
    const void* ins[] = {x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip};
    const void* outs[] = {h_re, h_im, y_re, y_im};
    for (const void* o : outs)
        for (const void* i : ins)
            if (o != nullptr && o == i) return CSSD_ERR_INVALID_ARG;
    if (y_re == y_im) return CSSD_ERR_INVALID_ARG;
    if (with_state && (h_re == h_im || y_re == h_re || y_re == h_im || y_im == h_re || y_im == h_im))
        return CSSD_ERR_INVALID_ARG;
    return CSSD_OK;
}

cssd::StepArgs step_args(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                         const float* x_re, const float* x_im, const float* B_re,
                         const float* B_im, const float* C_re, const float* C_im, const float* dt,
                         const float* A_re, const float* A_im, const float* Dskip, float* h_re,
                         float* h_im, float* y_re, float* y_im) {
    cssd::StepArgs a;
    a.B = batch; a.H = nheads; a.D = headdim; a.N = dstate;
    a.x_re = x_re; a.x_im = x_im; a.b_re = B_re; a.b_im = B_im; a.c_re = C_re; a.c_im = C_im;
    a.dt = dt; a.a_re = A_re; a.a_im = A_im; a.dskip = Dskip;
    a.h_re = h_re; a.h_im = h_im; a.y_re = y_re; a.y_im = y_im;
    return a;
}

}  // namespace

int cssd_step(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate, const float* x_re,
              const float* x_im, const float* B_re, const float* B_im, const float* C_re,
              const float* C_im, const float* dt, const float* A_re, const float* A_im,
              const float* Dskip, float* h_re, float* h_im, float* y_re, float* y_im,
              void* stream) {
    return cssd_step_n(batch, nheads, headdim, dstate, 1, x_re, x_im, B_re, B_im, C_re, C_im, dt,
                       A_re, A_im, Dskip, h_re, h_im, y_re, y_im, stream);
}

int cssd_step_n(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate, int64_t nsteps,
                const float* x_re, const float* x_im, const float* B_re, const float* B_im,
                const float* C_re, const float* C_im, const float* dt, const float* A_re,
                const float* A_im, const float* Dskip, float* h_re, float* h_im, float* y_re,
                float* y_im, void* stream) {
    if (nsteps < 1) return CSSD_ERR_INVALID_ARG;
    const int sz = step_sizes(batch, nheads, headdim, dstate);
    if (sz != CSSD_OK || batch == 0 || nheads == 0) return sz;
    const int st = check_step(batch, nheads, headdim, dstate, x_re, x_im, B_re, B_im, C_re, C_im,
                              dt, A_re, A_im, Dskip, h_re, h_im, y_re, y_im, true);
    if (st != CSSD_OK) return st;
    cssd::StepArgs a = step_args(batch, nheads, headdim, dstate, x_re, x_im, B_re, B_im, C_re,
                                 C_im, dt, A_re, A_im, Dskip, h_re, h_im, y_re, y_im);
    a.nsteps = nsteps;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (timed(cssd::K_STEP, s, [&] { return cssd::launch_step(a, s); }) != hipSuccess)
        return CSSD_ERR_HIP;
    return CSSD_OK;
}

int cssd_step_infinite(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                       const float* x_re, const float* x_im, const float* B_re, const float* B_im,
                       const float* C_re, const float* C_im, const float* dt, const float* A_re,
                       const float* A_im, const float* Dskip, float* y_re, float* y_im,
                       void* stream) {
    const int sz = step_sizes(batch, nheads, headdim, dstate);
    if (sz != CSSD_OK || batch == 0 || nheads == 0) return sz;
    const int st = check_step(batch, nheads, headdim, dstate, x_re, x_im, B_re, B_im, C_re, C_im,
                              dt, A_re, A_im, Dskip, nullptr, nullptr, y_re, y_im, false);
    if (st != CSSD_OK) return st;
    cssd::StepArgs a = step_args(batch, nheads, headdim, dstate, x_re, x_im, B_re, B_im, C_re,
                                 C_im, dt, A_re, A_im, Dskip, nullptr, nullptr, y_re, y_im);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (timed(cssd::K_STEP_INFINITE, s, [&] { return cssd::launch_step_infinite(a, s); }) !=
        hipSuccess)
        return CSSD_ERR_HIP;
    return CSSD_OK;
}

namespace {

// Threads that fill the chip at one wave per SIMD (256 CUs x 4 SIMDs x 64 lanes).
constexpr int64_t kPhaseThreads = 65536;

// Segment length of the phase scan: the caller's chunk (capped at seqlen), or,
// for chunk = 0, the whole sequence when batch x coordinates alone reach
// kPhaseThreads, else segments (a multiple of 16 steps) short enough for about
// four times that many threads (the segmented form reads the inputs twice, so it
// needs more waves in flight to approach the one-pass bandwidth).
int64_t phase_segment(int64_t B, int64_t T, int64_t HN, int64_t chunk) {
    if (chunk > 0) return chunk < T ? chunk : T;
    const int64_t rows = B * HN;
    if (rows >= kPhaseThreads) return T;
    const int64_t want = (4 * kPhaseThreads + rows - 1) / rows;
    int64_t L = (T + want - 1) / want;
    L = (L + 15) / 16 * 16;
    return L < T ? L : T;
}

int check_phase_shape(int64_t B, int64_t T, int64_t H, int64_t N, int64_t chunk) {
    if (B < 0 || T < 0 || H < 0 || N <= 0 || chunk < 0) return CSSD_ERR_INVALID_ARG;
    const int64_t lim = (int64_t)1 << 31, lim40 = (int64_t)1 << 40;
    if (B > lim || T > lim || H > lim || N > lim) return CSSD_ERR_UNSUPPORTED;
    const int64_t HN = H * N;
    if (HN > lim40 || (HN > 0 && B > lim40 / HN)) return CSSD_ERR_UNSUPPORTED;
    if (empty_problem(B, T, H)) return CSSD_OK;
    if (B * HN > lim40 / T) return CSSD_ERR_UNSUPPORTED;
    return CSSD_OK;
}

size_t phase_workspace(int64_t B, int64_t nch, int64_t HN) {
    if (nch == 1) return 0;
    return 6 * round_up((size_t)(B * nch * HN) * sizeof(float));
}

}  // namespace

int cssd_phase_scan_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                   int64_t dstate, int64_t chunk, size_t* bytes) {
    if (bytes == nullptr) return CSSD_ERR_INVALID_ARG;
    const int st = check_phase_shape(batch, seqlen, nheads, dstate, chunk);
    if (st != CSSD_OK) return st;
    if (empty_problem(batch, seqlen, nheads)) {
        *bytes = 0;
        return CSSD_OK;
    }
    const int64_t HN = nheads * dstate;
    const int64_t L = phase_segment(batch, seqlen, HN, chunk);
    *bytes = phase_workspace(batch, (seqlen + L - 1) / L, HN);
    return CSSD_OK;
}

int cssd_phase_scan(int64_t batch, int64_t seqlen, int64_t nheads, int64_t dstate, int64_t chunk,
                    const float* phi, const float* u, const float* b_re, const float* b_im,
                    const float* psi0_re, const float* psi0_im, float* psi_re, float* psi_im,
                    float* psiT_re, float* psiT_im, void* workspace, size_t workspace_bytes,
                    void* stream) {
    const int st = check_phase_shape(batch, seqlen, nheads, dstate, chunk);
    if (st != CSSD_OK) return st;
    if (empty_problem(batch, seqlen, nheads)) {
        // no step is taken: psiT = psi0 (zero without psi0), also in place
        if ((psi0_re == nullptr) != (psi0_im == nullptr) ||
            (psiT_re == nullptr) != (psiT_im == nullptr))
            return CSSD_ERR_INVALID_ARG;
        if (!aligned(psi0_re, 4) || !aligned(psi0_im, 4) || !aligned(psiT_re, 4) ||
            !aligned(psiT_im, 4))
            return CSSD_ERR_INVALID_ARG;
        if (psiT_re == nullptr) return CSSD_OK;
        if (psiT_re == psiT_im || psiT_re == psi0_im || psiT_im == psi0_re)
            return CSSD_ERR_INVALID_ARG;
        hipStream_t s = static_cast<hipStream_t>(stream);
        return fill_planes(psiT_re, psiT_im, psi0_re, psi0_im, batch * nheads * dstate, s) ==
                       hipSuccess
                   ? CSSD_OK
                   : CSSD_ERR_HIP;
    }
    const void* req[] = {phi, u, b_re, b_im, psi_re, psi_im};
    for (const void* p : req)
        if (p == nullptr || !aligned(p, 4)) return CSSD_ERR_INVALID_ARG;
    if ((psi0_re == nullptr) != (psi0_im == nullptr)) return CSSD_ERR_INVALID_ARG;
    if ((psiT_re == nullptr) != (psiT_im == nullptr)) return CSSD_ERR_INVALID_ARG;
    if (!aligned(psi0_re, 4) || !aligned(psi0_im, 4) || !aligned(psiT_re, 4) ||
        !aligned(psiT_im, 4))
        return CSSD_ERR_INVALID_ARG;
    // psiT may replace psi0 in place (same plane); nothing else may alias
    const void* ins[] = {phi, u, b_re, b_im, psi0_re, psi0_im};
    for (const void* i : ins)
        if (i == psi_re || i == psi_im) return CSSD_ERR_INVALID_ARG;
    const void* ins_t[] = {phi, u, b_re, b_im};
    if (psiT_re != nullptr) {
        for (const void* i : ins_t)
            if (i == psiT_re || i == psiT_im) return CSSD_ERR_INVALID_ARG;
        if (psiT_re == psi0_im || psiT_im == psi0_re) return CSSD_ERR_INVALID_ARG;
        if (psiT_re == psiT_im || psiT_re == psi_re || psiT_re == psi_im ||
            psiT_im == psi_re || psiT_im == psi_im)
            return CSSD_ERR_INVALID_ARG;
    }
    if (psi_re == psi_im) return CSSD_ERR_INVALID_ARG;

    cssd::PhaseArgs a;
    a.B = batch;
    a.T = seqlen;
    a.HN = nheads * dstate;
    a.L = phase_segment(batch, seqlen, a.HN, chunk);
    a.nch = (seqlen + a.L - 1) / a.L;
    a.phi = phi; a.u = u; a.b_re = b_re; a.b_im = b_im;
    a.psi0_re = psi0_re; a.psi0_im = psi0_im;
    a.psi_re = psi_re; a.psi_im = psi_im; a.psiT_re = psiT_re; a.psiT_im = psiT_im;
    a.p_re = a.p_im = a.s_re = a.s_im = a.in_re = a.in_im = nullptr;
    const size_t need = phase_workspace(batch, a.nch, a.HN);
    if (need > 0) {
        if (workspace == nullptr || !aligned(workspace, kAlign) || workspace_bytes < need)
            return CSSD_ERR_WORKSPACE;
        const size_t plane = need / 6;
        char* ws = static_cast<char*>(workspace);
        float** regions[] = {&a.p_re, &a.p_im, &a.s_re, &a.s_im, &a.in_re, &a.in_im};
        for (int r = 0; r < 6; ++r) *regions[r] = reinterpret_cast<float*>(ws + r * plane);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.nch > 1) {
        if (timed(cssd::K_PHASE_SUMMARY, s, [&] { return cssd::launch_phase_summary(a, s); }) !=
            hipSuccess)
            return CSSD_ERR_HIP;
        if (timed(cssd::K_PHASE_CARRY, s, [&] { return cssd::launch_phase_carry(a, s); }) !=
            hipSuccess)
            return CSSD_ERR_HIP;
    }
    if (timed(cssd::K_PHASE_OUT, s, [&] { return cssd::launch_phase_out(a, s); }) != hipSuccess)
        return CSSD_ERR_HIP;
    return CSSD_OK;
}

int cssd_born_attention(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int32_t in_dtype, const void* q_re, const void* q_im, const void* k_re,
                        const void* k_im, const void* v_re, const void* v_im, const float* tau,
                        float* out_re, float* out_im, void* stream) {
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim <= 0) return CSSD_ERR_INVALID_ARG;
    if (in_dtype != CSSD_F32 && in_dtype != CSSD_BF16) return CSSD_ERR_INVALID_ARG;
    if (headdim != 16 && headdim != 32 && headdim != 64) return CSSD_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t)1 << 31, lim40 = (int64_t)1 << 40;
    if (batch > lim || seqlen > lim || nheads > lim || batch * nheads > lim / 64 ||
        batch * nheads * seqlen > lim40 / headdim)
        return CSSD_ERR_UNSUPPORTED;
    if (empty_problem(batch, seqlen, nheads)) return CSSD_OK;  // no rows to write
    const void* req[] = {q_re, q_im, k_re, k_im, v_re, v_im, out_re, out_im};
    for (const void* p : req)
        if (p == nullptr || !aligned(p, 16)) return CSSD_ERR_INVALID_ARG;
    if (!aligned(tau, 4)) return CSSD_ERR_INVALID_ARG;
    const void* ins[] = {q_re, q_im, k_re, k_im, v_re, v_im, tau};
    for (const void* i : ins)
        if (i == out_re || i == out_im) return CSSD_ERR_INVALID_ARG;
    if (out_re == out_im) return CSSD_ERR_INVALID_ARG;
    cssd::BornArgs a;
    a.B = batch;
    a.T = seqlen;
    a.H = nheads;
    a.D = headdim;
    // query blocks of 64 rows (fp32 kernel) or 128 rows (bf16 kernel)
    const int64_t qrows = in_dtype == CSSD_F32 ? 64 : 128;
    a.nqb = (seqlen + qrows - 1) / qrows;
    a.npair = (a.nqb + 1) / 2;
    // heads sharing one 128-byte line of a time step go to the same XCD
    const int64_t row_bytes = headdim * (in_dtype == CSSD_F32 ? 4 : 2);
    a.hpl = row_bytes >= 128 ? 1 : 128 / row_bytes;
    a.in_dtype = in_dtype;
    a.q_re = static_cast<const float*>(q_re);
    a.q_im = static_cast<const float*>(q_im);
    a.k_re = static_cast<const float*>(k_re);
    a.k_im = static_cast<const float*>(k_im);
    a.v_re = static_cast<const float*>(v_re);
    a.v_im = static_cast<const float*>(v_im);
    a.tau = tau;
    a.out_re = out_re;
    a.out_im = out_im;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (timed(cssd::K_BORN, s, [&] { return cssd::launch_born(a, s); }) != hipSuccess)
        return CSSD_ERR_HIP;
    return CSSD_OK;
}

int cssd_profile_enable(int on) {
    Profiler& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    p.on = on != 0;
    return CSSD_OK;
}

int cssd_profile_read(double* ms, int64_t* launches, int capacity) {
    Profiler& p = prof();
    // take the pending brackets out under the lock, then wait for them without
    // it, so that other threads' launches are not held up meanwhile
    std::vector<Pending> mine;
    {
        std::lock_guard<std::mutex> g(p.mu);
        mine.swap(p.pending);
    }
    int status = CSSD_OK;
    std::vector<float> took(mine.size(), -1.f);
    for (size_t j = 0; j < mine.size(); ++j) {
        float t = 0.f;
        if (hipEventSynchronize(mine[j].stop) != hipSuccess ||
            hipEventElapsedTime(&t, mine[j].start, mine[j].stop) != hipSuccess)
            status = CSSD_ERR_HIP;
        else
            took[j] = t;
    }
    std::lock_guard<std::mutex> g(p.mu);
    for (size_t j = 0; j < mine.size(); ++j) {
        if (took[j] >= 0.f) {
            p.ms[mine[j].kernel] += took[j];
            p.launches[mine[j].kernel] += 1;
        }
        p.pool.push_back(mine[j].start);
        p.pool.push_back(mine[j].stop);
    }
    for (int k = 0; k < cssd::K_COUNT && k < capacity; ++k) {
        if (ms) ms[k] = p.ms[k];
        if (launches) launches[k] = p.launches[k];
    }
    for (int k = 0; k < cssd::K_COUNT; ++k) {
        p.ms[k] = 0;
        p.launches[k] = 0;
    }
    return status == CSSD_OK ? (int)cssd::K_COUNT : -status;
}

const char* cssd_kernel_name(int kernel_id) {
    static const char* names[cssd::K_COUNT] = {
        "k_cumsum", "k_chunk_state", "k_state_pass", "k_chunk_scan", "k_step",
        "k_step_infinite", "k_bwd_dx", "k_bwd_dc", "k_bwd_dz",
        "k_phase_summary", "k_phase_carry", "k_phase_out", "k_born", "k_bwd_db",
        "k_state_scan", "k_state_scan_adj", "k_fill", "k_scan_fused", "k_widen"};
    if (kernel_id < 0 || kernel_id >= cssd::K_COUNT) return nullptr;
    return names[kernel_id];
}

}  // extern "C"
