// AddressSanitizer driver of the C ABI's host layer: validation, workspace
// layout and kernel sequencing, with the kernel launchers replaced by the
// host-only stubs of launch_stubs.cpp (no device is touched).  Exits 0 when
// every expectation holds and prints the number of calls checked.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "cssd.h"

extern "C" void stub_register_workspace(const void* p, size_t bytes);
extern "C" int stub_bad(void);
extern "C" size_t stub_calls(void);
extern "C" const char* stub_call(size_t i);
extern "C" void stub_reset(void);

static int failures = 0, checks = 0;

#define EXPECT(cond, ...)                                        \
    do {                                                         \
        ++checks;                                                \
        if (!(cond)) {                                           \
            ++failures;                                          \
            std::fprintf(stderr, "line %d: ", __LINE__);         \
            std::fprintf(stderr, __VA_ARGS__);                   \
            std::fprintf(stderr, "\n");                          \
        }                                                        \
    } while (0)

// a 256-byte aligned host buffer standing in for device memory (never dereferenced
// by the layer under test)
struct Buf {
    void* p = nullptr;
    explicit Buf(size_t bytes) { p = std::aligned_alloc(256, (bytes + 255) / 256 * 256 + 256); }
    ~Buf() { std::free(p); }
    float* f(size_t off_bytes = 0) const { return reinterpret_cast<float*>((char*)p + off_bytes); }
};

static std::string calls() {
    std::string s;
    for (size_t i = 0; i < stub_calls(); ++i) s += std::string(stub_call(i)) + " ";
    return s;
}

struct Fwd {
    int64_t B, T, H, D, N, C;
    int32_t dt;
    Buf x_re, x_im, b_re, b_im, c_re, c_im, dtb, a_re, a_im, dsk, h0_re, h0_im, y_re, y_im, hT_re, hT_im;
    Fwd(int64_t B_, int64_t T_, int64_t H_, int64_t D_, int64_t N_, int64_t C_, int32_t dtype)
        : B(B_), T(T_), H(H_), D(D_), N(N_), C(C_), dt(dtype),
          x_re(sz(D)), x_im(sz(D)), b_re(sz(N)), b_im(sz(N)), c_re(sz(N)), c_im(sz(N)),
          dtb(B_ * T_ * H_ * 4 + 4), a_re(H_ * 4 + 4), a_im(H_ * 4 + 4), dsk(H_ * 4 + 4),
          h0_re(st()), h0_im(st()), y_re(B_ * T_ * H_ * D_ * 4 + 4), y_im(B_ * T_ * H_ * D_ * 4 + 4),
          hT_re(st()), hT_im(st()) {}
    size_t sz(int64_t w) const { return (size_t)(B * T * H * w) * (dt == CSSD_BF16 ? 2 : 4) + 16; }
    size_t st() const { return (size_t)(B * H * N * D) * 4 + 16; }
    int run(void* ws, size_t bytes, const void* xr = nullptr, float* yr = nullptr) {
        return cssd_forward(B, T, H, D, N, C, dt, xr ? xr : x_re.p, x_im.p, b_re.p, b_im.p, c_re.p,
                            c_im.p, dtb.f(), a_re.f(), a_im.f(), dsk.f(), h0_re.f(), h0_im.f(),
                            yr ? yr : y_re.f(), y_im.f(), hT_re.f(), hT_im.f(), ws, bytes, nullptr);
    }
};

int main() {
    // ---- forward: valid shapes with an exact workspace, every supported size
    const int64_t widths[] = {16, 32, 64, 128}, chunks[] = {16, 32, 64, 128};
    const int64_t lengths[] = {1, 15, 64, 65, 130};
    for (int64_t D : widths)
        for (int64_t N : widths)
            for (int64_t C : chunks)
                for (int64_t T : lengths)
                    for (int32_t dtype : {CSSD_F32, CSSD_BF16}) {
                        Fwd f(2, T, 3, D, N, C, dtype);
                        size_t bytes = 0;
                        EXPECT(cssd_forward_workspace_size(2, T, 3, D, N, C, &bytes) == CSSD_OK,
                               "size D%ld N%ld C%ld", (long)D, (long)N, (long)C);
                        Buf ws(bytes);
                        stub_reset();
                        stub_register_workspace(ws.p, bytes);
                        EXPECT(f.run(ws.p, bytes) == CSSD_OK, "forward D%ld N%ld C%ld T%ld",
                               (long)D, (long)N, (long)C, (long)T);
                        EXPECT(stub_bad() == 0, "workspace regions D%ld N%ld C%ld", (long)D,
                               (long)N, (long)C);
                        const bool fused = dtype == CSSD_BF16 && D == 64 && N == 64 && C == 64;
                        EXPECT(calls() == (fused ? "scan_fused " : "cumsum state_scan chunk_scan "),
                               "sequence %s", calls().c_str());
                        // one byte short, and misaligned
                        EXPECT(f.run(ws.p, bytes - 1) == CSSD_ERR_WORKSPACE, "short workspace");
                        EXPECT(f.run((char*)ws.p + 16, bytes) == CSSD_ERR_WORKSPACE, "misaligned");
                    }
    // ---- forward: argument errors
    {
        Fwd f(2, 100, 3, 64, 64, 64, CSSD_F32);
        size_t bytes = 0;
        cssd_forward_workspace_size(2, 100, 3, 64, 64, 64, &bytes);
        Buf ws(bytes);
        stub_register_workspace(ws.p, bytes);
        stub_reset();
        EXPECT(cssd_forward(2, 100, 3, 64, 64, 64, CSSD_F32, nullptr, f.x_im.p, f.b_re.p, f.b_im.p,
                            f.c_re.p, f.c_im.p, f.dtb.f(), f.a_re.f(), f.a_im.f(), nullptr, nullptr,
                            nullptr, f.y_re.f(), f.y_im.f(), nullptr, nullptr, ws.p, bytes,
                            nullptr) == CSSD_ERR_INVALID_ARG, "null x");
        EXPECT(cssd_forward(2, 100, 3, 64, 64, 64, CSSD_F32, f.x_re.p, f.x_im.p, f.b_re.f(4),
                            f.b_im.p, f.c_re.p, f.c_im.p, f.dtb.f(), f.a_re.f(), f.a_im.f(), nullptr,
                            nullptr, nullptr, f.y_re.f(), f.y_im.f(), nullptr, nullptr, ws.p, bytes,
                            nullptr) == CSSD_ERR_INVALID_ARG, "misaligned B");
        EXPECT(f.run(ws.p, bytes, f.y_re.p) == CSSD_ERR_INVALID_ARG, "y aliases x");
        EXPECT(cssd_forward(2, 100, 3, 48, 64, 64, CSSD_F32, f.x_re.p, f.x_im.p, f.b_re.p,
                            f.b_im.p, f.c_re.p, f.c_im.p, f.dtb.f(), f.a_re.f(), f.a_im.f(),
                            nullptr, nullptr, nullptr, f.y_re.f(), f.y_im.f(), nullptr, nullptr,
                            ws.p, bytes, nullptr) == CSSD_ERR_UNSUPPORTED, "D 48");
        EXPECT(cssd_forward(2, -1, 3, 64, 64, 64, CSSD_F32, f.x_re.p, f.x_im.p, f.b_re.p, f.b_im.p,
                            f.c_re.p, f.c_im.p, f.dtb.f(), f.a_re.f(), f.a_im.f(), nullptr,
                            nullptr, nullptr, f.y_re.f(), f.y_im.f(), nullptr, nullptr, ws.p,
                            bytes, nullptr) == CSSD_ERR_INVALID_ARG, "T -1");
        EXPECT(cssd_forward(2, 100, 3, 64, 64, 64, 7, f.x_re.p, f.x_im.p, f.b_re.p, f.b_im.p,
                            f.c_re.p, f.c_im.p, f.dtb.f(), f.a_re.f(), f.a_im.f(), nullptr,
                            nullptr, nullptr, f.y_re.f(), f.y_im.f(), nullptr, nullptr, ws.p,
                            bytes, nullptr) == CSSD_ERR_INVALID_ARG, "dtype 7");
        EXPECT(stub_calls() == 0, "nothing launched on errors: %s", calls().c_str());
        // an empty sequence: hT = h0 through the fill kernel, no workspace
        stub_reset();
        EXPECT(cssd_forward(2, 0, 3, 64, 64, 64, CSSD_F32, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr, nullptr, f.a_re.f(), f.a_im.f(), nullptr, f.h0_re.f(),
                            f.h0_im.f(), nullptr, nullptr, f.hT_re.f(), f.hT_im.f(), nullptr, 0,
                            nullptr) == CSSD_OK, "empty");
        EXPECT(calls() == "fill fill ", "empty sequence %s", calls().c_str());
    }
    // ---- backward: both state-pass forms, recomputed and saved
    for (int64_t D : widths)
        for (int64_t N : {(int64_t)32, (int64_t)64})
            for (int64_t C : {(int64_t)32, (int64_t)64}) {
                const int64_t B = 2, T = 130, H = 2;
                Fwd f(B, T, H, D, N, C, CSSD_F32);
                Buf dy_re(B * T * H * D * 4 + 16), dy_im(B * T * H * D * 4 + 16);
                Buf g[12] = {Buf(f.sz(D)), Buf(f.sz(D)), Buf(f.sz(N)), Buf(f.sz(N)), Buf(f.sz(N)),
                             Buf(f.sz(N)), Buf(B * T * H * 4 + 16), Buf(H * 4 + 16), Buf(H * 4 + 16),
                             Buf(H * 4 + 16), Buf(f.st()), Buf(f.st())};
                size_t bytes = 0;
                EXPECT(cssd_backward_workspace_size(B, T, H, D, N, C, &bytes) == CSSD_OK, "bws");
                Buf ws(bytes);
                stub_register_workspace(ws.p, bytes);
                for (int saved = 0; saved < 2; ++saved) {
                    stub_reset();
                    int st;
                    if (saved)
                        st = cssd_backward_saved(B, T, H, D, N, C, CSSD_F32, f.x_re.p, f.x_im.p,
                                                 f.b_re.p, f.b_im.p, f.c_re.p, f.c_im.p, f.dtb.f(),
                                                 f.a_re.f(), f.a_im.f(), f.dsk.f(), f.h0_re.f(),
                                                 f.h0_im.f(), f.y_re.f(), f.y_im.f(), f.hT_re.f(),
                                                 f.hT_im.f(), dy_re.f(), dy_im.f(), nullptr,
                                                 nullptr, g[0].f(), g[1].f(), g[2].f(), g[3].f(),
                                                 g[4].f(), g[5].f(), g[6].f(), g[7].f(), g[8].f(),
                                                 g[9].f(), g[10].f(), g[11].f(), ws.p, bytes,
                                                 nullptr);
                    else
                        st = cssd_backward(B, T, H, D, N, C, CSSD_F32, f.x_re.p, f.x_im.p, f.b_re.p,
                                           f.b_im.p, f.c_re.p, f.c_im.p, f.dtb.f(), f.a_re.f(),
                                           f.a_im.f(), f.dsk.f(), f.h0_re.f(), f.h0_im.f(),
                                           f.y_re.f(), f.y_im.f(), dy_re.f(), dy_im.f(), nullptr,
                                           nullptr, g[0].f(), g[1].f(), g[2].f(), g[3].f(),
                                           g[4].f(), g[5].f(), g[6].f(), g[7].f(), g[8].f(),
                                           g[9].f(), g[10].f(), g[11].f(), ws.p, bytes, nullptr);
                    EXPECT(st == CSSD_OK, "backward D%ld N%ld C%ld saved %d: %d", (long)D, (long)N,
                           (long)C, saved, st);
                    EXPECT(stub_bad() == 0, "backward workspace regions");
                    const bool fused = D == 64 && N == 64 && C == 64;
                    std::string want = saved ? "" : "cumsum state_scan ";
                    want += fused ? "state_scan_adj " : "chunk_state_adjoint state_pass_adjoint ";
                    want += "bwd_dx bwd_db bwd_dc bwd_dz ";
                    EXPECT(calls() == want, "backward sequence %s", calls().c_str());
                }
                // bf16 inputs: the fp32-size workspace is too small; with the bf16 size
                // the six planes are widened inside it, then the fp32 sequence runs;
                // the saved-state form takes fp32 only
                Fwd fb(B, T, H, D, N, C, CSSD_BF16);
                size_t bbytes = 0;
                EXPECT(cssd_backward_workspace_size_dtype(B, T, H, D, N, C, CSSD_BF16, &bbytes) ==
                           CSSD_OK, "bws bf16");
                EXPECT(bbytes > bytes, "bf16 workspace %zu against %zu", bbytes, bytes);
                Buf wsb(bbytes);
                // (y is not read: NULL here)
                auto bf16_backward = [&](size_t nbytes) {
                    return cssd_backward(B, T, H, D, N, C, CSSD_BF16, fb.x_re.p, fb.x_im.p,
                                         fb.b_re.p, fb.b_im.p, fb.c_re.p, fb.c_im.p, fb.dtb.f(),
                                         fb.a_re.f(), fb.a_im.f(), nullptr, nullptr, nullptr,
                                         nullptr, nullptr, dy_re.f(), dy_im.f(), nullptr,
                                         nullptr, g[0].f(), g[1].f(), g[2].f(), g[3].f(),
                                         g[4].f(), g[5].f(), g[6].f(), g[7].f(), g[8].f(),
                                         nullptr, nullptr, nullptr, wsb.p, nbytes, nullptr);
                };
                stub_register_workspace(wsb.p, bbytes);
                stub_reset();
                EXPECT(bf16_backward(bytes) == CSSD_ERR_WORKSPACE, "bf16 backward, fp32 workspace");
                EXPECT(calls().empty(), "bf16 backward refused, launched %s", calls().c_str());
                stub_reset();
                EXPECT(bf16_backward(bbytes) == CSSD_OK, "bf16 backward");
                EXPECT(stub_bad() == 0, "bf16 backward workspace regions");
                {
                    const bool fused = D == 64 && N == 64 && C == 64;
                    std::string want = "widen widen widen widen widen widen cumsum state_scan ";
                    want += fused ? "state_scan_adj " : "chunk_state_adjoint state_pass_adjoint ";
                    want += "bwd_dx bwd_db bwd_dc bwd_dz ";
                    EXPECT(calls() == want, "bf16 backward sequence %s", calls().c_str());
                }
                stub_reset();
                EXPECT(cssd_backward_saved(B, T, H, D, N, C, CSSD_BF16, fb.x_re.p, fb.x_im.p,
                                           fb.b_re.p, fb.b_im.p, fb.c_re.p, fb.c_im.p, fb.dtb.f(),
                                           fb.a_re.f(), fb.a_im.f(), nullptr, nullptr, nullptr,
                                           fb.y_re.f(), fb.y_im.f(), fb.hT_re.f(), fb.hT_im.f(),
                                           dy_re.f(), dy_im.f(), nullptr, nullptr, g[0].f(),
                                           g[1].f(), g[2].f(), g[3].f(), g[4].f(), g[5].f(),
                                           g[6].f(), g[7].f(), g[8].f(), nullptr, nullptr, nullptr,
                                           wsb.p, bbytes, nullptr) == CSSD_ERR_UNSUPPORTED,
                       "bf16 saved backward");
            }
    // ---- decode step and the constant-input calls
    {
        const int64_t B = 4, H = 3, D = 64, N = 128;
        Buf x_re(B * H * D * 4), x_im(B * H * D * 4), b_re(B * H * N * 4), b_im(B * H * N * 4),
            c_re(B * H * N * 4), c_im(B * H * N * 4), dt(B * H * 4), a_re(H * 4), a_im(H * 4),
            h_re(B * H * N * D * 4), h_im(B * H * N * D * 4), y_re(B * H * D * 4), y_im(B * H * D * 4);
        stub_reset();
        EXPECT(cssd_step(B, H, D, N, x_re.f(), x_im.f(), b_re.f(), b_im.f(), c_re.f(), c_im.f(),
                         dt.f(), a_re.f(), a_im.f(), nullptr, h_re.f(), h_im.f(), y_re.f(), y_im.f(),
                         nullptr) == CSSD_OK, "step");
        EXPECT(cssd_step_n(B, H, D, N, 0, x_re.f(), x_im.f(), b_re.f(), b_im.f(), c_re.f(),
                           c_im.f(), dt.f(), a_re.f(), a_im.f(), nullptr, h_re.f(), h_im.f(),
                           y_re.f(), y_im.f(), nullptr) == CSSD_ERR_INVALID_ARG, "n = 0");
        EXPECT(cssd_step(B, H, D, N, x_re.f(), x_im.f(), b_re.f(), b_im.f(), c_re.f(), c_im.f(),
                         dt.f(), a_re.f(), a_im.f(), nullptr, h_re.f(), h_im.f(), h_re.f(),
                         y_im.f(), nullptr) == CSSD_ERR_INVALID_ARG, "y aliases h");
        EXPECT(cssd_step_infinite(B, H, D, N, x_re.f(), x_im.f(), b_re.f(), b_im.f(), c_re.f(),
                                  c_im.f(), dt.f(), a_re.f(), a_im.f(), nullptr, y_re.f(), y_im.f(),
                                  nullptr) == CSSD_OK, "infinite");
        EXPECT(calls() == "step step_infinite ", "step sequence %s", calls().c_str());
    }
    // ---- phase scan (one pass and in segments) and Born attention
    {
        const int64_t B = 2, T = 300, H = 3, N = 16;
        Buf phi(B * T * H * N * 4), u(B * T * H * N * 4), b_re(B * T * H * N * 4),
            b_im(B * T * H * N * 4), p_re(B * T * H * N * 4), p_im(B * T * H * N * 4),
            t_re(B * H * N * 4), t_im(B * H * N * 4);
        for (int64_t chunk : {(int64_t)0, (int64_t)64}) {
            size_t bytes = 0;
            EXPECT(cssd_phase_scan_workspace_size(B, T, H, N, chunk, &bytes) == CSSD_OK, "pws");
            Buf ws(bytes + 1);
            stub_reset();
            EXPECT(cssd_phase_scan(B, T, H, N, chunk, phi.f(), u.f(), b_re.f(), b_im.f(), nullptr,
                                   nullptr, p_re.f(), p_im.f(), t_re.f(), t_im.f(), ws.p, bytes,
                                   nullptr) == CSSD_OK, "phase chunk %ld", (long)chunk);
            EXPECT(calls() == (bytes ? "phase_summary phase_carry phase_out " : "phase_out "),
                   "phase sequence %s", calls().c_str());
        }
        const int64_t D = 16;
        Buf q(B * T * H * D * 4), o_re(B * T * H * D * 4), o_im(B * T * H * D * 4);
        stub_reset();
        EXPECT(cssd_born_attention(B, T, H, D, CSSD_F32, q.p, q.p, q.p, q.p, q.p, q.p, nullptr,
                                   o_re.f(), o_im.f(), nullptr) == CSSD_OK, "born");
        EXPECT(cssd_born_attention(B, T, H, 48, CSSD_F32, q.p, q.p, q.p, q.p, q.p, q.p, nullptr,
                                   o_re.f(), o_im.f(), nullptr) == CSSD_ERR_UNSUPPORTED, "born D48");
        EXPECT(calls() == "born ", "born sequence %s", calls().c_str());
    }
    for (int st = 0; st < 7; ++st) EXPECT(cssd_status_string(st) != nullptr, "status string");
    std::printf("%d checks, %d failed\n", checks, failures);
    return failures == 0 ? 0 : 1;
}
