// Host-only stand-ins for the kernel launchers of libcssd.so, linked with the C
// ABI layer (cssd_api.hip) into an AddressSanitizer test binary that runs on the
// CPU.  Each stub records which kernel the entry point asked for and checks that
// every workspace region it was handed lies inside the workspace the test
// registered, then returns hipSuccess without touching a device.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "cssd_launch.h"

namespace stub {
const char* ws_lo = nullptr;
const char* ws_hi = nullptr;
std::vector<std::string> calls;
int bad = 0;

void check(const void* p, size_t bytes, const char* what) {
    const char* c = static_cast<const char*>(p);
    if (c == nullptr || c < ws_lo || c + bytes > ws_hi) {
        std::fprintf(stderr, "workspace region %s outside the workspace\n", what);
        ++bad;
    }
}

void check_fwd(const cssd::FwdArgs& a) {
    const size_t P = (size_t)(a.B * a.H * a.nC * a.C), S = (size_t)(a.B * a.H * a.nC);
    check(a.acs_re, P * 8, "acs_re");
    check(a.acs_im, P * 8, "acs_im");
    check(a.e_re, P * 4, "e_re");
    check(a.e_im, P * 4, "e_im");
    check(a.w_re, P * 4, "w_re");
    check(a.w_im, P * 4, "w_im");
    check(a.cd_re, S * 4, "cd_re");
    check(a.cd_im, S * 4, "cd_im");
    check(a.st_re, S * (size_t)(a.N * a.D) * 4, "st_re");
    check(a.st_im, S * (size_t)(a.N * a.D) * 4, "st_im");
}
}  // namespace stub

extern "C" void stub_register_workspace(const void* p, size_t bytes) {
    stub::ws_lo = static_cast<const char*>(p);
    stub::ws_hi = stub::ws_lo + bytes;
}
extern "C" int stub_bad(void) { return stub::bad; }
extern "C" size_t stub_calls(void) { return stub::calls.size(); }
extern "C" const char* stub_call(size_t i) {
    return i < stub::calls.size() ? stub::calls[i].c_str() : nullptr;
}
extern "C" void stub_reset(void) {
    stub::calls.clear();
    stub::bad = 0;
}

namespace cssd {
hipError_t device_cu_count(int* cus) {
    *cus = 256;
    return hipSuccess;
}
hipError_t launch_widen(const uint16_t*, float* dst, int64_t n, hipStream_t) {
    stub::check(dst, (size_t)n * 4, "widened plane");
    stub::calls.push_back("widen");
    return hipSuccess;
}
hipError_t launch_cumsum(const FwdArgs& a, hipStream_t) {
    stub::check_fwd(a);
    stub::calls.push_back("cumsum");
    return hipSuccess;
}
hipError_t launch_state_scan(const FwdArgs& a, hipStream_t) {
    stub::check_fwd(a);
    stub::calls.push_back("state_scan");
    return hipSuccess;
}
hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t) {
    stub::check_fwd(a);
    stub::calls.push_back("chunk_scan");
    return hipSuccess;
}
bool scan_fused(const FwdArgs& a) {
    return a.in_dtype == 1 && a.C == 64 && a.N == 64 && a.D == 64;
}
hipError_t launch_scan_fused(const FwdArgs&, hipStream_t) {
    stub::calls.push_back("scan_fused");
    return hipSuccess;
}
hipError_t launch_step(const StepArgs&, hipStream_t) {
    stub::calls.push_back("step");
    return hipSuccess;
}
hipError_t launch_chunk_state_adjoint(const FwdArgs& a, const float*, const float*, float* q_re,
                                      float* q_im, hipStream_t) {
    stub::check_fwd(a);
    const size_t S = (size_t)(a.B * a.H * a.nC) * (size_t)(a.N * a.D) * 4;
    stub::check(q_re, S, "r_re");
    stub::check(q_im, S, "r_im");
    stub::calls.push_back("chunk_state_adjoint");
    return hipSuccess;
}
hipError_t launch_state_pass_adjoint(const FwdArgs&, float*, float*, const float*, const float*,
                                     float*, float*, hipStream_t) {
    stub::calls.push_back("state_pass_adjoint");
    return hipSuccess;
}
static void check_bwd(const BwdArgs& a) {
    stub::check_fwd(a.f);
    const size_t P = (size_t)(a.f.B * a.f.H * a.f.nC * a.f.C);
    const size_t S = (size_t)(a.f.B * a.f.H * a.f.nC) * (size_t)(a.f.N * a.f.D);
    stub::check(a.r_re, S * 4, "r_re");
    stub::check(a.r_im, S * 4, "r_im");
    stub::check(a.q1_re, P * 4, "q1_re");
    stub::check(a.q1_im, P * 4, "q1_im");
    stub::check(a.q2_re, P * 4, "q2_re");
    stub::check(a.q2_im, P * 4, "q2_im");
    stub::check(a.ddp, P * 4, "ddp");
    stub::check(a.z_re, (size_t)(a.f.B * a.f.H * a.f.nC) * 16, "z_re");
    stub::check(a.z_im, (size_t)(a.f.B * a.f.H * a.f.nC) * 16, "z_im");
}
hipError_t launch_bwd_dx(const BwdArgs& a, hipStream_t) {
    check_bwd(a);
    stub::calls.push_back("bwd_dx");
    return hipSuccess;
}
hipError_t launch_bwd_db(const BwdArgs& a, hipStream_t) {
    check_bwd(a);
    stub::calls.push_back("bwd_db");
    return hipSuccess;
}
hipError_t launch_bwd_dc(const BwdArgs& a, hipStream_t) {
    check_bwd(a);
    stub::calls.push_back("bwd_dc");
    return hipSuccess;
}
bool state_scan_adjoint_fused(const FwdArgs& a) {
    return a.in_dtype == 0 && a.C == 64 && a.N == 64 && a.D == 64;
}
hipError_t launch_state_scan_adjoint(const FwdArgs& a, const float*, const float*, const float*,
                                     const float*, float*, float*, float*, float*, const float*,
                                     const float*, double*, double*, hipStream_t) {
    stub::check_fwd(a);
    stub::calls.push_back("state_scan_adj");
    return hipSuccess;
}
hipError_t launch_bwd_dz(const BwdArgs& a, bool, hipStream_t) {
    check_bwd(a);
    stub::calls.push_back("bwd_dz");
    return hipSuccess;
}
hipError_t launch_step_infinite(const StepArgs&, hipStream_t) {
    stub::calls.push_back("step_infinite");
    return hipSuccess;
}
hipError_t launch_phase_summary(const PhaseArgs&, hipStream_t) {
    stub::calls.push_back("phase_summary");
    return hipSuccess;
}
hipError_t launch_phase_carry(const PhaseArgs&, hipStream_t) {
    stub::calls.push_back("phase_carry");
    return hipSuccess;
}
hipError_t launch_phase_out(const PhaseArgs&, hipStream_t) {
    stub::calls.push_back("phase_out");
    return hipSuccess;
}
hipError_t launch_born(const BornArgs&, hipStream_t) {
    stub::calls.push_back("born");
    return hipSuccess;
}
hipError_t launch_fill(float*, const float*, int64_t, hipStream_t) {
    stub::calls.push_back("fill");
    return hipSuccess;
}
}  // namespace cssd
