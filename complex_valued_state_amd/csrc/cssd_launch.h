// Host-side launchers of the cssd kernels (internal to libcssd.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cssd {

enum KernelId { K_CUMSUM = 0, K_CHUNK_STATE = 1, K_STATE_PASS = 2, K_CHUNK_SCAN = 3, K_STEP = 4,
                K_STEP_INFINITE = 5, K_BWD_DX = 6, K_BWD_DC = 7, K_BWD_DZ = 8,
                K_PHASE_SUMMARY = 9, K_PHASE_CARRY = 10, K_PHASE_OUT = 11, K_BORN = 12,
                K_BWD_DB = 13, K_STATE_SCAN = 14, K_STATE_SCAN_ADJ = 15, K_FILL = 16,
                K_SCAN_FUSED = 17, K_WIDEN = 18, K_COUNT = 19 };

struct FwdArgs {
    int64_t B, T, H, D, N, C, nC;
    int in_dtype;  // 0 f32, 1 bf16
    const void *x_re, *x_im, *b_re, *b_im, *c_re, *c_im;
    const float *dt, *a_re, *a_im, *dskip, *h0_re, *h0_im;
    float *y_re, *y_im, *hT_re, *hT_im;
    // workspace regions
    double *acs_re, *acs_im;
    float *e_re, *e_im, *w_re, *w_im, *cd_re, *cd_im, *st_re, *st_im;
};

// The gradient pass: the forward problem and its workspace (f), the forward
// output and upstream gradients, the gradients, and the extra workspace.
struct BwdArgs {
    FwdArgs f;
    const float *dy_re, *dy_im;              // dL/dy
    const float *dhT_re, *dhT_im;            // dL/dhT or NULL
    float *dx_re, *dx_im, *db_re, *db_im, *dc_re, *dc_im, *ddt, *da_re, *da_im, *dd;
    float *dh0_re, *dh0_im;                  // or NULL
    // workspace
    float *r_re, *r_im;                      // adjoint chunk states Q_c, then R_{c+1}
    float *q1_re, *q1_im, *q2_re, *q2_im;    // per position: the dx and dC halves of q
    float *ddp;                              // per position: Re(dy . conj(x))
    const float *hT_re, *hT_im;              // the forward's final state (read only)
    double *z_re, *z_im;                     // per chunk, two partials: <R_{c+1}, H_{c+1}>
    double* pa;                              // per span of each (b, h): dA re, dA im, dDskip
};

struct StepArgs {
    int64_t B, H, D, N;
    int64_t nsteps = 1;  // constant-input steps applied at once (1: one decode step)
    const float *x_re, *x_im, *b_re, *b_im, *c_re, *c_im, *dt, *a_re, *a_im, *dskip;
    float *h_re, *h_im, *y_re, *y_im;
};

// The per-coordinate phase scan: HN = nheads * dstate coordinates per batch row,
// time cut into nch segments of L steps (the last one ragged).
struct PhaseArgs {
    int64_t B, T, HN, L, nch;
    const float *phi, *u, *b_re, *b_im, *psi0_re, *psi0_im;  // psi0 may be NULL
    float *psi_re, *psi_im, *psiT_re, *psiT_im;               // psiT may be NULL
    // workspace, [B, nch, HN] each (unused when nch == 1)
    float *p_re, *p_im, *s_re, *s_im, *in_re, *in_im;
};

// Causal Born attention over (B, T, H, D) planar q, k, v.  nqb query blocks of
// 64 rows (fp32) or 128 rows (bf16) per (b, h), taken in npair workgroups
// (blocks p and nqb - 1 - p);
// hpl heads share one 128-byte line of a time step and go to the same XCD.
struct BornArgs {
    int64_t B, T, H, D, nqb, npair, hpl;
    int in_dtype;  // 0: q, k, v float32; 1: bfloat16 bit patterns (read through the float pointers)
    const float *q_re, *q_im, *k_re, *k_im, *v_re, *v_im, *tau;  // tau may be NULL
    float *out_re, *out_im;
};

// Number of compute units of the current device (queried once per device).
hipError_t device_cu_count(int* cus);

// Each launcher enqueues one kernel on `stream` and returns hipGetLastError().
hipError_t launch_cumsum(const FwdArgs& a, hipStream_t stream);
// n bf16 values (16-byte aligned) widened to fp32 (16-byte aligned)
hipError_t launch_widen(const uint16_t* src, float* dst, int64_t n, hipStream_t stream);
// chunk states and the chunk-to-chunk pass fused (forward): writes H_c and hT
hipError_t launch_state_scan(const FwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t stream);
// the chunk states, the chunk-to-chunk pass and the output in one kernel that
// walks each (b, h)'s chunks (bf16 inputs at N = D = C = 64, where scan_fused holds)
bool scan_fused(const FwdArgs& a);
hipError_t launch_scan_fused(const FwdArgs& a, hipStream_t stream);
hipError_t launch_step(const StepArgs& a, hipStream_t stream);
hipError_t launch_chunk_state_adjoint(const FwdArgs& a, const float* dy_re, const float* dy_im,
                                      float* q_re, float* q_im, hipStream_t stream);
hipError_t launch_state_pass_adjoint(const FwdArgs& a, float* q_re, float* q_im,
                                     const float* dhT_re, const float* dhT_im, float* dh0_re,
                                     float* dh0_im, hipStream_t stream);
hipError_t launch_bwd_dx(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_db(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dc(const BwdArgs& a, hipStream_t stream);
// the adjoint chunk states and pass fused, with the log-decay boundary terms
// (shapes for which state_scan_adjoint_fused holds; hipErrorNotSupported else)
bool state_scan_adjoint_fused(const FwdArgs& a);
hipError_t launch_state_scan_adjoint(const FwdArgs& a, const float* dy_re, const float* dy_im,
                                     const float* dhT_re, const float* dhT_im, float* r_re,
                                     float* r_im, float* dh0_re, float* dh0_im,
                                     const float* hT_re, const float* hT_im, double* z_re,
                                     double* z_im, hipStream_t stream);
// with_zbound: compute the boundary terms <R_{c+1}, H_{c+1}> here (not yet done)
hipError_t launch_bwd_dz(const BwdArgs& a, bool with_zbound, hipStream_t stream);
hipError_t launch_step_infinite(const StepArgs& a, hipStream_t stream);
hipError_t launch_phase_summary(const PhaseArgs& a, hipStream_t stream);
hipError_t launch_phase_carry(const PhaseArgs& a, hipStream_t stream);
hipError_t launch_phase_out(const PhaseArgs& a, hipStream_t stream);
hipError_t launch_born(const BornArgs& a, hipStream_t stream);
// dst[0, n) = src[0, n), or zeros when src is NULL (the state and sums of an
// empty problem); nothing is launched for n <= 0 or dst == src
hipError_t launch_fill(float* dst, const float* src, int64_t n, hipStream_t stream);

}  // namespace cssd
