// Host-side launchers of the cssd kernels (internal to libcssd.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cssd {

enum KernelId { K_CUMSUM = 0, K_CHUNK_STATE = 1, K_STATE_PASS = 2, K_CHUNK_SCAN = 3, K_STEP = 4,
                K_STEP_INFINITE = 5, K_COUNT = 6 };

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

struct StepArgs {
    int64_t B, H, D, N;
    int64_t nsteps = 1;  // constant-input steps applied at once (1: one decode step)
    const float *x_re, *x_im, *b_re, *b_im, *c_re, *c_im, *dt, *a_re, *a_im, *dskip;
    float *h_re, *h_im, *y_re, *y_im;
};

// Number of compute units of the current device (queried once per device).
hipError_t device_cu_count(int* cus);

// Each launcher enqueues one kernel on `stream` and returns hipGetLastError().
hipError_t launch_cumsum(const FwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_state(const FwdArgs& a, hipStream_t stream);
hipError_t launch_state_pass(const FwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t stream);
hipError_t launch_step(const StepArgs& a, hipStream_t stream);
hipError_t launch_step_infinite(const StepArgs& a, hipStream_t stream);

}  // namespace cssd
