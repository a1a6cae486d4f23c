/*
 * cssd.h -- C ABI of libcssd.so: the complex-valued diagonal selective
 * state-space scan, computed in chunkwise form on AMD MI355X (gfx950), plus its
 * single-token recurrent decode step.
 *
 * The operation (Mamba-3-Lite docs, "SSD Theory -- Complex States & the
 * Chunkwise Algorithm", section 2, and "Complex-Valued State Spaces", "The
 * recurrence" and "Discretization"; the skip term D x follows the burn-mamba
 * "step_constant" module's readout):
 *
 *     abar_t = exp(softplus(dt_t) * A)          A: one complex scalar per head
 *     h_t    = abar_t * h_{t-1} + B_t (x) x_t   h_t: N x D complex per (batch, head)
 *     y_t    = sum_n C_t[n] * h_t[n, :] + D * x_t
 *
 * softplus acts on the real dt before the product with the complex A; C_t is
 * not conjugated; the outer product puts B_t on the state axis (N) and x_t on
 * the channel axis (D).  y is complex: both planes are returned.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Complex tensors are PLANAR: two separate, contiguous, row-major arrays
 *    (real plane, imaginary plane) of identical shape.  No interleaved data.
 *  - Every array pointer is a DEVICE pointer owned by the caller, C-contiguous
 *    with the shape given in its comment, and aligned as follows: arrays read
 *    or written as vectors (cssd_forward: B_*, C_*, h0_*, hT_*; cssd_step: x_*,
 *    h_*, y_*) to 16 bytes (8 bytes for bf16 B_*, C_*), every other array to
 *    its element size.  The library
 *    never allocates device memory, frees or synchronises; all work is enqueued
 *    on `stream` (a hipStream_t passed as void*; NULL = the legacy default
 *    stream) and is complete when that stream is.  Outputs are valid only after
 *    that point.  One exception to "on `stream`": a bf16-input cssd_forward at
 *    headdim = dstate = chunk = 64 with more (b, h) sequences than the GPU has
 *    CUs, but at most twice as many, runs part of its work on a second stream of
 *    the library's, which waits for `stream` before it starts, and which `stream`
 *    waits for afterwards (events), so the result is still complete when
 *    `stream` is, and graph capture of `stream` takes both in.  That stream and
 *    its two events are created on the first such call on a GPU and kept.
 *  - Validation is synchronous and host-side: bad arguments return an error
 *    status before anything is enqueued, and the library never reads device
 *    memory from the host.  Launch failures return CSSD_ERR_HIP.  No C++
 *    exception crosses this boundary.
 *  - Supported sizes of the scan entry points (cssd_forward, cssd_backward,
 *    cssd_step*): headdim D and dstate N in {16, 32, 64, 128} (each kernel is
 *    compiled per width; other multiples of 16 are not built: zero-padding x, B
 *    and C to the next supported width gives the same y and, in the leading
 *    block, the same state); chunk in
 *    {16, 32, 64, 128}; any seqlen >= 0 (a partial last chunk is masked inside
 *    the kernels, nothing is padded in memory); batch, nheads >= 0, with
 *    batch*seqlen*nheads*max(D,N) < 2^31 elements per plane and, for
 *    cssd_forward and cssd_backward, chunk*nheads*max(D,N) <= 2^30.  The phase scan
 *    and Born attention state their own limits.  Other sizes return
 *    CSSD_ERR_UNSUPPORTED.  There is one kernel path and no fallback.
 *  - Empty problems: batch, seqlen or nheads may be 0 in every entry point
 *    (seqlen where it has one).  Arrays with a zero extent are never accessed
 *    and may be NULL, and so may the workspace (its size is then 0).  What is
 *    left is what a scan of no time steps gives: the final state equals the
 *    initial one (cssd_forward's hT = h0, cssd_phase_scan's psiT = psi0; zero
 *    when the initial state is NULL), cssd_backward's dh0 = dhT (or zero) and
 *    its sums over batch and time, dA and dDskip, are zero.
 *  - Outputs must not alias inputs (except the decode state, updated in place).
 *  - The library keeps no per-call state and is safe to call from several host
 *    threads on different streams.  The optional profiler (cssd_profile_*)
 *    is process-wide and guarded by a lock.
 *  - Debugging: with CSSD_DEBUG_SYNC=1 in the environment when the library is
 *    first called, every entry point synchronises its stream after each kernel
 *    it launches and returns CSSD_ERR_HIP as soon as one reports an error (a
 *    stream being captured into a graph is not synchronised).  This is the one
 *    exception to "never synchronises" and is off by default.
 */
#ifndef CSSD_H
#define CSSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSSD_VERSION 108 /* major*100 + minor */

typedef enum cssd_status {
    CSSD_OK = 0,
    CSSD_ERR_INVALID_ARG = 1, /* null required pointer, negative size, misalignment, aliasing */
    CSSD_ERR_UNSUPPORTED = 2, /* sizes outside the supported set */
    CSSD_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned */
    CSSD_ERR_HIP = 4,         /* a HIP launch or runtime call failed */
    CSSD_ERR_TOO_LARGE = 5    /* cssd_forward_noalloc: the workspace would exceed its fixed array */
} cssd_status;

typedef enum cssd_dtype {
    CSSD_F32 = 0,  /* x, B, C planes are float32 */
    CSSD_BF16 = 1  /* x, B, C planes are bfloat16 bit patterns (uint16); all else float32 */
} cssd_dtype;

/* Library version, CSSD_VERSION of the build. */
int cssd_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *cssd_status_string(int status);

/*
 * Bytes of device workspace cssd_forward needs for this shape (written to
 * *bytes).  Passage: the chunk states and the chunk-level scan of the SSD
 * decomposition (Mamba-3-Lite docs, "SSD Theory" 4.5): the workspace holds one
 * N x D complex state per chunk and the chunk-local cumulative log-decay; the
 * C x C segment matrix L is never materialised (it lives in registers), so no
 * term grows like 8*B*T*H*C bytes ("SSD Theory" section 5).
 *
 * Layout (nC = ceil(T/C), P = nC*C padded positions, every region 256-byte
 * aligned, in this order; a caller may read it after the stream completes,
 * except after a bf16-input call with headdim = dstate = chunk = 64, which runs
 * as one kernel that keeps these quantities on chip and writes nothing here):
 *   acs_re, acs_im : double [B][H][P]     inclusive chunk-local cumsum of
 *                                         softplus(dt)*A (0 increments on
 *                                         padded positions), real part in log2
 *                                         units (/ln 2), imaginary in turns (/2pi)
 *   e_re,  e_im    : float  [B][H][P]     exp(acs[l])
 *   w_re,  w_im    : float  [B][H][P]     exp(acs[C-1] - acs[l])
 *   cd_re, cd_im   : float  [B][H][nC]    exp(acs[C-1]) (chunk decay)
 *   st_re, st_im   : float  [B][H][nC][N*D]  chunk end states S_c, replaced
 *                                         in place by the carry-in states H_c
 *                                         (the state after step cC-1); each
 *                                         N x D block in MFMA-fragment order:
 *                                         element (n, p) at
 *                                         (((n/16)(D/16) + p/16)*4 + (n%16)/4)*64
 *                                         + (p%16)*4 + n%4
 * Returns CSSD_OK, CSSD_ERR_INVALID_ARG (null bytes / negative size) or
 * CSSD_ERR_UNSUPPORTED.
 */
int cssd_forward_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                int64_t headdim, int64_t dstate, int64_t chunk,
                                size_t *bytes);

/*
 * Chunkwise forward over a whole sequence (Mamba-3-Lite docs, "SSD Theory"
 * section 4 and "The Chunkwise Complex SSD Algorithm" section 4): per chunk,
 * the cumulative log-decay, the causal segment matrix
 * L[l,s] = exp(acs[l]-acs[s]) 1[l>=s], the intra-chunk term (C B^T . L) X, the
 * chunk end state, a T/C-step pass carrying the state between chunks, and the
 * output combine Y_diag + exp(acs) C H_c + D x.  The result equals the
 * sequential recurrence above (the SSD decomposition is exact; only rounding
 * order differs).
 *
 *   in_dtype         CSSD_F32 or CSSD_BF16 (applies to x, B, C planes only)
 *   x_re, x_im       [B,T,H,D]   input channels
 *   B_re, B_im       [B,T,H,N]   input coupling B_t
 *   C_re, C_im       [B,T,H,N]   readout C_t
 *   dt               [B,T,H]     float32 raw step; softplus is applied inside
 *   A_re, A_im       [H]         float32 per-head complex rate
 *   Dskip            [H]         float32 skip weight, or NULL for D = 0
 *   h0_re, h0_im     [B,H,N,D]   float32 initial state, or both NULL for zero
 *   y_re, y_im       [B,T,H,D]   float32 output (written)
 *   hT_re, hT_im     [B,H,N,D]   float32 state after step T-1 (written), or
 *                                both NULL.  Same layout as cssd_step's state,
 *                                so a prefill hands over to decode directly.
 *   workspace        device buffer of >= cssd_forward_workspace_size bytes,
 *                    256-byte aligned; contents on entry are ignored.
 *   stream           hipStream_t (as void*), or NULL.
 * Padded positions of a partial last chunk contribute nothing and do not
 * decay hT.  Returns CSSD_OK or an error status (nothing enqueued on error,
 * except CSSD_ERR_HIP, which may leave earlier kernels of the call enqueued).
 */
int cssd_forward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                 int64_t dstate, int64_t chunk, int32_t in_dtype,
                 const void *x_re, const void *x_im,
                 const void *B_re, const void *B_im,
                 const void *C_re, const void *C_im,
                 const float *dt, const float *A_re, const float *A_im,
                 const float *Dskip,
                 const float *h0_re, const float *h0_im,
                 float *y_re, float *y_im,
                 float *hT_re, float *hT_im,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * cssd_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, result and errors as cssd_forward, minus the workspace: it runs in
 * a fixed device array of CSSD_NOALLOC_SCRATCH_BYTES (64 MiB) inside the
 * library, one per GPU, held from the first call on that GPU until the process
 * ends.  The call allocates nothing itself (its first call on a GPU looks the
 * array's address up once, and the first bf16 call in the two-stream shape
 * described above creates that stream and its events); the caller still owns
 * every input and output.
 * A problem whose cssd_forward_workspace_size exceeds the array returns
 * CSSD_ERR_TOO_LARGE before anything is enqueued (at D = N = chunk = 64 the
 * array holds about 1,900 chunks, batch * nheads * ceil(seqlen / chunk)).
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (on different streams, or from several host threads) race on it and
 * must be ordered by the caller; calls on one stream are ordered already.  The
 * array needs no clearing between calls (every region is written before it is
 * read); it holds the last call's workspace contents afterwards.
 */
#define CSSD_NOALLOC_SCRATCH_BYTES (64u << 20)
int cssd_forward_noalloc(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                         int64_t dstate, int64_t chunk, int32_t in_dtype,
                         const void *x_re, const void *x_im,
                         const void *B_re, const void *B_im,
                         const void *C_re, const void *C_im,
                         const float *dt, const float *A_re, const float *A_im,
                         const float *Dskip,
                         const float *h0_re, const float *h0_im,
                         float *y_re, float *y_im,
                         float *hT_re, float *hT_im, void *stream);

/*
 * One recurrent decode step for every (batch, head), state updated in place
 * (the loop body of the sequential scan, Mamba-3-Lite docs, "Complex-Valued
 * State Spaces", walkthrough of the naive scan; fixed-size state, no cache of
 * past tokens):
 *     h <- exp(softplus(dt) A) h + B (x) x ;   y = sum_n C[n] h[n,:] + D x
 *
 *   x_re, x_im   [B,H,D]     float32
 *   B_re, B_im   [B,H,N]     float32
 *   C_re, C_im   [B,H,N]     float32
 *   dt           [B,H]       float32 raw step
 *   A_re, A_im   [H]         float32
 *   Dskip        [H] or NULL
 *   h_re, h_im   [B,H,N,D]   float32 state, read and overwritten
 *   y_re, y_im   [B,H,D]     float32 output
 * Returns CSSD_OK or an error status.
 */
int cssd_step(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
              const float *x_re, const float *x_im,
              const float *B_re, const float *B_im,
              const float *C_re, const float *C_im,
              const float *dt, const float *A_re, const float *A_im,
              const float *Dskip,
              float *h_re, float *h_im,
              float *y_re, float *y_im, void *stream);

/*
 * Workspace bytes cssd_backward needs for this shape (at least the forward's),
 * with fp32 inputs.
 */
int cssd_backward_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                 int64_t headdim, int64_t dstate, int64_t chunk,
                                 size_t *bytes);

/*
 * Workspace bytes cssd_backward needs for this shape with inputs of in_dtype:
 * for CSSD_F32 as cssd_backward_workspace_size; for CSSD_BF16 that plus the fp32
 * copies of x, B, C it widens the inputs into (4 bytes an element, 2 planes each,
 * each rounded up to 256 bytes).  Returns CSSD_ERR_INVALID_ARG for another
 * in_dtype or a NULL bytes, and the shape checks of cssd_backward_workspace_size.
 */
int cssd_backward_workspace_size_dtype(int64_t batch, int64_t seqlen, int64_t nheads,
                                       int64_t headdim, int64_t dstate, int64_t chunk,
                                       int32_t in_dtype, size_t *bytes);

/*
 * Gradients of cssd_forward (the pages train the scan by automatic
 * differentiation of complex tensors: Mamba-3-Lite docs, "SSD Theory", autograd
 * notes; "The Chunkwise Complex SSD Algorithm", the complex-dtype
 * requirement).  For a real loss L and a complex value u + i v the gradient is
 * the planar pair (dL/du, dL/dv), which is also the convention of complex
 * autograd (grad = dL/du + i dL/dv).  Given the upstream gradients dy of y and,
 * optionally, dhT of the final state, this returns dx, dB, dC (the layouts of
 * x, B, C), ddt [B,T,H], dA [H] and dDskip [H] (summed over batch and time), and
 * dh0 [B,H,N,D].
 *
 *   x_* .. h0_*      exactly the inputs of the cssd_forward call.  With
 *                    in_dtype CSSD_BF16 (the bf16-input setting of the pages'
 *                    training: the phase-state paper, §7, training protocol)
 *                    x, B, C are bf16 planes: they are widened to fp32 once into
 *                    the workspace (which must then hold
 *                    cssd_backward_workspace_size_dtype bytes) and the gradients
 *                    are those of the scan at exactly the rounded values, in fp32
 *   y_re, y_im       not read, may be NULL (that call's output y has a place in
 *                    the signature; the gradients need only the inputs, see
 *                    below)
 *   dy_re, dy_im     [B,T,H,D] upstream gradient of y
 *   dhT_re, dhT_im   [B,H,N,D] upstream gradient of the final state, or both
 *                    NULL (zero)
 *   dx_*, dB_*, dC_* gradients of x, B, C (written)
 *   ddt              [B,T,H] gradient of the raw step dt (written)
 *   dA_re, dA_im     [H] gradient of A (written)
 *   dD               [H] gradient of Dskip, or NULL (not computed)
 *   dh0_re, dh0_im   [B,H,N,D] gradient of the initial state, or both NULL
 *   workspace        >= cssd_backward_workspace_size bytes, 256-byte aligned
 * The forward's chunk states are recomputed inside.  The log-decay gradient
 * dz_t (z_t = softplus(dt_t) A) uses the identity
 *   dz_t = sum_{l>=t} [dy_l . conj(y_l - D x_l) - conj(x_l) . (dx_l - D dy_l)]
 *          + <dhT, hT>,
 * obtained by summing the reverse recurrence of dL/dh_t (<u, v> = sum u conj(v)),
 * with dy_l . conj(y_l - D x_l) taken as conj(C_l) . dC_l (y_l - D x_l = C_l h_l,
 * dC_l = dy_l conj(h_l)).  So y is never read, and the gradients do not take the
 * rounding of the forward that produced it: those sums cancel, and a bf16
 * forward's y would make ddt and dA several percent wrong.
 * Alignment: x, B, C, dy (and h0, dhT, dh0) 16 bytes (bf16 planes too), the
 * rest their element size.  Outputs may not alias inputs or each other.
 * Launches with bf16 inputs: six widen launches, then the kernels of the fp32
 * call.
 */
int cssd_backward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                  int64_t dstate, int64_t chunk, int32_t in_dtype,
                  const void *x_re, const void *x_im,
                  const void *B_re, const void *B_im,
                  const void *C_re, const void *C_im,
                  const float *dt, const float *A_re, const float *A_im,
                  const float *Dskip,
                  const float *h0_re, const float *h0_im,
                  const float *y_re, const float *y_im,
                  const float *dy_re, const float *dy_im,
                  const float *dhT_re, const float *dhT_im,
                  float *dx_re, float *dx_im, float *dB_re, float *dB_im,
                  float *dC_re, float *dC_im, float *ddt,
                  float *dA_re, float *dA_im, float *dD,
                  float *dh0_re, float *dh0_im,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * cssd_backward without the forward recomputation: the caller ran cssd_forward
 * for these same inputs and chunk on `workspace` (a buffer of at least
 * cssd_backward_workspace_size bytes; the backward's layout begins with the
 * forward's), left it untouched since, and passes that call's final state.  The
 * cumsums and chunk states the forward stored there are used as they are (the
 * autograd of the pages keeps forward tensors for the gradient in the same
 * way: Mamba-3-Lite docs, "SSD Theory", autograd notes), which saves the
 * recomputation's launches (ids 0 and 14).  The gradients are bit-identical to
 * cssd_backward's for the same inputs.
 *   y_re, y_im     not read, may be NULL (as in cssd_backward)
 *   hT_re, hT_im   [B,H,N,D] the forward's final state; required when dhT is
 *                  given (it enters <dhT, hT>), else may be NULL
 * Every other argument as cssd_backward, except that in_dtype must be CSSD_F32
 * (else CSSD_ERR_UNSUPPORTED: the bf16-input forward keeps no chunk states).  A
 * workspace that does not hold that forward's results gives undefined gradients
 * (this is not detected).
 */
int cssd_backward_saved(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int64_t chunk, int32_t in_dtype,
                        const void *x_re, const void *x_im,
                        const void *B_re, const void *B_im,
                        const void *C_re, const void *C_im,
                        const float *dt, const float *A_re, const float *A_im,
                        const float *Dskip,
                        const float *h0_re, const float *h0_im,
                        const float *y_re, const float *y_im,
                        const float *hT_re, const float *hT_im,
                        const float *dy_re, const float *dy_im,
                        const float *dhT_re, const float *dhT_im,
                        float *dx_re, float *dx_im, float *dB_re, float *dB_im,
                        float *dC_re, float *dC_im, float *ddt,
                        float *dA_re, float *dA_im, float *dD,
                        float *dh0_re, float *dh0_im,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * n recurrent steps that all receive the same input, applied at once in O(1)
 * work per state element (burn-mamba docs, module step_constant: the unrolled
 * constant-input steps form a geometric series; this is its case with no
 * rotation between steps and unit input weight):
 *     a = exp(softplus(dt) A)
 *     h <- a^n h + (1 - a^n) / (1 - a) * B (x) x      (the ratio is n when a = 1)
 *     y  = sum_n C[n] h[n,:] + D x                    (the n-th step's output)
 * Arguments and layouts as cssd_step, plus nsteps >= 1 (else
 * CSSD_ERR_INVALID_ARG); nsteps = 1 is exactly cssd_step.  a^n and the ratio are
 * formed per (batch, head) in fp64, the ratio as expm1(n z) / expm1(z) with
 * z = softplus(dt) A (accurate as a -> 1), the phases reduced mod 2 pi (so
 * rotation angles stay exact to about 1e-16 * n |z| radians).
 */
int cssd_step_n(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                int64_t nsteps,
                const float *x_re, const float *x_im,
                const float *B_re, const float *B_im,
                const float *C_re, const float *C_im,
                const float *dt, const float *A_re, const float *A_im,
                const float *Dskip,
                float *h_re, float *h_im,
                float *y_re, float *y_im, void *stream);

/*
 * The stationary output of an endless constant input, the limit of
 * cssd_step_n's y as n grows (burn-mamba docs, module step_constant: the
 * fixed point, which no starting state influences):
 *     y = (sum_n C[n] B[n]) / (1 - a) * x + D x
 * Meaningful for |a| < 1, i.e. softplus(dt) Re A < 0; otherwise the series
 * does not converge and the formula's value is returned (inf or NaN where
 * a = 1).  No state is read or written.  Arguments and layouts as cssd_step
 * without h_re, h_im.
 */
int cssd_step_infinite(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                       const float *x_re, const float *x_im,
                       const float *B_re, const float *B_im,
                       const float *C_re, const float *C_im,
                       const float *dt, const float *A_re, const float *A_im,
                       const float *Dskip,
                       float *y_re, float *y_im, void *stream);

/*
 * The per-coordinate complex recurrence of the phase-state paper ("Complex
 * Phase-State Dynamics Reduce the Optimization Steps of Sequence Models",
 * section 5.2, eq. 2 and 3): every coordinate k of every (batch, head) row
 * evolves on its own,
 *     lambda = (1 + i phi) / (1 - i phi)    (Cayley transform, |lambda| = 1)
 *     alpha  = 1 / (1 + exp(-u))            (gate in (0, 1))
 *     psi_t  = alpha_t lambda_t psi_{t-1} + b_t
 * and every state psi_1..psi_T is returned.  The evaluation follows section
 * 5.3: time is cut into segments, each segment's end state seeds the next.
 * Arguments (device pointers, fp32, planar complex, row-major):
 *   phi, u          [B,T,H,N] phase parameter and gate logit (any finite values)
 *   b_re, b_im      [B,T,H,N] input term b_t
 *   psi0_re/_im     [B,H,N] initial state, or both NULL (zero)
 *   psi_re, psi_im  [B,T,H,N] the state after each step (written)
 *   psiT_re/_im     [B,H,N] the final state, or both NULL (not written); may be
 *                   the same arrays as psi0_re/_im (the state advances in place)
 *   chunk           segment length in steps; 0 lets the library choose (the
 *                   whole sequence in one pass when batch*H*N >= 65536, else
 *                   shorter segments for parallelism); chunk >= seqlen is one
 *                   pass.  The result is the same up to rounding.
 *   workspace       >= cssd_phase_scan_workspace_size bytes (0 for one pass,
 *                   then workspace may be NULL), 256-byte aligned
 * Within a segment the recurrence is stepped forward in fp32; no reciprocal of a
 * cumulative product is formed, so the page's floor on the log-magnitude of
 * that product is not needed and the trajectory is exact up to rounding, also
 * where the product underflows.  Limits: batch*seqlen*H*N < 2^40.  Alignment:
 * element size.  Outputs may not alias inputs except psiT on psi0.
 */
int cssd_phase_scan_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                   int64_t dstate, int64_t chunk, size_t *bytes);
int cssd_phase_scan(int64_t batch, int64_t seqlen, int64_t nheads, int64_t dstate,
                    int64_t chunk,
                    const float *phi, const float *u,
                    const float *b_re, const float *b_im,
                    const float *psi0_re, const float *psi0_im,
                    float *psi_re, float *psi_im,
                    float *psiT_re, float *psiT_im,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Causal Born attention of the phase-state paper ("Complex Phase-State Dynamics
 * Reduce the Optimization Steps of Sequence Models", section 5.5, eq. 5, and
 * Appendix A, Algorithm 3), for every (batch, head):
 *     s_ij  = |<q_i|k_j>|^2 / (D tau_i)   for j <= i,  <q|k> = sum_d conj(q_d) k_d
 *     psi_i = (sum_{j<=i} s_ij v_j) / (sum_{j<=i} s_ij)
 * a causal average of the values weighted by the squared modulus of the complex
 * overlap (no softmax).  Accumulation is fp32 throughout.
 * Arguments (device pointers, planar complex, row-major):
 *   q_*, k_*, v_*   [B,T,H,D] queries, keys, values: float32 (CSSD_F32) or
 *                   bfloat16 bit patterns (CSSD_BF16; the page's half-precision
 *                   setting: products on the bf16 matrix cores, accumulation in
 *                   fp32, the weights rounded to bf16 before they multiply the
 *                   values and the normaliser summing those rounded weights)
 *   tau             [B,T,H] float32 temperatures, or NULL (all 1).  tau_i and D
 *                   scale every score of row i alike and so cancel in the
 *                   normalisation; they change only rounding.
 *   out_re, out_im  [B,T,H,D] float32 psi (written)
 * Supported: headdim D in {16, 32, 64}; any seqlen >= 0; batch*nheads*seqlen*D
 * < 2^40.  A row whose scores are all zero (its query orthogonal to every key
 * up to it, e.g. a zero query) is returned as zero.  Alignment: q, k, v, out
 * 16 bytes, tau 4.  Accuracy: fp32 inputs agree with the exact result to about
 * 1e-6 relative; bf16 inputs to about 1e-2 (bf16 rounding of the scaled queries
 * and of the weights).  Outputs may not alias inputs or each other.
 */
int cssd_born_attention(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int32_t in_dtype,
                        const void *q_re, const void *q_im,
                        const void *k_re, const void *k_im,
                        const void *v_re, const void *v_im,
                        const float *tau,
                        float *out_re, float *out_im, void *stream);

/*
 * Optional per-kernel timing (a measurement aid, not part of the operation).
 * While enabled, every kernel launch of every entry point is bracketed by
 * two hipEvents recorded on the caller's stream.  cssd_profile_read waits for
 * the recorded events, writes the accumulated milliseconds and launch counts
 * per kernel id into ms[k] and launches[k] for k < min(capacity, number of
 * kernels), resets the accumulators and returns the number of kernel ids (or a
 * negative status on error).  Kernel ids: 0 cumsum, 1 chunk_state,
 * 2 state_pass, 3 chunk_scan, 4 step (also cssd_step_n), 5 step_infinite,
 * 14 state_scan (cssd_forward: the chunk states fused with the state pass),
 * 6 bwd_dx, 7 bwd_dc, 8 bwd_dz, 13 bwd_db (cssd_backward also runs ids 0 and 14,
 * cssd_backward_saved does not; both then run 15 state_scan_adj, the adjoint chunk states and pass fused, where
 * dstate = headdim = chunk = 64, else 1 and 2 in their adjoint modes), 9 phase_summary,
 * 10 phase_carry, 11 phase_out (cssd_phase_scan), 12 born (cssd_born_attention),
 * 16 fill (the states and zeroed sums of an empty problem, one launch per plane),
 * 17 scan_fused (cssd_forward with bf16 inputs at headdim = dstate = chunk = 64),
 * 18 widen (cssd_backward with bf16 inputs: one launch per widened plane).
 * cssd_kernel_name(k) gives the device symbol stem of each id (NULL if out of
 * range).
 * Launches on a stream that is being captured into a HIP graph are not
 * bracketed (the events would be captured with the kernels and would time no
 * replay): they are neither timed nor counted.  cssd_profile_read waits for the
 * events without holding the library's lock, so other threads keep launching
 * meanwhile; launches bracketed after it took the pending list are left for
 * the next read.
 */
int cssd_profile_enable(int on);
int cssd_profile_read(double *ms, int64_t *launches, int capacity);
const char *cssd_kernel_name(int kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* CSSD_H */
