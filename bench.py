"""Throughput of the complex chunkwise scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]

One step = one cssd_forward over the Mamba-style layer workload (batch 8,
T = 2048, 48 heads, head dim 64, state 64, chunk 64, fp32 complex planes): the
discretise + chunk-local cumsum, the chunk states with the inter-chunk state
pass (one fused kernel) and the intra-chunk output with the combine, all in the
library's HIP kernels.
Inputs are seeded synthetic data already resident in HBM when timing starts.
Each timed call first runs untimed for 200 ms (the GPU clocks settle), then W
warm-up calls, then exactly K timed calls.  Prints ONE JSON line.  Per-kernel
durations come from HIP events the library records around each launch on the
launch stream, during a second timed pass of the same K calls.

Extra figures in the same line: the bf16-input variant of the same workload, the
backward pass of the same workload (recomputing the forward's states, and on the
states a forward call saved), the decode step at batch 256 x 48 heads x
N128 x D64 over 512 pre-staged tokens, the constant-input calls at that shape,
the per-coordinate phase-state scan at 256 x 1024 x 16 x 16, causal Born
attention at 256 x 1024 x 16 heads x width 16, and the other forward
workloads (the tiny 64-step one, the long sequence and the phase-associative
memory), each with the oracle timed beside it on a bounded sample.  Step
times are taken with the per-kernel profiler off; the per-kernel averages come
from a second, profiled pass of the same K calls.  "traffic" figures are
HBM bytes per launch from committed rocprofv3 counter runs (profiles/traffic.json),
null once the kernel's sources have changed since.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "complex SSD fwd tokens/s at B8 T2048 H48; % of MFMA/HBM roofline"
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E peak
PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
# source files that make up each kernel (besides the shared device/launch headers),
# by the kernel's name stem as rocprofv3 reports it
_SCAN_SRC = ("k_chunk_scan.h", "k_chunk_scan_lds.h", "k_chunk_scan_bf16.h", "k_chunk_scan_nb.h",
             "k_chunk_scan_wide.h", "k_chunk_scan.hip",
             "k_chunk_scan_c16.hip", "k_chunk_scan_c32.hip", "k_chunk_scan_c64.hip",
             "k_chunk_scan_c128.hip")
KERNEL_SRC = {"k_chunk_scan": _SCAN_SRC, "k_chunk_scan_lds": _SCAN_SRC, "k_chunk_scan_nb": _SCAN_SRC,
              "k_chunk_scan_wide": _SCAN_SRC,
              "k_chunk_scan_bf16": _SCAN_SRC,
              "k_chunk_state": ("k_chunk_state.hip",), "k_state_pass": ("k_state_pass.hip",),
              "k_cumsum": ("k_cumsum.hip",), "k_step": ("k_step.hip",),
              "k_step_infinite": ("k_step.hip",),
              "k_bwd_tiles": ("k_backward.hip",), "k_bwd_zbound": ("k_backward.hip",),
              "k_bwd_lds": ("k_backward.hip", "k_chunk_scan_lds.h"),
              "k_bwd_dc_lds": ("k_backward.hip", "k_chunk_scan_lds.h"),
              "k_bwd_dz": ("k_backward.hip",), "k_bwd_reduce": ("k_backward.hip",),
              "k_phase_summary": ("k_phase_scan.hip",), "k_phase_carry": ("k_phase_scan.hip",),
              "k_phase_out": ("k_phase_scan.hip",), "k_born": ("k_born.hip",),
              "k_born_bf16": ("k_born.hip",), "k_state_scan": ("k_state_scan.hip",),
              "k_state_scan_lds": ("k_state_scan.hip",), "k_state_scan_mm": ("k_state_scan.hip",),
              "k_state_scan_cp": ("k_state_scan.hip",),
              "k_scan_fused_bf16": ("k_scan_fused_bf16.hip",), "k_widen": ("k_widen.hip",)}


# ---------------------------------------------------------------------------
# algorithmic work: what the method must read, write and multiply, not what the kernels do
# ---------------------------------------------------------------------------
def chunk_scan_flops(B, T, H, D, N, C):
    """Real flops one k_chunk_scan launch must do: per chunk, the causal score
    G = C B^T on the lower triangle incl. the diagonal (C(C+1)/2 x N complex MACs),
    the masked product with X (C(C+1)/2 x D), and the carried-state readout
    (C x N x D); 8 real flops per complex MAC."""
    nC = math.ceil(T / C)
    tri = C * (C + 1) // 2
    return 8 * B * H * nC * (tri * N + tri * D + C * N * D)


def chunk_state_flops(B, T, H, D, N, C):
    nC = math.ceil(T / C)
    return 8 * B * H * nC * C * N * D


def state_scan_hbm_bytes(B, T, H, D, N, C, in_bytes=4):
    """The fused chunk-state scan: read the B and X rows once, write every carry-in
    state H_c and the final state (fp32)."""
    nC = math.ceil(T / C)
    return B * T * H * (N + D) * 2 * in_bytes + B * H * (nC + 1) * N * D * 2 * 4


def cumsum_hbm_bytes(B, T, H, C):
    """Read dt (4 bytes) and write the fp64 cumsum, exp(acs) and w (32 bytes) per
    position, plus the chunk decay (8 bytes) per chunk."""
    nC = math.ceil(T / C)
    return B * T * H * 4 + B * H * nC * C * 32 + B * H * nC * 8


def forward_hbm_bytes(B, T, H, D, N, in_bytes=4):
    """Read x, B, C, dt once; write y and the final state once."""
    return (B * T * H * (D + 2 * N) * 2 * in_bytes + B * T * H * 4
            + B * T * H * D * 2 * 4 + B * H * N * D * 2 * 4)


def scan_fused_hbm_bytes(B, T, H, D, N, in_bytes=2):
    """The one-kernel forward after the cumsum: read x, B, C once, write y and the
    final state once (dt is read by the cumsum kernel)."""
    return (B * T * H * (D + 2 * N) * 2 * in_bytes + B * T * H * D * 2 * 4
            + B * H * N * D * 2 * 4)


def decode_hbm_bytes(B, H, D, N):
    """Per token: read and write the state, read x, B, C, dt, write y."""
    return B * H * N * D * 2 * 4 * 2 + B * H * (2 * D + 2 * N) * 2 * 4 + B * H * 4


def phase_scan_hbm_bytes(B, T, H, N):
    """Read phi, u, b (16 bytes) and write psi (8 bytes) per coordinate and step;
    read psi0 and write psiT once."""
    return B * T * H * N * 24 + B * H * N * 16


def born_flops(B, T, H, D):
    """Real flops of causal Born attention: per (query, key <= query) pair the
    complex overlap (D complex MACs, 8 flops each), its squared modulus (3), the
    weighted value sum (D real-by-complex MACs, 4 flops each) and the normaliser (1)."""
    return B * H * (T * (T + 1) // 2) * (12 * D + 4)


def chunk_scan_symbol(N, D, C, dtype):
    """The kernel the library launches for the chunk-scan step at this shape (the
    rule of launch_chunk_scan_c: the n-blocked staged kernels for fp32 inputs at
    C = 64 or 128, N = 128, D = 64; the LDS-staged kernel for fp32 inputs with
    C <= 64, C*N <= 4096, D <= 64 and not (C = 64, D = 16)), as rocprofv3 names it."""
    if dtype == "f32" and C == 64 and N == 128 and D == 64:
        return "k_chunk_scan_nb<64, 128, 64>"
    if dtype == "f32" and C == 128 and N == 128 and D == 64:
        return "k_chunk_scan_wide<128, 128, 64>"
    if dtype == "f32" and C <= 64 and C * N <= 4096 and D <= 64 and not (C == 64 and D == 16):
        return f"k_chunk_scan_lds<{C}, {N}, {D}>"
    return f"k_chunk_scan<cssd::In{'F32' if dtype == 'f32' else 'BF16'}, {C}, {N}, {D}>"


def src_hash(symbol):
    """Hash of the sources of the kernel named `symbol` (its stem before any '<')."""
    d = os.path.join(ROOT, "complex_valued_state_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SRC[symbol.split("<")[0]] + ("cssd_device.h", "cssd_launch.h"):
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(symbol):
    """HBM bytes per launch of the kernel `symbol` (as rocprofv3 names it) from the
    committed counter runs over this benchmark, or None when there are none or the
    kernel's sources changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(symbol)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("src_sha256_16") != src_hash(symbol):
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _to_dev(inp, dev):
    import numpy as np
    import torch
    io = torch.bfloat16 if inp.in_dtype == "bf16" else torch.float32
    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    return [t(inp.x_re, io), t(inp.x_im, io), t(inp.B_re, io), t(inp.B_im, io), t(inp.C_re, io),
            t(inp.C_im, io), t(inp.dt), t(inp.A_re), t(inp.A_im),
            None if inp.Dskip is None else t(inp.Dskip)]


SETTLE_S = 0.2


def settle(call, dev, seconds=SETTLE_S):
    """Run `call` untimed for `seconds` of wall time before the warm-up steps.  An
    idle GPU (it waits while the host draws the inputs) takes tens of milliseconds
    of work to reach its steady clocks, longer than a few warm-up calls: measured
    on the forward workload, 0.87 ms per step in the first 20 steps after five
    warm-up calls and 0.78 ms once settled."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            call()
        torch.cuda.synchronize(dev)


def time_forward(inp, steps, warmup, dev):
    """Times K forward calls twice after the settle and warm-up calls: first with
    the per-kernel profiler off (the step time reported), then with it on (each
    launch bracketed by two HIP events on its stream: the per-kernel averages).
    Returns (ms per step, {kernel: avg ms per launch}, ms per step profiled)."""
    import torch
    import complex_valued_state_amd as cssd
    s = inp.shape
    args = _to_dev(inp, dev)
    y_re = torch.empty((s["B"], s["T"], s["H"], s["D"]), dtype=torch.float32, device=dev)
    y_im = torch.empty_like(y_re)
    h_re = torch.empty((s["B"], s["H"], s["N"], s["D"]), dtype=torch.float32, device=dev)
    h_im = torch.empty_like(h_re)
    ws = torch.empty(cssd.cssd_forward_workspace_size(s["B"], s["T"], s["H"], s["D"], s["N"],
                                                      s["C"]), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    run = lambda: cssd.cssd_forward(*args, None, chunk=s["C"], out=(y_re, y_im, h_re, h_im),
                                    workspace=ws, stream=stream)
    settle(run, dev)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    total_ms = e0.elapsed_time(e1)
    with cssd.profile() as prof:
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize(dev)
    prof_ms = e0.elapsed_time(e1)
    kern = {k: prof.ms[k] / prof.launches[k] for k in prof.ms if prof.launches[k]}
    del args, ws
    return total_ms / steps, kern, prof_ms / steps


def forward_entry(inp, steps, warmup, dev, cpu_budget_s=None):
    """One forward workload: tokens/s, ms per step (profiler off), the per-kernel
    averages (profiled pass), the chunk-scan kernel's roofline object, the whole
    forward's fractions and, with a budget, the oracle on the host beside it."""
    import torch
    sh = inp.shape
    B, T, H, D, N, C = sh["B"], sh["T"], sh["H"], sh["D"], sh["N"], sh["C"]
    dtype = "bf16" if inp.in_dtype == "bf16" else "f32"
    ms, kern, ms_prof = time_forward(inp, steps, warmup, dev)
    k2_flops = chunk_scan_flops(B, T, H, D, N, C)
    fwd_flops = k2_flops + chunk_state_flops(B, T, H, D, N, C)
    in_bytes = 2 if dtype == "bf16" else 4
    hbm = forward_hbm_bytes(B, T, H, D, N, in_bytes=in_bytes)
    peak = PEAK_BF16_MFMA_TFLOPS if dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
    if "k_scan_fused" in kern:
        # one kernel does the chunk states, the chunk-to-chunk pass and the output:
        # HBM binds it; its algorithmic bytes are the forward's without dt
        f_ms = kern["k_scan_fused"]
        f_bytes = scan_fused_hbm_bytes(B, T, H, D, N, in_bytes)
        f_gbs = f_bytes / (f_ms * 1e-3) / 1e9
        # the launch shapes the library's launcher chooses: eight-wave workgroups
        # when every sequence has a CU of its own; up to two sequences a CU, whole
        # four-wave workgroups beside half-width ones on a second stream (the
        # profiler's time and the traffic cover both kernels); else four waves
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        if B * H <= cus:
            fsyms = ["k_scan_fused_bf16<8, false>"]
        elif B * H <= 2 * cus:
            fsyms = ["k_scan_fused_bf16<4, false>", "k_scan_fused_bf16<4, true>"]
        else:
            fsyms = ["k_scan_fused_bf16<4, false>"]
        tr = [load_traffic(x) for x in fsyms]
        roof = {"bound": "hbm", "kernel": "k_scan_fused", "symbol": " + ".join(fsyms),
                "achieved": round(f_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(f_gbs / PEAK_HBM_GBS, 4),
                "traffic": None if None in tr else sum(tr),
                "algorithmic_bytes_per_launch": f_bytes, "avg_launch_ms": round(f_ms, 5),
                "mfma_frac": round(fwd_flops / (f_ms * 1e-3) / 1e12 / peak, 4)}
    else:
        k2_ms = kern.get("k_chunk_scan")
        sym = chunk_scan_symbol(N, D, C, dtype)
        k2_achieved = k2_flops / (k2_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "k_chunk_scan", "symbol": sym,
                "achieved": round(k2_achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(k2_achieved / peak, 4), "traffic": load_traffic(sym),
                "algorithmic_flops_per_launch": k2_flops, "avg_launch_ms": round(k2_ms, 5)}
    e = {"tokens_per_s": round(B * T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
         "ms_per_step_profiled": round(ms_prof, 4),
         "kernels_avg_ms": {k: round(v, 5) for k, v in kern.items()},
         "roofline": roof,
         "forward_mfma_frac": round(fwd_flops / (ms * 1e-3) / 1e12 / peak, 4),
         "forward_hbm_frac": round(hbm / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
         "algorithmic_bytes": hbm}
    ss_ms = kern.get("k_state_scan")
    if ss_ms:
        ss_flops = chunk_state_flops(B, T, H, D, N, C)
        e["kernels_achieved"] = {"k_state_scan": {
            "TFLOP/s": round(ss_flops / (ss_ms * 1e-3) / 1e12, 2),
            "frac_peak": round(ss_flops / (ss_ms * 1e-3) / 1e12 / peak, 4),
            "GB/s": round(state_scan_hbm_bytes(B, T, H, D, N, C,
                                               in_bytes=2 if dtype == "bf16" else 4)
                          / (ss_ms * 1e-3) / 1e9, 1)}}
    cs_ms = kern.get("k_cumsum")
    if cs_ms:
        e.setdefault("kernels_achieved", {})["k_cumsum"] = {
            "GB/s": round(cumsum_hbm_bytes(B, T, H, C) / (cs_ms * 1e-3) / 1e9, 1)}
    if cpu_budget_s:
        e["cpu_baseline"] = cpu_baseline(inp, budget_s=cpu_budget_s)
    return e


def timed_pair(call, steps, stream, dev, reset=None):
    """`steps` calls timed with HIP events on `stream`, the library's per-kernel
    profiler off; then the same number of calls again with it on (`reset`, if
    given, runs untimed before each pass).  Returns (ms per call of the first
    pass, the profile of the second)."""
    import torch
    import complex_valued_state_amd as cssd
    if reset is not None:
        reset()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    if reset is not None:
        reset()
        torch.cuda.synchronize(dev)
    with cssd.profile() as prof:
        for _ in range(steps):
            call()
        torch.cuda.synchronize(dev)
    return ms, prof


def time_constant_input(B, H, D, N, nsteps, reps, warmup, dev, seed=4):
    """cssd_step_n (nsteps at once) and cssd_step_infinite on one seeded token;
    returns per-call ms of each (HIP events on the launch stream)."""
    import torch
    import complex_valued_state_amd as cssd
    import cssd_workloads as wl
    g = torch.Generator(device=dev).manual_seed(seed)
    r = math.sqrt(0.5)
    x = [torch.randn((B, H, D), generator=g, device=dev) * r for _ in range(2)]
    bm = [torch.randn((B, H, N), generator=g, device=dev) * r for _ in range(2)]
    cm = [torch.randn((B, H, N), generator=g, device=dev) * r for _ in range(2)]
    dt = torch.randn((B, H), generator=g, device=dev)
    a_re, a_im, dk = (torch.from_numpy(v).to(dev) for v in wl.decode_params(seed, H))
    h_re = torch.zeros((B, H, N, D), dtype=torch.float32, device=dev)
    h_im = torch.zeros_like(h_re)
    args = (x[0], x[1], bm[0], bm[1], cm[0], cm[1], dt, a_re, a_im, dk)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, call in (("step_n", lambda: cssd.cssd_step_n(*args, h_re, h_im, nsteps, stream=stream)),
                       ("step_infinite", lambda: cssd.cssd_step_infinite(*args, stream=stream))):
        settle(call, dev)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        res[name] = e0.elapsed_time(e1) / reps
    return res


def backward_dx_flops(B, T, H, D, N, C):
    """Algorithmic real flops of k_bwd_dx: per chunk, over the causal triangle, the
    score C B^T (tri x N) and the product giving dX (tri x D), and the state term
    conj(B) R (C x N x D); 8 real flops per complex MAC.  k_bwd_db does the same
    amount with N and D exchanged in the triangle terms."""
    nC = -(-T // C)
    tri = C * (C + 1) // 2
    return 8 * B * H * nC * (tri * (N + D) + C * N * D)


def time_phase_scan(B, T, H, N, steps, warmup, dev, chunk=0, seed=5):
    """cssd_phase_scan over device-drawn inputs with the distributions of
    cssd_workloads.phase_inputs; returns (ms per call, per-kernel ms per call)."""
    import torch
    import complex_valued_state_amd as cssd
    import cssd_workloads as wl
    g = torch.Generator(device=dev).manual_seed(seed)
    shp = (B, T, H, N)
    step = torch.pow(10.0, -3.0 + 2.0 * torch.rand((B, T, H, 1), generator=g, device=dev))
    omega = torch.from_numpy(wl.phase_frequencies(H, N)).to(dev)
    phi = (0.5 * step * (torch.randn(shp, generator=g, device=dev) + omega)).contiguous()
    u = torch.randn(shp, generator=g, device=dev) * 2.0 + 1.5
    b_re = torch.randn(shp, generator=g, device=dev) * math.sqrt(0.5)
    b_im = torch.randn(shp, generator=g, device=dev) * math.sqrt(0.5)
    psi0 = (torch.randn((B, H, N), generator=g, device=dev) * 0.25,
            torch.randn((B, H, N), generator=g, device=dev) * 0.25)
    outs = (torch.empty(shp, device=dev), torch.empty(shp, device=dev),
            torch.empty((B, H, N), device=dev), torch.empty((B, H, N), device=dev))
    ws = torch.empty(max(1, cssd.cssd_phase_scan_workspace_size(B, T, H, N, chunk)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    call = lambda: cssd.cssd_phase_scan(phi, u, b_re, b_im, psi0, chunk=chunk, out=outs,
                                        workspace=ws, stream=stream)
    settle(call, dev)
    for _ in range(warmup):
        call()
    ms, prof = timed_pair(call, steps, stream, dev)
    kern = {k: v / steps for k, v in prof.ms.items() if prof.launches[k]}
    return ms, kern


def time_born(B, T, H, D, steps, warmup, dev, seed=6, bf16=False):
    """cssd_born_attention over device-drawn inputs with the distributions of
    cssd_workloads.born_inputs (q, k, v in bf16 when `bf16`); returns (ms per
    call, kernel ms per call)."""
    import torch
    import complex_valued_state_amd as cssd
    g = torch.Generator(device=dev).manual_seed(seed)
    shp = (B, T, H, D)
    r = math.sqrt(0.5)
    planes = [torch.randn(shp, generator=g, device=dev) * r for _ in range(6)]
    if bf16:
        planes = [t.to(torch.bfloat16) for t in planes]
    tau = 0.5 + 1.5 * torch.rand((B, T, H), generator=g, device=dev)
    out = (torch.empty(shp, device=dev), torch.empty(shp, device=dev))
    stream = torch.cuda.current_stream(dev)
    call = lambda: cssd.cssd_born_attention(*planes, tau, out=out, stream=stream)
    settle(call, dev)
    for _ in range(warmup):
        call()
    ms, prof = timed_pair(call, steps, stream, dev)
    return ms, prof.ms["k_born"] / max(1, prof.launches["k_born"])


def time_backward(inp, steps, warmup, dev, seed=9, saved=False):
    """cssd_backward with the forward output and seeded upstream gradients resident
    (saved: cssd_backward_saved on the states the forward left in the workspace)."""
    import torch
    import complex_valued_state_amd as cssd
    a = _to_dev(inp, dev)
    d = dict(zip(("x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt", "A_re", "A_im", "Dskip"), a))
    d["h0"] = None
    Bsz, T, H, D = inp.x_re.shape
    N = inp.B_re.shape[-1]
    g = torch.Generator(device=dev).manual_seed(seed)
    r = math.sqrt(0.5)
    dy = [torch.randn((Bsz, T, H, D), generator=g, device=dev) * r for _ in range(2)]
    dhT = [torch.randn((Bsz, H, N, D), generator=g, device=dev) * r for _ in range(2)]
    code = cssd.CSSD_BF16 if inp.in_dtype == "bf16" else cssd.CSSD_F32
    ws = torch.empty(cssd.cssd_backward_workspace_size(Bsz, T, H, D, N, inp.chunk, code),
                     dtype=torch.uint8, device=dev)
    ins = (d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"], d["dt"], d["A_re"],
           d["A_im"], d["Dskip"], d["h0"])
    if code == cssd.CSSD_BF16:
        y, hT = None, None  # recomputed in fp32 inside the call
    else:
        out = cssd.cssd_forward(*ins, chunk=inp.chunk, workspace=ws)
        y, hT = out[:2], out[2:]
    stream = torch.cuda.current_stream(dev)

    def run():
        if saved:
            cssd.cssd_backward_saved(*ins, y, hT, dy, dhT, chunk=inp.chunk, workspace=ws,
                                     stream=stream)
        else:
            cssd.cssd_backward(*ins, y, dy, dhT, chunk=inp.chunk, workspace=ws, stream=stream)

    settle(run, dev)
    for _ in range(warmup):
        run()
    ms, prof = timed_pair(run, steps, stream, dev)
    kern = {k: v / max(prof.launches[k], 1) for k, v in prof.ms.items() if prof.launches[k]}
    return ms, kern


def time_decode(B, H, D, N, tokens, warmup, dev, seed=4):
    """cssd_step over `tokens` pre-staged tokens (seeded device-side draws)."""
    import torch
    import complex_valued_state_amd as cssd
    import cssd_workloads as wl
    g = torch.Generator(device=dev).manual_seed(seed)
    r = math.sqrt(0.5)
    xs = [torch.randn((tokens, B, H, D), generator=g, device=dev) * r for _ in range(2)]
    bs = [torch.randn((tokens, B, H, N), generator=g, device=dev) * r for _ in range(2)]
    cs = [torch.randn((tokens, B, H, N), generator=g, device=dev) * r for _ in range(2)]
    dts = torch.randn((tokens, B, H), generator=g, device=dev)
    a_re, a_im, dk = (torch.from_numpy(v).to(dev) for v in wl.decode_params(seed, H))
    h_re = torch.zeros((B, H, N, D), dtype=torch.float32, device=dev)
    h_im = torch.zeros_like(h_re)
    y_re = torch.empty((tokens, B, H, D), dtype=torch.float32, device=dev)
    y_im = torch.empty_like(y_re)
    stream = torch.cuda.current_stream(dev)

    def step(t):
        cssd.cssd_step(xs[0][t], xs[1][t], bs[0][t], bs[1][t], cs[0][t], cs[1][t], dts[t], a_re,
                       a_im, dk, h_re, h_im, out=(y_re[t], y_im[t]), stream=stream)

    settle(lambda: step(0), dev)
    for t in range(warmup):
        step(t % tokens)
    torch.cuda.synchronize(dev)
    pos = [0]

    def reset():  # each pass over the tokens starts from a zero state
        h_re.zero_()
        h_im.zero_()
        pos[0] = 0

    def next_token():
        step(pos[0])
        pos[0] += 1

    ms, prof = timed_pair(next_token, tokens, stream, dev, reset=reset)
    kms = prof.ms["k_step"] / max(1, prof.launches["k_step"])
    return ms, kms


def host_threads():
    """Host threads the oracle may use: every core this process may run on,
    capped by OMP_NUM_THREADS where the job sets it (the share of the machine's
    cores the job is given)."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return min(n, cap) if cap > 0 else n


def cpu_baseline(inp, budget_s=15.0):
    """The fp64 oracle, untuned, on a bounded sample of the same workload: the
    first b_s batch rows (all heads, full length), b_s calibrated so the run
    takes roughly `budget_s` seconds; the whole workload, repeated up to ten
    times (median taken), when it fits the budget.  Returns tokens/s scaled to
    the sample."""
    import numpy as np
    import oracle
    threads = host_threads()
    lib = oracle.load()

    cache = {}

    def run(bs):
        if bs not in cache:  # the complex fp64 copies are made once per sample size
            cache.clear()
            cache[bs] = _rows(inp, bs).complex()
        x, Bm, Cm, dt, A, Dk, h0 = cache[bs]
        t0 = time.perf_counter()
        oracle.forward(x, Bm, Cm, dt, A, Dk, h0, nthreads=threads, lib=lib)
        return time.perf_counter() - t0

    s = inp.shape
    t1 = run(1)
    bs = int(max(1, min(s["B"], round(budget_s / max(t1, 1e-3)))))
    times = [t1] if bs == 1 else [run(bs)]
    # the whole workload may finish well inside the budget on many cores:
    # repeat it (at most 10 runs) and take the median run
    while bs == s["B"] and sum(times) < budget_s * 0.6 and len(times) < 10:
        times.append(run(bs))
    t = float(np.median(times))
    cache.clear()
    # one thread on one (b, h) sequence, scaled to the H sequences a token spans
    one = _one_sequence(inp).complex()
    t_one = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.forward(*one, nthreads=1, lib=lib)
        t_one.append(time.perf_counter() - t0)
    t1s = float(np.median(t_one))
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(bs * s["T"] / t, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model,
            "sample": f"{bs} of {s['B']} batch rows (all {s['H']} heads, full T={s['T']}) of the "
                      f"same workload, median of {len(times)} run(s); fp64 sequential recurrence, "
                      f"OpenMP over (batch, head) on {threads} threads; {t:.3f} s wall per run",
            "single_thread": {"value": round(s["T"] / (s["H"] * t1s), 1), "unit": "tokens/s",
                              "cores": 1,
                              "sample": f"one (b, h) sequence of T={s['T']} on one thread, median "
                                        f"of 3 runs ({t1s:.4f} s), scaled by the {s['H']} heads "
                                        f"a token spans"}}


def _one_sequence(inp):
    """Batch row 0, head 0 of the workload (H = 1)."""
    import cssd_workloads as wl
    import numpy as np
    c = lambda a: None if a is None else np.ascontiguousarray(a[:1, :, :1])
    h = lambda a: None if a is None else np.ascontiguousarray(a[:1])
    return wl.ForwardInputs(c(inp.x_re), c(inp.x_im), c(inp.B_re), c(inp.B_im), c(inp.C_re),
                            c(inp.C_im), c(inp.dt), h(inp.A_re), h(inp.A_im), h(inp.Dskip),
                            inp.chunk, c(inp.h0_re), c(inp.h0_im), inp.in_dtype, inp.name)


def _rows(inp, bs):
    import cssd_workloads as wl
    import numpy as np
    c = lambda a: None if a is None else np.ascontiguousarray(a[:bs])
    return wl.ForwardInputs(c(inp.x_re), c(inp.x_im), c(inp.B_re), c(inp.B_im), c(inp.C_re),
                            c(inp.C_im), c(inp.dt), inp.A_re, inp.A_im, inp.Dskip, inp.chunk,
                            c(inp.h0_re), c(inp.h0_im), inp.in_dtype, inp.name)


def born_entry(steps, dev, bf16):
    """Causal Born attention at B256 T1024 H16 D16 (fp32 or bf16 inputs): tokens/s and
    the matrix-core roofline of the attention kernel."""
    bb, bt, bhd, bd = 256, 1024, 16, 16
    ms, kms = time_born(bb, bt, bhd, bd, max(3, steps // 2), 2, dev, bf16=bf16)
    fl = born_flops(bb, bt, bhd, bd)
    kern = "k_born_bf16" if bf16 else "k_born"
    peak = PEAK_BF16_MFMA_TFLOPS if bf16 else PEAK_FP32_MFMA_TFLOPS
    # the bf16 kernel's 32-bit-view instance serves rows that span under 2 GB per (b, h)
    small = ((bt + 2 * 64) * bhd * bd + bd) * 4 < (1 << 31)
    sym = f"{kern}<{bd}, {'true' if small else 'false'}>" if bf16 else f"{kern}<{bd}>"
    return {
        "tokens_per_s": round(bb * bt / (ms * 1e-3), 1), "ms_per_call": round(ms, 5),
        "roofline": {"bound": "mfma", "kernel": kern, "symbol": sym,
                     "traffic": load_traffic(sym),
                     "achieved": round(fl / (kms * 1e-3) / 1e12, 2),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(fl / (kms * 1e-3) / 1e12 / peak, 4),
                     "algorithmic_flops_per_launch": fl, "avg_launch_ms": round(kms, 5)}}


# the workloads --only can time alone: name -> (generator function, argument) for the
# forward and backward ones; the Born attention ones take no inputs from here
ONLY = {"forward_f32": ("config1", "f32"), "forward_bf16": ("config1", "bf16"),
        "forward_tiny": ("config0", None), "forward_long": ("config2", None),
        "forward_pam": ("config3", "re"), "born_f32": None, "born_bf16": None,
        "backward_f32": ("config1", "f32"), "backward_bf16": ("config1", "bf16")}


def only_inputs(name):
    import cssd_workloads as wl
    fn, arg = ONLY[name]
    return getattr(wl, fn)() if arg is None else getattr(wl, fn)(arg)


def copy_calibration(dev, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size, for scaling HBM byte counters:
    each copy reads exactly `nbytes` and writes exactly `nbytes` (the buffers are
    four times larger than the on-package caches), so what FETCH_SIZE and
    WRITE_SIZE report for it gives the factor between the counters' units and
    bytes on this machine."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize(dev)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copied_bytes": nbytes, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the headline workload")
    ap.add_argument("--only", choices=sorted(ONLY), default=None,
                    help="time one workload alone (a forward, the backward or the Born "
                         "attention) and print its figures (for profiler runs); not the "
                         "benchmark line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="copy a 1 GiB buffer three times (the reference kernel that scales "
                         "the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding across GPUs is not implemented", file=sys.stderr)
        sys.exit(2)

    import torch
    import complex_valued_state_amd as cssd
    import cssd_workloads as wl
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
        return
    cssd.load_library()
    if args.only:
        progress(f"timing {args.only} alone")
        if args.only.startswith("born_"):
            e = born_entry(args.steps, dev, bf16=args.only == "born_bf16")
        elif args.only.startswith("backward_"):
            bms, bk = time_backward(only_inputs(args.only), max(3, args.steps // 2), 2, dev)
            e = {"ms_per_step": round(bms, 4), "kernels_avg_ms": {k: round(v, 5) for k, v in bk.items()}}
        else:
            e = forward_entry(only_inputs(args.only), args.steps, args.warmup, dev)
        print(json.dumps({"workload": args.only, **e}), flush=True)
        return

    s = wl.CONFIG_SHAPES[1]
    B, T, H, D, N, C = s["B"], s["T"], s["H"], s["D"], s["N"], s["C"]
    progress("generating the B8 T2048 H48 D64 N64 C64 inputs")
    inp = wl.config1("f32")
    progress("timing the fp32 forward")
    head = forward_entry(inp, args.steps, args.warmup, dev)
    ms = head["ms_per_step"]
    progress(f"fp32 forward {ms:.4f} ms/step")
    tokens = B * T
    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "complex chunkwise scan forward, Mamba-style layer: batch 8, T 2048, "
                               "48 heads, head dim 64, state 64, chunk 64, fp32 complex planes",
                   "batch": B, "seqlen": T, "heads": H, "headdim": D, "dstate": N, "chunk": C,
                   "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "ms_per_step_profiled": head["ms_per_step_profiled"],
        "kernels_avg_ms": head["kernels_avg_ms"],
        "kernels_achieved": head["kernels_achieved"],
        "forward_mfma_frac": head["forward_mfma_frac"],
        "forward_hbm_frac": head["forward_hbm_frac"],
    }
    extra = {}
    if not args.no_extras:
        progress("timing the bf16-input forward")
        inp16 = wl.config1("bf16")
        e16 = forward_entry(inp16, args.steps, args.warmup, dev)
        # HBM binds this variant: its fraction of the HBM roofline is the headline one
        e16["hbm_roofline_frac"] = e16.pop("forward_hbm_frac")
        e16["bf16_mfma_frac"] = e16.pop("forward_mfma_frac")
        extra["forward_B8_T2048_H48_D64_N64_C64_bf16_inputs"] = e16
        del inp16
        # the other forward workloads, each with the oracle timed beside it
        for name, mk, budget in (
                ("forward_tiny_B1_T64_H2_D16_N16_C16", wl.config0, 2.0),
                ("forward_long_B1_T16384_H48_D64_N128_C128", wl.config2, 6.0),
                ("forward_pam_B16_T1024_H12_D64_N128_C64", lambda: wl.config3("re"), 4.0)):
            progress(f"timing {name}")
            i2 = mk()
            extra[name] = forward_entry(i2, args.steps, args.warmup, dev,
                                        cpu_budget_s=None if args.no_cpu_baseline else budget)
            del i2
        d4 = wl.CONFIG_SHAPES[4]
        progress("timing the backward pass")
        bms, bk = time_backward(inp, max(3, args.steps // 2), 2, dev)
        bfl = backward_dx_flops(B, T, H, D, N, C)
        bsym = "k_bwd_lds<true>" if C == N == D == 64 else f"k_bwd_tiles<{C}, {N}, {D}, 0>"
        extra["backward_B8_T2048_H48_D64_N64_C64_f32"] = {
            "tokens_per_s": round(tokens / (bms * 1e-3), 1), "ms_per_step": round(bms, 4),
            "kernels_avg_ms": {k: round(v, 5) for k, v in bk.items()},
            "roofline": {"bound": "mfma", "kernel": "k_bwd_dx", "symbol": bsym,
                         "traffic": load_traffic(bsym),
                         "achieved": round(bfl / (bk["k_bwd_dx"] * 1e-3) / 1e12, 2),
                         "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(bfl / (bk["k_bwd_dx"] * 1e-3) / 1e12
                                       / PEAK_FP32_MFMA_TFLOPS, 4),
                         "algorithmic_flops_per_launch": bfl,
                         "avg_launch_ms": round(bk["k_bwd_dx"], 5)}}
        progress("timing the backward pass with bf16 inputs")
        inp16 = wl.config1("bf16")
        b16ms, b16k = time_backward(inp16, max(3, args.steps // 2), 2, dev)
        del inp16
        extra["backward_B8_T2048_H48_D64_N64_C64_bf16_inputs"] = {
            "tokens_per_s": round(tokens / (b16ms * 1e-3), 1), "ms_per_step": round(b16ms, 4),
            "kernels_avg_ms": {k: round(v, 5) for k, v in b16k.items()}}
        progress("timing the backward pass on the forward's saved states")
        sms, sk = time_backward(inp, max(3, args.steps // 2), 2, dev, saved=True)
        extra["backward_saved_states_B8_T2048_H48_D64_N64_C64_f32"] = {
            "tokens_per_s": round(tokens / (sms * 1e-3), 1), "ms_per_step": round(sms, 4),
            "kernels_avg_ms": {k: round(v, 5) for k, v in sk.items()}}
        progress("timing the decode step")
        dms, dkms = time_decode(d4["B"], d4["H"], d4["D"], d4["N"], d4["steps"], 8, dev)
        dbytes = decode_hbm_bytes(d4["B"], d4["H"], d4["D"], d4["N"])
        extra["decode_B256_H48_N128_D64"] = {
            "tokens_per_s": round(d4["B"] / (dms * 1e-3), 1), "ms_per_token_step": round(dms, 5),
            "roofline": {"bound": "hbm", "kernel": "k_step",
                         "symbol": f"k_step<{d4['N']}, {d4['D']}>",
                         "traffic": load_traffic(f"k_step<{d4['N']}, {d4['D']}>"),
                         "achieved": round(dbytes / (dkms * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(dbytes / (dkms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes_per_launch": dbytes, "avg_launch_ms": round(dkms, 5)}}
        progress("timing the constant-input entry points")
        nconst = 4096
        cms = time_constant_input(d4["B"], d4["H"], d4["D"], d4["N"], nconst, 20, 3, dev)
        extra["constant_input_B256_H48_N128_D64"] = {
            "step_n": {"nsteps": nconst, "ms_per_call": round(cms["step_n"], 5),
                       "tokens_per_s": round(d4["B"] * nconst / (cms["step_n"] * 1e-3), 1),
                       "hbm_GBs": round(dbytes / (cms["step_n"] * 1e-3) / 1e9, 1),
                       "hbm_frac": round(dbytes / (cms["step_n"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "step_infinite": {"ms_per_call": round(cms["step_infinite"], 5)}}
        progress("timing the phase-state scan")
        pb, pt, ph, pn = 256, 1024, 16, 16
        pms, pk = time_phase_scan(pb, pt, ph, pn, args.steps, args.warmup, dev)
        pbytes = phase_scan_hbm_bytes(pb, pt, ph, pn)
        pout = pk.get("k_phase_out", pms)
        extra["phase_scan_B256_T1024_H16_N16"] = {
            "tokens_per_s": round(pb * pt / (pms * 1e-3), 1), "ms_per_call": round(pms, 5),
            "kernels_avg_ms": {k: round(v, 5) for k, v in pk.items()},
            "roofline": {"bound": "hbm", "kernel": "k_phase_out", "symbol": "k_phase_out",
                         "traffic": load_traffic("k_phase_out"),
                         "achieved": round(pbytes / (pout * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(pbytes / (pout * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes_per_launch": pbytes, "avg_launch_ms": round(pout, 5)}}
        progress("timing causal Born attention")
        extra["born_attention_B256_T1024_H16_D16_f32"] = born_entry(args.steps, dev, bf16=False)
        progress("timing causal Born attention with bf16 inputs")
        extra["born_attention_B256_T1024_H16_D16_bf16_inputs"] = born_entry(args.steps, dev, bf16=True)
    out["extra"] = extra
    if not args.no_cpu_baseline:
        progress("timing the fp64 oracle on the host cores")
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
