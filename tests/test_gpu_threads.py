"""Concurrent use of the library: several host threads, each on a stream of its own,
calling cssd_forward at the same time with the per-kernel profiler switched on.

The library keeps no per-call state (the profiler's accumulators are the one
process-wide object, behind a lock), so every thread's outputs must equal, bit for
bit, those of the same call made alone, and the profiler must count every launch
once.  The calls made alone are also checked against the fp64 oracle (max|err| /
max|ref| <= 2e-4 on the complex modulus, y and the final state separately)."""
import threading

import numpy as np
import pytest

import cssd_workloads as wl
from gpu_util import dev_inputs, gpu_forward, log, oracle_forward, rel_err

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-4
REPS = 6

# (seed, B, T, H, D, N, C): the LDS-staged kernels (N = D = C = 64), the register-
# operand chunk scan (C*N > 4096) and a small chunk, each with a ragged tail
CASES = [
    (301, 2, 200, 3, 64, 64, 64),
    (302, 1, 300, 2, 64, 128, 64),
    (303, 2, 130, 2, 32, 32, 16),
    (304, 3, 257, 2, 64, 64, 64),
]


def test_threads_on_separate_streams_match_serial_calls():
    import torch
    import complex_valued_state_amd as cssd

    inps = [wl.random_forward(s, B, T, H, D, N, C, with_h0=True, name=f"thr{s}")
            for (s, B, T, H, D, N, C) in CASES]
    serial = []
    for inp in inps:
        y, hT = gpu_forward(inp)
        yr, hr = oracle_forward(inp)
        ey, eh = rel_err(y, yr), rel_err(hT, hr)
        log(f"  serial {inp.name} {inp.shape}: rel err y={ey:.3e} hT={eh:.3e}")
        assert ey <= TOL_F32 and eh <= TOL_F32, (inp.name, ey, eh)
        serial.append((y, hT))

    dev = [dev_inputs(inp) for inp in inps]
    streams = [torch.cuda.Stream() for _ in inps]  # default priority
    results = [None] * len(inps)
    errors = []
    barrier = threading.Barrier(len(inps))

    def work(i):
        try:
            d, s = dev[i], streams[i]
            s.wait_stream(torch.cuda.default_stream())
            with torch.cuda.stream(s):
                outs = []
                barrier.wait()
                for _ in range(REPS):
                    outs.append(cssd.cssd_forward(
                        d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"],
                        d["dt"], d["A_re"], d["A_im"], d["Dskip"], d["h0"],
                        chunk=inps[i].chunk, stream=s))
            s.synchronize()
            to = lambda r, im: r.double().cpu().numpy() + 1j * im.double().cpu().numpy()
            results[i] = [(to(o[0], o[1]), to(o[2], o[3])) for o in outs]
        except Exception as e:  # reported on the main thread
            errors.append((i, repr(e)))
            barrier.abort()

    log(f"  {len(inps)} threads x {REPS} forward calls, profiler on")
    with cssd.profile() as prof:
        threads = [threading.Thread(target=work, args=(i,)) for i in range(len(inps))]
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=120)
        assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
        torch.cuda.synchronize()
    assert not errors, errors

    for i, inp in enumerate(inps):
        for rep, (y, hT) in enumerate(results[i]):
            assert np.array_equal(y, serial[i][0]), (inp.name, rep, "y")
            assert np.array_equal(hT, serial[i][1]), (inp.name, rep, "hT")
    calls = len(inps) * REPS
    log(f"  profiler launches: cumsum {prof.launches['k_cumsum']}, "
        f"chunk_scan {prof.launches['k_chunk_scan']}, state_scan {prof.launches['k_state_scan']}")
    assert prof.launches["k_cumsum"] == calls
    assert prof.launches["k_chunk_scan"] == calls
    assert prof.launches["k_state_scan"] == calls
    assert all(prof.ms[k] > 0.0 for k in ("k_cumsum", "k_chunk_scan", "k_state_scan"))


def test_side_stream_call_without_workspace():
    """A call given a stream other than torch's current one, with no workspace or
    outputs passed: the binding allocates them from that stream's pool, so the
    blocks it frees on return are not handed to new work on the current stream
    while the kernels still run.  The current stream then allocates and fills
    tensors of the same sizes at once; the results must equal those of the same
    call made alone on the current stream, bit for bit, and the oracle within
    2e-4."""
    import torch
    import complex_valued_state_amd as cssd
    inp = wl.random_forward(305, 4, 1024, 8, 64, 64, 64, with_h0=True, name="side_stream")
    d = dev_inputs(inp)
    ins = (d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"], d["dt"], d["A_re"],
           d["A_im"], d["Dskip"], d["h0"])
    ref = cssd.cssd_forward(*ins, chunk=inp.chunk)
    torch.cuda.synchronize()
    ref = [t.clone() for t in ref]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ws_bytes = cssd.cssd_forward_workspace_size(4, 1024, 8, 64, 64, 64)
    log("  forward on a side stream, binding-owned workspace and outputs")
    for rep in range(4):
        got = cssd.cssd_forward(*ins, chunk=inp.chunk, stream=side)
        # new work on the current stream, sized like the blocks the call just freed
        junk = [torch.full((ws_bytes // 4,), float("nan"), device="cuda:0") for _ in range(2)]
        junk += [torch.full(tuple(t.shape), float("nan"), device="cuda:0") for t in ref]
        side.synchronize()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (rep, k)
        del junk, got
    to = lambda r, im: r.double().cpu().numpy() + 1j * im.double().cpu().numpy()
    yr, hr = oracle_forward(inp)
    assert rel_err(to(ref[0], ref[1]), yr) <= TOL_F32
    assert rel_err(to(ref[2], ref[3]), hr) <= TOL_F32
