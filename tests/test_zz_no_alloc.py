"""cssd_forward_noalloc, the forward whose workspace is the library's fixed
device array (callers that cannot allocate), against cssd_forward on the same
inputs: two calls in a row, the second smaller than the first (the array keeps
the first call's contents), each bit for bit equal to cssd_forward with a fresh
workspace and within 2e-4 of the fp64 oracle; a problem too large for the array
is refused before anything runs."""
import numpy as np
import pytest

import cssd_workloads as wl
from gpu_util import dev_inputs, log, oracle_forward, rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-4

# (seed, B, T, H, D, N, C, dtype): a larger problem first, then a smaller one with
# another shape and chunk size; both have ragged last chunks
CALLS = [(501, 2, 1000, 6, 64, 64, 64, "f32"), (502, 1, 300, 3, 32, 128, 32, "f32")]


def _ins(d):
    return (d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"], d["dt"], d["A_re"],
            d["A_im"], d["Dskip"], d["h0"])


def test_noalloc_matches_forward_on_two_calls():
    import torch
    import complex_valued_state_amd as cssd
    to = lambda r, i: r.double().cpu().numpy() + 1j * i.double().cpu().numpy()
    for (seed, B, T, H, D, N, C, dt) in CALLS:
        size = cssd.cssd_forward_workspace_size(B, T, H, D, N, C)
        assert 0 < size <= cssd.CSSD_NOALLOC_SCRATCH_BYTES
        inp = wl.random_forward(seed, B, T, H, D, N, C, with_h0=True, in_dtype=dt)
        d = dev_inputs(inp)
        log(f"  noalloc B{B} T{T} H{H} D{D} N{N} C{C} {dt} (workspace {size} B)")
        out = [torch.full((B, T, H, D), float("nan"), device="cuda:0") for _ in range(2)] + \
              [torch.full((B, H, N, D), float("nan"), device="cuda:0") for _ in range(2)]
        cssd.cssd_forward_noalloc(*_ins(d), chunk=C, out=tuple(out))
        ref = cssd.cssd_forward(*_ins(d), chunk=C)
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(out, ref)):
            assert torch.equal(a, b), (seed, k)
        yr, hr = oracle_forward(inp)
        ey, eh = rel_err(to(out[0], out[1]), yr), rel_err(to(out[2], out[3]), hr)
        log(f"    rel err y={ey:.3e} hT={eh:.3e}")
        assert ey <= TOL and eh <= TOL


def test_noalloc_bf16_two_stream_split():
    """bf16 inputs with more sequences than CUs (at most twice as many): the
    forward runs part of its work on the library's second stream, set up once on
    the first such call (possibly this one), and the no-alloc entry point gives
    cssd_forward's result bit for bit, on two calls in a row."""
    import torch
    import complex_valued_state_amd as cssd
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for rep, (T, H) in enumerate(((100, cus + 9), (70, 2 * cus))):
        B, D, N, C = 1, 64, 64, 64
        assert cssd.cssd_forward_workspace_size(B, T, H, D, N, C) <= cssd.CSSD_NOALLOC_SCRATCH_BYTES
        inp = wl.random_forward(511 + rep, B, T, H, D, N, C, with_h0=True, in_dtype="bf16")
        d = dev_inputs(inp)
        log(f"  noalloc bf16 B{B} T{T} H{H} ({B * H} sequences, {cus} CUs)")
        out = [torch.full((B, T, H, D), float("nan"), device="cuda:0") for _ in range(2)] + \
              [torch.full((B, H, N, D), float("nan"), device="cuda:0") for _ in range(2)]
        cssd.cssd_forward_noalloc(*_ins(d), chunk=C, out=tuple(out))
        ref = cssd.cssd_forward(*_ins(d), chunk=C)
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(out, ref)):
            assert torch.equal(a, b), (rep, k)


def test_noalloc_refuses_a_problem_too_large_for_its_array():
    import torch
    import complex_valued_state_amd as cssd
    B, T, H, D, N, C = 4, 2048, 48, 64, 64, 64
    assert cssd.cssd_forward_workspace_size(B, T, H, D, N, C) > cssd.CSSD_NOALLOC_SCRATCH_BYTES
    z = lambda *s: torch.zeros(s, device="cuda:0")
    with pytest.raises(cssd.CSSDError) as e:
        cssd.cssd_forward_noalloc(z(B, T, H, D), z(B, T, H, D), z(B, T, H, N), z(B, T, H, N),
                                  z(B, T, H, N), z(B, T, H, N), z(B, T, H), z(H), z(H),
                                  chunk=C)
    assert e.value.status == 5
