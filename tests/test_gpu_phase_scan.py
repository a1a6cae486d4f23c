"""GPU parity of cssd_phase_scan, the per-coordinate Cayley-phase x gate scan,
against the oracle's sequential fp64 recurrence (needs an MI355X)."""
import numpy as np
import pytest

import cssd_workloads as wl
import oracle
from gpu_util import log, rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-4


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def _c(r, i):
    return r.double().cpu().numpy() + 1j * i.double().cpu().numpy()


def _run(p, chunk=0, with_psi0=True, return_state=True):
    import torch
    import complex_valued_state_amd as cssd
    psi0 = (_dev(p.psi0_re), _dev(p.psi0_im)) if with_psi0 else None
    out = cssd.cssd_phase_scan(_dev(p.phi), _dev(p.u), _dev(p.b_re), _dev(p.b_im), psi0,
                               chunk=chunk, return_state=return_state)
    torch.cuda.synchronize()
    psi = _c(out[0], out[1])
    psiT = _c(out[2], out[3]) if return_state else None
    return psi, psiT


def _want(p, with_psi0=True):
    return oracle.phase_scan(p.phi, p.u, p.b(), p.psi0() if with_psi0 else None)


@pytest.mark.parametrize("B,T,H,N,chunk", [
    (1, 1, 1, 1, 0),          # one step, one coordinate
    (2, 1, 3, 5, 16),         # one step with an explicit segment length
    (3, 77, 2, 5, 0),         # odd coordinate count, ragged everything
    (2, 333, 4, 16, 16),      # 21 segments, ragged last one
    (2, 333, 4, 16, 0),       # the library's choice (short segments for few rows)
    (1, 1000, 3, 7, 64),
    (2, 64, 2, 16, 1),        # every step its own segment
    (2, 130, 2, 16, 7),       # segment not a multiple of the prefetch block
    (4, 600, 16, 16, 5000),   # chunk >= seqlen: one pass
])
def test_phase_scan_vs_oracle(B, T, H, N, chunk):
    log(f"  phase_scan B{B} T{T} H{H} N{N} chunk{chunk}")
    p = wl.phase_inputs(80 + T, B, T, H, N)
    psi, psiT = _run(p, chunk)
    want, wantT = _want(p)
    assert rel_err(psi, want) <= TOL, rel_err(psi, want)
    assert rel_err(psiT, wantT) <= TOL, rel_err(psiT, wantT)


@pytest.mark.parametrize("chunk", [0, 16, 48])
def test_phase_scan_without_initial_state(chunk):
    p = wl.phase_inputs(81, 2, 200, 3, 16)
    psi, psiT = _run(p, chunk, with_psi0=False)
    want, wantT = _want(p, with_psi0=False)
    assert rel_err(psi, want) <= TOL
    assert rel_err(psiT, wantT) <= TOL
    psi2, none = _run(p, chunk, with_psi0=False, return_state=False)
    assert none is None and np.array_equal(psi2, psi)


def test_phase_scan_segmentations_agree():
    """One pass and several segment lengths give the same trajectory (each checked
    against the oracle, and against each other at rounding level)."""
    p = wl.phase_inputs(82, 2, 1024, 4, 16)
    want, wantT = _want(p)
    runs = [_run(p, c) for c in (1024, 256, 64, 16)]
    for psi, psiT in runs:
        assert rel_err(psi, want) <= TOL
        assert rel_err(psiT, wantT) <= TOL
    for psi, _ in runs[1:]:
        assert rel_err(psi, runs[0][0]) <= TOL


def test_phase_scan_state_in_place():
    """psiT may be the psi0 arrays: two half-sequence calls chained in place equal
    one call over the whole sequence."""
    import torch
    import complex_valued_state_amd as cssd
    B, T, H, N = 2, 300, 2, 16
    p = wl.phase_inputs(83, B, T, H, N)
    want, wantT = _want(p)
    s_re, s_im = _dev(p.psi0_re), _dev(p.psi0_im)
    halves = []
    for lo, hi, chunk in ((0, 140, 32), (140, T, 0)):
        sl = lambda a: _dev(a[:, lo:hi])
        out = cssd.cssd_phase_scan(sl(p.phi), sl(p.u), sl(p.b_re), sl(p.b_im), (s_re, s_im),
                                   chunk=chunk, out=(torch.empty((B, hi - lo, H, N), device="cuda:0"),
                                                     torch.empty((B, hi - lo, H, N), device="cuda:0"),
                                                     s_re, s_im))
        halves.append(_c(out[0], out[1]))
    torch.cuda.synchronize()
    assert rel_err(np.concatenate(halves, axis=1), want) <= TOL
    assert rel_err(_c(s_re, s_im), wantT) <= TOL


def test_phase_scan_transport_over_4096_steps():
    """No input, gate fully open: the modulus is carried exactly and the phase
    advances by sum 2 atan(phi) (the phase-state paper, Lemma 6.2), 4096 steps."""
    B, T, H, N = 2, 4096, 2, 16
    p = wl.phase_inputs(84, B, T, H, N)
    p.u[:] = 60.0
    p.b_re[:] = 0.0
    p.b_im[:] = 0.0
    for chunk in (0, 4096, 128):
        psi, psiT = _run(p, chunk)
        want, wantT = _want(p)
        assert rel_err(psi, want) <= TOL, (chunk, rel_err(psi, want))
        assert rel_err(psiT, wantT) <= TOL
        mod = np.abs(psiT) / np.abs(p.psi0())
        assert np.max(np.abs(mod - 1.0)) <= TOL, np.max(np.abs(mod - 1.0))


def test_phase_scan_extreme_parameters():
    """phi across the whole float range (the Cayley transform stays on the unit
    circle: -1 as phi -> inf), gates that vanish or saturate."""
    B, T, H, N = 1, 40, 1, 16
    p = wl.phase_inputs(85, B, T, H, N)
    specials = np.array([0.0, 1.0, -1.0, 1.0000001, 0.9999999, 1e-30, -1e-30, 1e10, -1e10,
                         3e19, -3e19, 1e30, -1e35, 3.0e38, 0.5, -2.0], dtype=np.float32)
    p.phi[:] = specials[None, None, None, :]
    p.u[:, ::3] = -200.0
    p.u[:, 1::3] = 200.0
    psi, psiT = _run(p, 0)
    assert np.all(np.isfinite(psi))
    want, wantT = _want(p)
    assert rel_err(psi, want) <= TOL
    assert rel_err(psiT, wantT) <= TOL


def test_phase_scan_layer_shape():
    """The H-Mamba layer shape of the phase-state paper per GPU: 256 sequences of
    1024 steps, 16 heads of 16 coordinates (one pass); every element against the
    oracle."""
    B, T, H, N = 256, 1024, 16, 16
    log(f"  phase_scan layer shape B{B} T{T} H{H} N{N}")
    p = wl.phase_inputs(1, B, T, H, N)
    psi, psiT = _run(p, 0)
    want, wantT = _want(p)
    assert rel_err(psi, want) <= TOL, rel_err(psi, want)
    assert rel_err(psiT, wantT) <= TOL
    for h in range(H):  # every head on its own scale
        assert rel_err(psi[:, :, h], want[:, :, h]) <= TOL, h
