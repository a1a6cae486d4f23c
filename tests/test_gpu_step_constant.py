"""GPU parity of the constant-input entry points (cssd_step_n, cssd_step_infinite)
against the oracle's closed forms, which are pinned to the one-step recurrence
(needs an MI355X)."""
import numpy as np
import pytest

import cssd_workloads as wl
import oracle
from gpu_util import log, rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-4


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _c(r, i):
    return r.double().cpu().numpy() + 1j * i.double().cpu().numpy()


def _heads(H):
    """Per-head A covering a decaying rotation, a pure rotation (|a| = 1), no decay
    and no rotation (a = 1) and a vanishing decay, then config-0 draws."""
    a_re, a_im, dk = wl.decode_params(60, H)
    special = [(-0.4, 1.3), (0.0, 0.7), (0.0, 0.0), (-1e4, 0.3)]
    for k, (r, i) in enumerate(special[:H]):
        a_re[k], a_im[k] = r, i
    return a_re.astype(np.float32), a_im.astype(np.float32), dk


def _inputs(seed, B, H, D, N):
    tok = wl.decode_step(seed, 0, B, H, D, N)
    A_re, A_im, Dk = _heads(H)
    rng = np.random.default_rng(seed)
    h0 = (np.sqrt(0.5) * (rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D)))
          ).astype(np.complex64)
    return tok, A_re, A_im, Dk, h0


def _args(tok, A_re, A_im, Dk):
    return ([_dev(getattr(tok, f)) for f in ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt")]
            + [_dev(A_re), _dev(A_im), None if Dk is None else _dev(Dk)])


def _oracle_args(tok, A_re, A_im, Dk):
    x, Bm, Cm, dt = tok.complex()
    A = A_re.astype(np.float64) + 1j * A_im.astype(np.float64)
    return x, Bm, Cm, dt, A, None if Dk is None else Dk.astype(np.float64)


@pytest.mark.parametrize("n", [1, 2, 17, 4096, 10 ** 9])
def test_step_n_vs_oracle(n):
    import torch
    import complex_valued_state_amd as cssd
    B, H, D, N = 3, 6, 32, 64
    tok, A_re, A_im, Dk, h0 = _inputs(70, B, H, D, N)
    log(f"  step_n n={n} B{B} H{H} D{D} N{N}")
    h_re, h_im = _dev(h0.real.copy()), _dev(h0.imag.copy())
    y = cssd.cssd_step_n(*_args(tok, A_re, A_im, Dk), h_re, h_im, n)
    torch.cuda.synchronize()
    yw, hw = oracle.step_n(*_oracle_args(tok, A_re, A_im, Dk), h0.astype(np.complex128), n)
    assert rel_err(_c(*y), yw) <= TOL, rel_err(_c(*y), yw)
    assert rel_err(_c(h_re, h_im), hw) <= TOL, rel_err(_c(h_re, h_im), hw)
    for k in range(H):  # every head on its own scale (a = 1 grows like n)
        assert rel_err(_c(*y)[:, k], yw[:, k]) <= TOL, (k, rel_err(_c(*y)[:, k], yw[:, k]))
        assert rel_err(_c(h_re, h_im)[:, k], hw[:, k]) <= TOL, k


def test_step_n_is_repeated_steps():
    """n calls of cssd_step with the same token leave the same state as one
    cssd_step_n(n) (both on the GPU, fp32)."""
    import torch
    import complex_valued_state_amd as cssd
    B, H, D, N, n = 2, 4, 64, 128, 33
    tok, A_re, A_im, Dk, h0 = _inputs(71, B, H, D, N)
    args = _args(tok, A_re, A_im, Dk)
    h1 = [_dev(h0.real.copy()), _dev(h0.imag.copy())]
    h2 = [_dev(h0.real.copy()), _dev(h0.imag.copy())]
    for _ in range(n):
        y1 = cssd.cssd_step(*args, *h1)
    y2 = cssd.cssd_step_n(*args, *h2, n)
    torch.cuda.synchronize()
    assert rel_err(_c(*y2), _c(*y1)) <= TOL
    assert rel_err(_c(*h2), _c(*h1)) <= TOL


def test_step_n_one_is_step_bitwise():
    import torch
    import complex_valued_state_amd as cssd
    B, H, D, N = 2, 4, 16, 32
    tok, A_re, A_im, Dk, h0 = _inputs(72, B, H, D, N)
    args = _args(tok, A_re, A_im, Dk)
    h1 = [_dev(h0.real.copy()), _dev(h0.imag.copy())]
    h2 = [_dev(h0.real.copy()), _dev(h0.imag.copy())]
    y1 = cssd.cssd_step(*args, *h1)
    y2 = cssd.cssd_step_n(*args, *h2, 1)
    torch.cuda.synchronize()
    for a, b in zip(list(y1) + h1, list(y2) + h2):
        assert torch.equal(a, b)


def test_step_n_full_decode_shape():
    """The decode shape (batch 256, 48 heads, N 128, D 64) for 4096 steps at once."""
    import torch
    import complex_valued_state_amd as cssd
    B, H, D, N, n = 256, 48, 64, 128, 4096
    tok = wl.decode_step(4, 0, B, H, D, N)
    A_re, A_im, Dk = wl.decode_params(4, H)
    log(f"  step_n decode shape n={n}")
    h_re = torch.zeros((B, H, N, D), dtype=torch.float32, device="cuda:0")
    h_im = torch.zeros_like(h_re)
    y = cssd.cssd_step_n(*_args(tok, A_re, A_im, Dk), h_re, h_im, n)
    torch.cuda.synchronize()
    yw, hw = oracle.step_n(*_oracle_args(tok, A_re, A_im, Dk), np.zeros((B, H, N, D)), n)
    assert rel_err(_c(*y), yw) <= TOL
    assert rel_err(_c(h_re, h_im), hw) <= TOL


@pytest.mark.parametrize("B,H,D,N", [(3, 4, 16, 16), (2, 6, 64, 128), (256, 48, 64, 128)])
def test_step_infinite_vs_oracle(B, H, D, N):
    import torch
    import complex_valued_state_amd as cssd
    tok = wl.decode_step(73, 0, B, H, D, N)
    A_re, A_im, Dk = wl.decode_params(73, H)
    A_re[0] = -1e4                     # a vanishing decay: y = (C . B) x + D x
    log(f"  step_infinite B{B} H{H} D{D} N{N}")
    y = cssd.cssd_step_infinite(*_args(tok, A_re, A_im, Dk))
    torch.cuda.synchronize()
    yw = oracle.step_infinite(*_oracle_args(tok, A_re, A_im, Dk))
    assert rel_err(_c(*y), yw) <= TOL
    for k in range(H):
        assert rel_err(_c(*y)[:, k], yw[:, k]) <= TOL, k


def test_step_infinite_is_the_limit_of_step_n():
    """cssd_step_n with n large enough that |a|^n underflows gives the stationary
    output, whatever the start state."""
    import torch
    import complex_valued_state_amd as cssd
    B, H, D, N = 2, 5, 32, 32
    tok = wl.decode_step(74, 0, B, H, D, N)
    A_re, A_im, Dk = wl.decode_params(74, H)
    args = _args(tok, A_re, A_im, Dk)
    rng = np.random.default_rng(74)
    h_re = _dev(rng.standard_normal((B, H, N, D)).astype(np.float32))
    h_im = _dev(rng.standard_normal((B, H, N, D)).astype(np.float32))
    y_n = cssd.cssd_step_n(*args, h_re, h_im, 1 << 20)
    y_inf = cssd.cssd_step_infinite(*args)
    torch.cuda.synchronize()
    assert rel_err(_c(*y_n), _c(*y_inf)) <= TOL
