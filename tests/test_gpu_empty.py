"""Empty problems on the GPU (needs an MI355X): zero time steps, batch rows or
heads, through the C-ABI, against the oracle on the same seeded inputs.  A scan
of no steps leaves the state as it was, so these results are exact copies or
exact zeros and are compared bit for bit.  Outputs are pre-filled with NaN so
that a value not written shows."""
import numpy as np
import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    return t if dtype is None else t.to(dtype)


def _nan(*shape):
    import torch
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda:0")


def _problem(seed, Bsz, T, H, D, N):
    rng = np.random.default_rng(seed)
    c = lambda *s: (rng.standard_normal(s) + 1j * rng.standard_normal(s)).astype(np.complex64)
    x, Bm, Cm = c(Bsz, T, H, D), c(Bsz, T, H, N), c(Bsz, T, H, N)
    dt = rng.standard_normal((Bsz, T, H)).astype(np.float32)
    A = (-rng.uniform(0.1, 1.0, H) + 1j * rng.uniform(-3, 3, H)).astype(np.complex64)
    Dk = rng.standard_normal(H).astype(np.float32)
    h0 = c(Bsz, H, N, D)
    return x, Bm, Cm, dt, A, Dk, h0


def _to_np(re, im):
    return re.double().cpu().numpy() + 1j * im.double().cpu().numpy()


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("with_h0", [True, False])
def test_forward_zero_steps_passes_the_state(bf16, with_h0):
    import torch
    import complex_valued_state_amd as cssd
    import oracle
    Bsz, T, H, D, N, C = 2, 0, 3, 32, 64, 64
    log(f"forward T=0 bf16={bf16} h0={with_h0}")
    x, Bm, Cm, dt, A, Dk, h0 = _problem(11, Bsz, T, H, D, N)
    io = torch.bfloat16 if bf16 else torch.float32
    pl = lambda a: (_dev(a.real, io), _dev(a.imag, io))
    hT = (_nan(Bsz, H, N, D), _nan(Bsz, H, N, D))
    y = (_nan(Bsz, T, H, D), _nan(Bsz, T, H, D))
    with cssd.profile() as prof:
        out = cssd.cssd_forward(*pl(x), *pl(Bm), *pl(Cm), _dev(dt), _dev(A.real), _dev(A.imag),
                                _dev(Dk), (_dev(h0.real), _dev(h0.imag)) if with_h0 else None,
                                chunk=C, out=(*y, *hT))
        torch.cuda.synchronize()
    assert prof.launches["k_fill"] == 2 and prof.launches["k_chunk_scan"] == 0
    assert out[0].shape == (Bsz, 0, H, D)
    _, want = oracle.forward(x.astype(np.complex128), Bm.astype(np.complex128),
                             Cm.astype(np.complex128), dt.astype(np.float64),
                             A.astype(np.complex128), Dk.astype(np.float64),
                             h0.astype(np.complex128) if with_h0 else None)
    assert np.array_equal(_to_np(*hT), want)


@pytest.mark.parametrize("shape", [(0, 64, 3, 16, 16, 16), (2, 64, 0, 16, 16, 16),
                                   (0, 0, 0, 64, 64, 64)])
def test_forward_no_rows_or_heads(shape):
    import torch
    import complex_valued_state_amd as cssd
    Bsz, T, H, D, N, C = shape
    log(f"forward empty {shape}")
    e = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda:0")
    y_re, y_im, hT_re, hT_im = cssd.cssd_forward(
        e(Bsz, T, H, D), e(Bsz, T, H, D), e(Bsz, T, H, N), e(Bsz, T, H, N), e(Bsz, T, H, N),
        e(Bsz, T, H, N), e(Bsz, T, H), e(H), e(H), None, None, chunk=C)
    torch.cuda.synchronize()
    assert y_re.shape == (Bsz, T, H, D) and hT_re.shape == (Bsz, H, N, D)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("with_dhT", [True, False])
def test_backward_zero_steps(with_dhT, bf16):
    """T = 0: dh0 = dhT, dA and dDskip are empty sums; with bf16 x, B, C (and no
    y, which the backward does not read) nothing is widened either."""
    import torch
    import complex_valued_state_amd as cssd
    import oracle
    Bsz, T, H, D, N, C = 2, 0, 3, 64, 64, 64
    log(f"backward T=0 dhT={with_dhT} bf16={bf16}")
    x, Bm, Cm, dt, A, Dk, h0 = _problem(12, Bsz, T, H, D, N)
    rng = np.random.default_rng(13)
    dhT = (rng.standard_normal((Bsz, H, N, D)) + 1j * rng.standard_normal((Bsz, H, N, D))
           ).astype(np.complex64)
    pl = lambda a: (_dev(a.real), _dev(a.imag))
    io = (lambda a: tuple(t.to(torch.bfloat16) for t in pl(a))) if bf16 else pl
    dy = np.zeros((Bsz, T, H, D), np.complex64)
    with cssd.profile() as prof:
        g = cssd.cssd_backward(*io(x), *io(Bm), *io(Cm), _dev(dt), _dev(A.real), _dev(A.imag),
                               _dev(Dk), pl(h0), None if bf16 else pl(dy), pl(dy),
                               pl(dhT) if with_dhT else None, chunk=C)
        torch.cuda.synchronize()
    assert prof.launches["k_fill"] == 5 and prof.launches["k_bwd_dx"] == 0
    assert prof.launches["k_widen"] == 0
    w = oracle.backward(x.astype(np.complex128), Bm.astype(np.complex128),
                        Cm.astype(np.complex128), dt.astype(np.float64), A.astype(np.complex128),
                        Dk.astype(np.float64), h0.astype(np.complex128), dy.astype(np.complex128),
                        dhT.astype(np.complex128) if with_dhT else None)
    assert np.array_equal(_to_np(g["dh0_re"], g["dh0_im"]), w["dh0"])
    assert np.array_equal(_to_np(g["dA_re"], g["dA_im"]), w["dA"])
    assert np.array_equal(g["dD"].double().cpu().numpy(), w["dD"])
    assert g["dx_re"].shape == (Bsz, 0, H, D) and g["ddt"].shape == (Bsz, 0, H)


def test_backward_no_batch_zeroes_the_head_sums():
    import torch
    import complex_valued_state_amd as cssd
    Bsz, T, H, D, N, C = 0, 64, 4, 16, 32, 16
    log("backward B=0")
    e = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda:0")
    g = cssd.cssd_backward(e(Bsz, T, H, D), e(Bsz, T, H, D), e(Bsz, T, H, N), e(Bsz, T, H, N),
                           e(Bsz, T, H, N), e(Bsz, T, H, N), e(Bsz, T, H), e(H), e(H), e(H),
                           None, (e(Bsz, T, H, D), e(Bsz, T, H, D)),
                           (e(Bsz, T, H, D), e(Bsz, T, H, D)), None, chunk=C)
    torch.cuda.synchronize()
    for k in ("dA_re", "dA_im", "dD"):
        assert g[k].shape == (H,) and not torch.any(g[k] != 0).item(), k


@pytest.mark.parametrize("mode", ["copy", "in_place", "zero"])
def test_phase_scan_zero_steps(mode):
    import torch
    import complex_valued_state_amd as cssd
    import oracle
    Bsz, T, H, N = 3, 0, 2, 16
    log(f"phase scan T=0 {mode}")
    rng = np.random.default_rng(14)
    psi0 = (rng.standard_normal((Bsz, H, N)) + 1j * rng.standard_normal((Bsz, H, N))
            ).astype(np.complex64)
    z = _dev(np.zeros((Bsz, T, H, N), np.float32))
    p0 = (_dev(psi0.real), _dev(psi0.imag))
    psiT = p0 if mode == "in_place" else (_nan(Bsz, H, N), _nan(Bsz, H, N))
    cssd.cssd_phase_scan(z, z.clone(), z.clone(), z.clone(), None if mode == "zero" else p0,
                         out=(z.clone(), z.clone(), *psiT))
    torch.cuda.synchronize()
    zz = np.zeros((Bsz, T, H, N))
    _, want = oracle.phase_scan(zz, zz, zz.astype(complex),
                                None if mode == "zero" else psi0.astype(np.complex128))
    assert np.array_equal(_to_np(*psiT), want)


@pytest.mark.parametrize("bf16", [False, True])
def test_born_attention_no_rows(bf16):
    import torch
    import complex_valued_state_amd as cssd
    log(f"born T=0 bf16={bf16}")
    dt = torch.bfloat16 if bf16 else torch.float32
    e = torch.zeros((2, 0, 3, 32), dtype=dt, device="cuda:0")
    out = cssd.cssd_born_attention(e, e.clone(), e.clone(), e.clone(), e.clone(), e.clone())
    torch.cuda.synchronize()
    assert out[0].shape == (2, 0, 3, 32)


def test_decode_no_rows():
    import torch
    import complex_valued_state_amd as cssd
    log("decode B=0")
    H, D, N = 4, 32, 16
    e = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda:0")
    y = cssd.cssd_step(e(0, H, D), e(0, H, D), e(0, H, N), e(0, H, N), e(0, H, N), e(0, H, N),
                       e(0, H), e(H), e(H), None, e(0, H, N, D), e(0, H, N, D))
    torch.cuda.synchronize()
    assert y[0].shape == (0, H, D)
