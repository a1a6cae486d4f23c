"""GPU parity of cssd_backward (the gradients of the chunkwise scan) against the
oracle's reverse-mode recurrence, which is pinned by finite differences
(needs an MI355X)."""
import numpy as np
import pytest

import cssd_workloads as wl
import oracle
from gpu_util import dev_inputs, log, rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-4


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _grads(inp: wl.ForwardInputs, with_dhT: bool, seed: int, chunk=None):
    """(gpu gradients, oracle gradients) as complex / real numpy arrays."""
    import torch
    import complex_valued_state_amd as cssd
    d = dev_inputs(inp)
    Bsz, T, H, D = inp.x_re.shape
    N = inp.B_re.shape[-1]
    rng = np.random.default_rng(seed)
    gy = (np.sqrt(0.5) * (rng.standard_normal((Bsz, T, H, D))
                          + 1j * rng.standard_normal((Bsz, T, H, D)))).astype(np.complex64)
    ghT = None
    if with_dhT:
        ghT = (np.sqrt(0.5) * (rng.standard_normal((Bsz, H, N, D))
                               + 1j * rng.standard_normal((Bsz, H, N, D)))).astype(np.complex64)
    c = chunk or inp.chunk
    y = cssd.cssd_forward(d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"],
                          d["dt"], d["A_re"], d["A_im"], d["Dskip"], d["h0"], chunk=c,
                          return_state=False)[:2]
    g = cssd.cssd_backward(d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"],
                           d["dt"], d["A_re"], d["A_im"], d["Dskip"], d["h0"], y,
                           (_dev(gy.real.copy()), _dev(gy.imag.copy())),
                           None if ghT is None else (_dev(ghT.real.copy()), _dev(ghT.imag.copy())),
                           chunk=c)
    torch.cuda.synchronize()
    n = lambda t: None if t is None else t.double().cpu().numpy()
    got = {"dx": n(g["dx_re"]) + 1j * n(g["dx_im"]), "dB": n(g["dB_re"]) + 1j * n(g["dB_im"]),
           "dC": n(g["dC_re"]) + 1j * n(g["dC_im"]), "ddt": n(g["ddt"]),
           "dA": n(g["dA_re"]) + 1j * n(g["dA_im"]), "dD": n(g["dD"]),
           "dh0": n(g["dh0_re"]) + 1j * n(g["dh0_im"])}
    x, Bm, Cm, dt, A, Dk, h0 = inp.complex()
    want = oracle.backward(x, Bm, Cm, dt, A, Dk, h0, gy.astype(np.complex128),
                           None if ghT is None else ghT.astype(np.complex128))
    return got, want


def _check(got, want, skip_dD=False):
    for k in ("dx", "dB", "dC", "ddt", "dA", "dh0") + (() if skip_dD else ("dD",)):
        err = rel_err(got[k], want[k])
        log(f"    {k}: rel err {err:.2e}")
        assert err <= TOL, (k, err)


SMALL = [
    # (B, T, H, D, N, C, with_h0, with_dskip, with_dhT)
    (1, 1, 1, 16, 16, 16, True, True, True),     # a single step
    (1, 15, 2, 16, 16, 16, True, True, False),   # T < C
    (1, 64, 2, 16, 16, 64, False, True, True),   # one chunk
    (2, 100, 3, 32, 64, 16, True, True, True),   # ragged tail, many chunks
    (1, 257, 2, 64, 32, 64, False, False, False),
    (2, 130, 2, 32, 64, 64, True, True, True),
    (1, 300, 2, 16, 128, 128, True, True, True),  # largest N and C
    (2, 50, 2, 128, 16, 32, False, True, True),   # largest D
    (3, 128, 2, 64, 64, 32, True, True, True),
    (2, 200, 3, 64, 64, 64, True, True, True),    # N = D = C = 64 (fused adjoint pass), ragged tail
    (1, 64, 2, 64, 64, 64, False, True, False),   # the same, one chunk, no dhT
    (3, 190, 3, 64, 64, 64, True, False, False),  # the same, no dhT, 9 (b, h) over 8 XCDs
    (1, 512, 2, 32, 32, 16, True, True, True),    # 32 chunks per (b, h) in the recompute
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}T{}H{}D{}N{}C{}{}{}{}".format(
    *c[:6], "_h0" if c[6] else "", "_D" if c[7] else "", "_dhT" if c[8] else ""))
def test_backward_small_shapes(case):
    B, T, H, D, N, C, with_h0, with_d, with_dhT = case
    inp = wl.random_forward(2000 + T, B, T, H, D, N, C, with_h0=with_h0, with_dskip=with_d,
                            name="bwd")
    log(f"  backward {case}")
    got, want = _grads(inp, with_dhT, seed=T)
    _check(got, want, skip_dD=not with_d)


def test_backward_chunk_size_invariance():
    """The gradients do not depend on the chunk size the scan is evaluated with."""
    inp = wl.random_forward(31, 2, 128, 3, 32, 32, 16, with_h0=True, name="bwd_cinv")
    ref = None
    for C in (16, 32, 64, 128):
        got, want = _grads(inp, True, seed=5, chunk=C)
        _check(got, want)
        if ref is None:
            ref = got
        for k in ("dx", "dB", "dC", "ddt", "dA", "dh0"):
            assert rel_err(got[k], ref[k]) <= TOL, (C, k)


def test_backward_mamba_layer_shape_reduced_batch():
    """The B8 T2048 H48 D64 N64 C64 layer shape at batch 1 and 6 heads, every
    gradient against the oracle."""
    inp = wl.random_forward(1, 1, 2048, 6, 64, 64, 64, name="bwd_cfg1")
    log("  backward B1 T2048 H6 D64 N64 C64")
    got, want = _grads(inp, True, seed=11)
    _check(got, want)


SAVED = [
    # (B, T, H, D, N, C, with_h0, with_dskip, with_dhT)
    (2, 200, 3, 64, 64, 64, True, True, True),     # staged kernels and fused adjoint pass
    (3, 190, 3, 64, 64, 64, False, True, False),
    (2, 100, 3, 32, 64, 16, True, True, True),     # tile kernels, adjoint pass in two launches
    (1, 300, 2, 16, 128, 128, True, False, False),
]


@pytest.mark.parametrize("case", SAVED, ids=lambda c: "B{}T{}H{}D{}N{}C{}{}{}{}".format(
    *c[:6], "_h0" if c[6] else "", "_D" if c[7] else "", "_dhT" if c[8] else ""))
def test_backward_saved_states(case):
    """cssd_backward_saved on the workspace and final state a cssd_forward call
    left gives cssd_backward's gradients bit for bit (same kernels on the same
    states), and both meet the oracle."""
    import torch
    import complex_valued_state_amd as cssd
    Bsz, T, H, D, N, C, with_h0, with_d, with_dhT = case
    log(f"backward saved {case}")
    inp = wl.random_forward(61, Bsz, T, H, D, N, C, with_h0=with_h0, with_dskip=with_d)
    d = dev_inputs(inp)
    rng = np.random.default_rng(62)
    cz = lambda *s: (np.sqrt(0.5) * (rng.standard_normal(s) + 1j * rng.standard_normal(s))
                     ).astype(np.complex64)
    gy = cz(Bsz, T, H, D)
    ghT = cz(Bsz, H, N, D) if with_dhT else None
    pl = lambda a: (_dev(a.real.copy()), _dev(a.imag.copy()))
    ins = (d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"], d["dt"], d["A_re"],
           d["A_im"], d["Dskip"], d["h0"])
    ws = torch.empty(cssd.cssd_backward_workspace_size(Bsz, T, H, D, N, C), dtype=torch.uint8,
                     device="cuda:0")
    y_re, y_im, hT_re, hT_im = cssd.cssd_forward(*ins, chunk=C, workspace=ws)
    with cssd.profile() as prof:
        gs = cssd.cssd_backward_saved(*ins, (y_re, y_im), (hT_re, hT_im), pl(gy),
                                      None if ghT is None else pl(ghT), chunk=C, workspace=ws)
        torch.cuda.synchronize()
    assert prof.launches["k_cumsum"] == 0 and prof.launches["k_state_scan"] == 0
    g = cssd.cssd_backward(*ins, (y_re, y_im), pl(gy), None if ghT is None else pl(ghT), chunk=C)
    torch.cuda.synchronize()
    for k, v in g.items():
        if v is not None:
            assert torch.equal(v, gs[k]), k
    n = lambda t: None if t is None else t.double().cpu().numpy()
    got = {"dx": n(gs["dx_re"]) + 1j * n(gs["dx_im"]), "dB": n(gs["dB_re"]) + 1j * n(gs["dB_im"]),
           "dC": n(gs["dC_re"]) + 1j * n(gs["dC_im"]), "ddt": n(gs["ddt"]),
           "dA": n(gs["dA_re"]) + 1j * n(gs["dA_im"]), "dD": n(gs["dD"]),
           "dh0": n(gs["dh0_re"]) + 1j * n(gs["dh0_im"])}
    x, Bm, Cm, dt, A, Dk, h0 = inp.complex()
    want = oracle.backward(x, Bm, Cm, dt, A, Dk, h0, gy.astype(np.complex128),
                           None if ghT is None else ghT.astype(np.complex128))
    _check(got, want, skip_dD=not with_d)


TOL_BF16 = 2e-2

BF16_BWD = [
    # (B, T, H, D, N, C, with_h0, with_dskip, with_dhT)
    (2, 130, 2, 64, 64, 64, True, True, True),    # bf16 matrix-core forward, fused adjoint pass
    (1, 100, 3, 32, 64, 32, False, True, False),  # register-operand forward, ragged tail
    (1, 70, 2, 32, 32, 64, True, False, True),    # matrix-core forward at N = D = 32
    (1, 300, 2, 16, 128, 128, True, True, True),  # largest N and C (tile kernels)
    (2, 50, 2, 128, 16, 32, False, True, True),   # largest D, ragged tail
]


@pytest.mark.parametrize("case", BF16_BWD, ids=lambda c: "B{}T{}H{}D{}N{}C{}{}{}{}".format(
    *c[:6], "_h0" if c[6] else "", "_D" if c[7] else "", "_dhT" if c[8] else ""))
def test_backward_bf16_inputs(case):
    """bf16 x, B, C into cssd_backward.  The widening to fp32 is exact and y is
    not read (the log-decay gradient takes conj(C) . dC in its place), so the
    gradients equal those of the fp32 call on the rounded values bit for bit,
    whichever forward's y is passed, or none; every gradient meets the fp32 bar
    against the oracle on the rounded inputs, and the bf16-input bar against the
    oracle on the pre-rounding inputs."""
    import torch
    import complex_valued_state_amd as cssd
    Bsz, T, H, D, N, C, with_h0, with_d, with_dhT = case
    log(f"backward bf16 inputs {case}")
    kw = dict(with_h0=with_h0, with_dskip=with_d, name="bwd_bf16")
    inp32 = wl.random_forward(71 + T, Bsz, T, H, D, N, C, **kw)
    inp16 = wl.random_forward(71 + T, Bsz, T, H, D, N, C, in_dtype="bf16", **kw)
    d16 = dev_inputs(inp16)
    # the same rounded values as fp32 device planes
    d32 = dict(d16)
    for k in ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im"):
        d32[k] = d16[k].float()
    rng = np.random.default_rng(72)
    cz = lambda *s: (np.sqrt(0.5) * (rng.standard_normal(s) + 1j * rng.standard_normal(s))
                     ).astype(np.complex64)
    gy = cz(Bsz, T, H, D)
    ghT = cz(Bsz, H, N, D) if with_dhT else None
    pl = lambda a: (_dev(a.real.copy()), _dev(a.imag.copy()))
    ins = lambda d: (d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"], d["dt"],
                     d["A_re"], d["A_im"], d["Dskip"], d["h0"])
    dyt, dhTt = pl(gy), None if ghT is None else pl(ghT)
    n = lambda t: None if t is None else t.double().cpu().numpy()

    # the fp32 call on the rounded values, given the fp32 forward's y of them
    y32 = cssd.cssd_forward(*ins(d32), chunk=C, return_state=False)[:2]
    g32 = cssd.cssd_backward(*ins(d32), y32, dyt, dhTt, chunk=C)
    # the bf16 call: y not passed, and the bf16 forward's y passed
    g16 = cssd.cssd_backward(*ins(d16), None, dyt, dhTt, chunk=C)
    y16 = cssd.cssd_forward(*ins(d16), chunk=C, return_state=False)[:2]
    g16y = cssd.cssd_backward(*ins(d16), y16, dyt, dhTt, chunk=C)
    torch.cuda.synchronize()
    for k, v in g32.items():
        if v is not None:
            assert torch.equal(g16[k], v), k
            assert torch.equal(g16y[k], v), k

    got = {"dx": n(g16["dx_re"]) + 1j * n(g16["dx_im"]),
           "dB": n(g16["dB_re"]) + 1j * n(g16["dB_im"]),
           "dC": n(g16["dC_re"]) + 1j * n(g16["dC_im"]), "ddt": n(g16["ddt"]),
           "dA": n(g16["dA_re"]) + 1j * n(g16["dA_im"]), "dD": n(g16["dD"]),
           "dh0": n(g16["dh0_re"]) + 1j * n(g16["dh0_im"])}
    gyc = gy.astype(np.complex128)
    ghc = None if ghT is None else ghT.astype(np.complex128)
    want16 = oracle.backward(*inp16.complex(), gyc, ghc)
    want32 = oracle.backward(*inp32.complex(), gyc, ghc)
    for k in ("dx", "dB", "dC", "ddt", "dA", "dh0") + (("dD",) if with_d else ()):
        err, err32 = rel_err(got[k], want16[k]), rel_err(got[k], want32[k])
        log(f"    {k}: rel err {err:.2e} vs the rounded inputs, {err32:.2e} vs pre-rounding")
        assert err <= TOL, (k, err)
        assert err32 <= TOL_BF16, (k, err32)


def test_backward_ignores_y():
    """y is not read by either backward entry point: with fp32 inputs, passing no
    y, the forward's y or an unrelated tensor gives the same gradients bit for
    bit, on the staged (N = D = C = 64) and the tile kernels."""
    import torch
    import complex_valued_state_amd as cssd
    for (Bsz, T, H, D, N, C) in ((2, 130, 2, 64, 64, 64), (1, 100, 3, 32, 64, 16)):
        log(f"backward without y B{Bsz} T{T} H{H} D{D} N{N} C{C}")
        inp = wl.random_forward(81 + T, Bsz, T, H, D, N, C, with_h0=True, name="bwd_noy")
        d = dev_inputs(inp)
        ins = (d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"], d["dt"],
               d["A_re"], d["A_im"], d["Dskip"], d["h0"])
        g = torch.Generator(device="cuda:0").manual_seed(82)
        pl = lambda *s: tuple(torch.randn(s, generator=g, device="cuda:0") for _ in range(2))
        dy, dhT, junk = pl(Bsz, T, H, D), pl(Bsz, H, N, D), pl(Bsz, T, H, D)
        y = cssd.cssd_forward(*ins, chunk=C, return_state=False)[:2]
        ref = cssd.cssd_backward(*ins, y, dy, dhT, chunk=C)
        for other in (None, junk):
            got = cssd.cssd_backward(*ins, other, dy, dhT, chunk=C)
            torch.cuda.synchronize()
            for k, v in ref.items():
                if v is not None:
                    assert torch.equal(got[k], v), k


def test_backward_maximum_size_sampled():
    """The gradient pass at the largest size the entry points accept at
    D = N = C = 64 with 64 heads, taken as B64 T8191 H64 (2^31 - 2^18 elements
    per plane, a ragged last chunk, the size checks met with equality; about 180
    GB of HBM with inputs, outputs and workspaces).  Inputs are drawn on the
    device (torch's seeded generator, the config-0 distributions).  The oracle
    runs three whole (b, h) sequences, among them the last one (the highest
    addresses); dA and dDskip sum over every batch row and are checked at the
    smaller sizes above."""
    import math
    import torch
    import complex_valued_state_amd as cssd
    Bsz, T, H, D, N, C = 64, 8191, 64, 64, 64, 64
    assert Bsz * T * H * max(D, N) == (1 << 31) - (1 << 18)
    log("backward max size: drawing inputs on the device")
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(92)
    r = math.sqrt(0.5)
    pl = lambda *s: [torch.randn(s, generator=g, device=dev).mul_(r) for _ in range(2)]
    x, Bm, Cm, dy = pl(Bsz, T, H, D), pl(Bsz, T, H, N), pl(Bsz, T, H, N), pl(Bsz, T, H, D)
    dhT = pl(Bsz, H, N, D)
    dt = torch.randn((Bsz, T, H), generator=g, device=dev)
    a_re = -(0.1 + 0.9 * torch.rand(H, generator=g, device=dev))
    a_im = (2 * torch.rand(H, generator=g, device=dev) - 1) * math.pi
    dk = torch.randn(H, generator=g, device=dev)
    ins = (*x, *Bm, *Cm, dt, a_re, a_im, dk, None)
    log("backward max size: forward, backward")
    y = cssd.cssd_forward(*ins, chunk=C, return_state=False)[:2]
    torch.cuda.synchronize()
    gr = cssd.cssd_backward(*ins, y, dy, dhT, chunk=C)
    torch.cuda.synchronize()
    log("backward max size: oracle")
    f64 = lambda t: t.double().cpu().numpy()
    cplx = lambda p, sl: f64(sl(p[0])) + 1j * f64(sl(p[1]))
    for b, h in ((Bsz - 1, H - 1), (0, 0), (37, 21)):
        sl = lambda t: t[b:b + 1, :, h:h + 1]
        slh = lambda t: t[b:b + 1, h:h + 1]
        A = np.array([float(a_re[h]) + 1j * float(a_im[h])])
        want = oracle.backward(cplx(x, sl), cplx(Bm, sl), cplx(Cm, sl), f64(sl(dt)), A,
                               np.array([float(dk[h])]), None, cplx(dy, sl), cplx(dhT, slh))
        got = {"dx": f64(sl(gr["dx_re"])) + 1j * f64(sl(gr["dx_im"])),
               "dB": f64(sl(gr["dB_re"])) + 1j * f64(sl(gr["dB_im"])),
               "dC": f64(sl(gr["dC_re"])) + 1j * f64(sl(gr["dC_im"])),
               "ddt": f64(sl(gr["ddt"])),
               "dh0": f64(slh(gr["dh0_re"])) + 1j * f64(slh(gr["dh0_im"]))}
        for k, v in got.items():
            err = rel_err(v, want[k])
            log(f"  (b, h) = ({b}, {h}) {k}: rel err {err:.2e}")
            assert err <= TOL, (b, h, k, err)
    del x, Bm, Cm, dy, dhT, dt, y, gr
    torch.cuda.empty_cache()
