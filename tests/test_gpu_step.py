"""GPU parity of cssd_step (the recurrent decode step) against the oracle and
the constant-input closed forms (needs an MI355X)."""
import math

import numpy as np
import pytest

import cssd_workloads as wl
from gpu_util import dev_inputs, gpu_forward, log, oracle_forward, rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-4


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _run_steps(steps: wl.StepInputs, A_re, A_im, Dskip, h0=None):
    """Drive cssd_step over the leading (token) axis; returns (y (S,B,H,D), h) complex."""
    import torch
    import complex_valued_state_amd as cssd
    S, B, H, D = steps.x_re.shape
    N = steps.B_re.shape[-1]
    d = {f: _dev(getattr(steps, f)) for f in ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt")}
    a_re, a_im = _dev(A_re), _dev(A_im)
    dk = None if Dskip is None else _dev(Dskip)
    if h0 is None:
        h_re = torch.zeros((B, H, N, D), dtype=torch.float32, device="cuda:0")
        h_im = torch.zeros_like(h_re)
    else:
        h_re, h_im = _dev(h0.real.astype(np.float32)), _dev(h0.imag.astype(np.float32))
    ys_re = torch.empty((S, B, H, D), dtype=torch.float32, device="cuda:0")
    ys_im = torch.empty_like(ys_re)
    for s in range(S):
        cssd.cssd_step(d["x_re"][s], d["x_im"][s], d["B_re"][s], d["B_im"][s], d["C_re"][s],
                       d["C_im"][s], d["dt"][s], a_re, a_im, dk, h_re, h_im,
                       out=(ys_re[s], ys_im[s]))
    torch.cuda.synchronize()
    c = lambda r, i: r.double().cpu().numpy() + 1j * i.double().cpu().numpy()
    return c(ys_re, ys_im), c(h_re, h_im)


def _as_sequence(steps: wl.StepInputs, A_re, A_im, Dskip, chunk=16):
    """The same tokens as one (B, T=S, H, .) sequence for the oracle."""
    t = lambda a: np.ascontiguousarray(np.moveaxis(a, 0, 1))
    return wl.ForwardInputs(t(steps.x_re), t(steps.x_im), t(steps.B_re), t(steps.B_im),
                            t(steps.C_re), t(steps.C_im), t(steps.dt), A_re, A_im, Dskip, chunk)


@pytest.mark.parametrize("B,H,D,N", [(2, 3, 16, 32), (1, 2, 128, 16), (3, 2, 32, 128), (2, 2, 64, 64)])
def test_step_small_vs_oracle(B, H, D, N):
    S = 20
    steps = wl.decode_steps(40 + D + N, S, B, H, D, N)
    A_re, A_im, Dk = wl.decode_params(40, H)
    log(f"  step B{B} H{H} D{D} N{N} x{S}")
    y, h = _run_steps(steps, A_re, A_im, Dk)
    yr, hr = oracle_forward(_as_sequence(steps, A_re, A_im, Dk))
    assert rel_err(np.moveaxis(y, 0, 1), yr) <= TOL
    assert rel_err(h, hr) <= TOL


def test_step_decay_zero():
    B, H, D, N = 2, 3, 64, 128
    steps = wl.decode_steps(41, 3, B, H, D, N)
    steps.dt[:] = 0
    A_re = np.full(H, -1e4, dtype=np.float32)
    A_im = np.array([0.3, -1.0, 2.0], dtype=np.float32)
    Dk = np.array([0.5, -1.5, 2.0], dtype=np.float32)
    y, h = _run_steps(steps, A_re, A_im, Dk)
    x, Bm, Cm, _ = steps.complex()
    want = np.einsum("sbhn,sbhn->sbh", Cm, Bm)[..., None] * x + Dk[None, None, :, None] * x
    assert rel_err(y, want) <= TOL
    assert rel_err(h, np.einsum("bhn,bhd->bhnd", Bm[-1], x[-1])) <= TOL


def test_step_512_tokens_vs_oracle():
    """512 consecutive tokens at the decode shape's H, N, D (batch 4)."""
    B, H, D, N, S = 4, 48, 64, 128, 512
    steps = wl.decode_steps(4, S, B, H, D, N)
    A_re, A_im, Dk = wl.decode_params(4, H)
    log(f"  step 512 tokens B{B} H{H}")
    y, h = _run_steps(steps, A_re, A_im, Dk)
    yr, hr = oracle_forward(_as_sequence(steps, A_re, A_im, Dk))
    ey, eh = rel_err(np.moveaxis(y, 0, 1), yr), rel_err(h, hr)
    log(f"    rel err y={ey:.3e} h={eh:.3e}")
    assert ey <= TOL and eh <= TOL


def test_step_full_decode_shape_sampled():
    """B256 H48 N128 D64 for 16 tokens; sampled sequences against the oracle."""
    s = wl.CONFIG_SHAPES[4]
    B, H, D, N, S = s["B"], s["H"], s["D"], s["N"], 16
    steps = wl.decode_steps(4, S, B, H, D, N)
    A_re, A_im, Dk = wl.decode_params(4, H)
    log(f"  step full shape x{S}")
    y, h = _run_steps(steps, A_re, A_im, Dk)
    import oracle
    for (b, hh) in [(0, 0), (17, 5), (130, 47), (255, 20), (64, 33)]:
        sub = wl.StepInputs(*[np.ascontiguousarray(getattr(steps, f)[:, b:b + 1, hh:hh + 1])
                              for f in ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt")])
        seq = _as_sequence(sub, A_re[hh:hh + 1], A_im[hh:hh + 1], Dk[hh:hh + 1])
        x, Bm, Cm, dt, A, Dd, _ = seq.complex()
        yr, hr = oracle.forward(x, Bm, Cm, dt, A, Dd, None)
        assert rel_err(y[:, b, hh], yr[0, :, 0]) <= TOL, (b, hh)
        assert rel_err(h[b, hh], hr[0, 0]) <= TOL, (b, hh)


def test_step_decode_workload_as_written():
    """The decode workload exactly as specified: batch 256 x 48 heads, N128 D64,
    512 consecutive tokens from a zero state, token s drawn from the streams
    SeedSequence([4, s, k]) (generated on the host in batches while the GPU
    steps).  Every step's y and the final state of six sampled (b, h), the last
    one (255, 47) included, are compared with the oracle run over the same 512
    tokens ("Complex-Valued State Spaces", the naive scan, one token at a time)."""
    import torch
    import complex_valued_state_amd as cssd
    from concurrent.futures import ThreadPoolExecutor
    s4 = wl.CONFIG_SHAPES[4]
    B, H, D, N, S = s4["B"], s4["H"], s4["D"], s4["N"], s4["steps"]
    A_re, A_im, Dk = wl.decode_params(4, H)
    a_re, a_im, dk = _dev(A_re), _dev(A_im), _dev(Dk)
    pairs = [(0, 0), (17, 5), (130, 47), (64, 33), (200, 11), (255, 47)]
    h_re = torch.zeros((B, H, N, D), dtype=torch.float32, device="cuda:0")
    h_im = torch.zeros_like(h_re)
    y_re = torch.empty((S, B, H, D), dtype=torch.float32, device="cuda:0")
    y_im = torch.empty_like(y_re)
    fields = ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt")
    kept = {f: [] for f in fields}  # the sampled sequences' inputs, token by token
    batch = 32
    log(f"  decode workload B{B} H{H} N{N} D{D}, {S} tokens")
    with ThreadPoolExecutor(16) as ex:
        nxt = ex.map(lambda t: wl.decode_step(4, t, B, H, D, N), range(0, min(batch, S)))
        for t0 in range(0, S, batch):
            toks = list(nxt)
            if t0 + batch < S:
                nxt = ex.map(lambda t: wl.decode_step(4, t, B, H, D, N),
                             range(t0 + batch, min(t0 + 2 * batch, S)))
            for j, tok in enumerate(toks):
                d = {f: _dev(getattr(tok, f)) for f in fields}
                cssd.cssd_step(d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"],
                               d["dt"], a_re, a_im, dk, h_re, h_im,
                               out=(y_re[t0 + j], y_im[t0 + j]))
                for f in fields:
                    a = getattr(tok, f)
                    kept[f].append(np.stack([a[b, hh] for b, hh in pairs]))
            torch.cuda.synchronize()
    import oracle
    c = lambda r, i: r.double().cpu().numpy() + 1j * i.double().cpu().numpy()
    worst_y = worst_h = 0.0
    for m, (b, hh) in enumerate(pairs):
        sub = wl.StepInputs(*[np.ascontiguousarray(np.stack(kept[f])[:, m][:, None, None])
                              for f in fields])
        seq = _as_sequence(sub, A_re[hh:hh + 1], A_im[hh:hh + 1], Dk[hh:hh + 1])
        x, Bm, Cm, dt, A, Dd, _ = seq.complex()
        yr, hr = oracle.forward(x, Bm, Cm, dt, A, Dd, None)
        ey = rel_err(c(y_re[:, b, hh], y_im[:, b, hh]), yr[0, :, 0])
        eh = rel_err(c(h_re[b, hh], h_im[b, hh]), hr[0, 0])
        worst_y, worst_h = max(worst_y, ey), max(worst_h, eh)
        assert ey <= TOL and eh <= TOL, (b, hh, ey, eh)
    log(f"    rel err over {S} steps: y={worst_y:.3e} h={worst_h:.3e}")


def test_step_constant_input_closed_form():
    """One draw of (x, B, C, dt) held for n = 4096 tokens at the full decode
    shape, from a zero state: y_n = (1 - a^n)/(1 - a) (C . B) x + D x, and at
    n = 4096 the stationary value (C . B) x / (1 - a) + D x (burn-mamba
    step_constant: the n-step geometric series and its n -> infinity limit, with
    no rotation operator)."""
    import torch
    import complex_valued_state_amd as cssd
    s = wl.CONFIG_SHAPES[4]
    B, H, D, N = s["B"], s["H"], s["D"], s["N"]
    one = wl.decode_step(4, 10_000, B, H, D, N)
    A_re, A_im, Dk = wl.decode_params(4, H)
    d = {f: _dev(getattr(one, f)) for f in ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt")}
    a_re, a_im, dk = _dev(A_re), _dev(A_im), _dev(Dk)
    h_re = torch.zeros((B, H, N, D), dtype=torch.float32, device="cuda:0")
    h_im = torch.zeros_like(h_re)
    x, Bm, Cm, dt = one.complex()
    A = A_re.astype(np.float64) + 1j * A_im.astype(np.float64)
    logdec = np.logaddexp(0.0, dt) * A[None, :]                      # (B, H)
    a = np.exp(logdec)
    score = np.einsum("bhn,bhn->bh", Cm, Bm)
    checkpoints = {1, 2, 64, 1000, 4096}
    # every n = 1..4096 on the first SB batch rows (all heads), in blocks of NB steps
    SB, NB = 8, 512
    keep = [torch.empty((NB, SB, H, D), dtype=torch.float32, device="cuda:0") for _ in range(2)]
    log("  constant-input run, 4096 tokens (every step checked on 8 batch rows)")
    y_re = y_im = None
    worst = 0.0
    for n in range(1, 4097):
        y_re, y_im = cssd.cssd_step(d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"],
                                    d["C_im"], d["dt"], a_re, a_im, dk, h_re, h_im)
        keep[0][(n - 1) % NB].copy_(y_re[:SB])
        keep[1][(n - 1) % NB].copy_(y_im[:SB])
        if n % NB == 0:
            torch.cuda.synchronize()
            ys = keep[0].double().cpu().numpy() + 1j * keep[1].double().cpu().numpy()
            for j in range(NB):
                m = n - NB + 1 + j
                geo = (1.0 - np.exp(m * logdec[:SB])) / (1.0 - a[:SB])
                want = (geo * score[:SB])[..., None] * x[:SB] + Dk[None, :, None] * x[:SB]
                e = rel_err(ys[j], want)
                worst = max(worst, e)
                assert e <= TOL, (m, e)
        if n in checkpoints:
            torch.cuda.synchronize()
            y = y_re.double().cpu().numpy() + 1j * y_im.double().cpu().numpy()
            geo = (1.0 - np.exp(n * logdec)) / (1.0 - a)
            want = (geo * score)[..., None] * x + Dk[None, :, None] * x
            e = rel_err(y, want)
            log(f"    n={n} rel err {e:.3e} (whole batch)")
            assert e <= TOL, n
    log(f"    worst rel err over n = 1..4096 on {SB} batch rows: {worst:.3e}")
    yinf = (score / (1.0 - a))[..., None] * x + Dk[None, :, None] * x
    assert np.max(np.abs(a)) ** 4096 < 1e-6
    assert rel_err(y, yinf) <= TOL


def test_prefill_then_decode():
    """forward over T1 tokens hands its final state to cssd_step, which continues
    the sequence; both match one forward over all T tokens."""
    import torch
    import complex_valued_state_amd as cssd
    B, T, T1, H, D, N = 2, 96, 70, 3, 32, 64
    inp = wl.random_forward(321, B, T, H, D, N, 32, with_h0=True, name="prefill")
    y_all, h_all = gpu_forward(inp)
    pre = wl.ForwardInputs(*[np.ascontiguousarray(getattr(inp, f)[:, :T1]) for f in
                             ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt")],
                           inp.A_re, inp.A_im, inp.Dskip, inp.chunk, inp.h0_re, inp.h0_im)
    d = dev_inputs(pre)
    _, _, h_re, h_im = cssd.cssd_forward(d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"],
                                         d["C_im"], d["dt"], d["A_re"], d["A_im"], d["Dskip"],
                                         d["h0"], chunk=32)
    full = dev_inputs(inp)
    ys = []
    for t in range(T1, T):
        yr_, yi_ = cssd.cssd_step(*(full[k][:, t].contiguous() for k in
                                    ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt")),
                                  full["A_re"], full["A_im"], full["Dskip"], h_re, h_im)
        ys.append(yr_.double().cpu().numpy() + 1j * yi_.double().cpu().numpy())
    torch.cuda.synchronize()
    y_dec = np.stack(ys, axis=1)
    h_dec = h_re.double().cpu().numpy() + 1j * h_im.double().cpu().numpy()
    yr, hr = oracle_forward(inp)
    assert rel_err(y_dec, yr[:, T1:]) <= TOL and rel_err(h_dec, hr) <= TOL
    assert rel_err(y_dec, y_all[:, T1:]) <= TOL and rel_err(h_dec, h_all) <= TOL


def test_step_maximum_size_sampled():
    """The largest decode step accepted at D = 64, N = 128: batch 4096 x 64 heads,
    2^31 elements per state plane (16 GB of state, updated in place).  Inputs are
    drawn on the device (torch's seeded generator); the oracle steps sampled
    (b, h) rows, the last one included."""
    import torch
    import complex_valued_state_amd as cssd
    import oracle
    B, H, D, N = 4096, 64, 64, 128
    assert B * H * D * N == 1 << 31
    log("step max size: drawing inputs on the device")
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(93)
    r = math.sqrt(0.5)
    pl = lambda *s: [torch.randn(s, generator=g, device=dev).mul_(r) for _ in range(2)]
    x, Bm, Cm, h = pl(B, H, D), pl(B, H, N), pl(B, H, N), pl(B, H, N, D)
    dt = torch.randn((B, H), generator=g, device=dev)
    a_re = -(0.1 + 0.9 * torch.rand(H, generator=g, device=dev))
    a_im = (2 * torch.rand(H, generator=g, device=dev) - 1) * math.pi
    dk = torch.randn(H, generator=g, device=dev)
    rows = ((B - 1, H - 1), (0, 0), (2049, 33))
    f64 = lambda t: t.double().cpu().numpy()
    h_before = {bh: (f64(h[0][bh[0], bh[1]]), f64(h[1][bh[0], bh[1]])) for bh in rows}
    log("step max size: step")
    y = cssd.cssd_step(*x, *Bm, *Cm, dt, a_re, a_im, dk, h[0], h[1])
    torch.cuda.synchronize()
    for b, hh in rows:
        one = lambda p: f64(p[0][b:b + 1, hh:hh + 1]) + 1j * f64(p[1][b:b + 1, hh:hh + 1])
        h0 = (h_before[(b, hh)][0] + 1j * h_before[(b, hh)][1])[None, None]
        yr, hr = oracle.step(one(x), one(Bm), one(Cm), f64(dt[b:b + 1, hh:hh + 1]),
                             np.array([float(a_re[hh]) + 1j * float(a_im[hh])]),
                             np.array([float(dk[hh])]), h0)
        ey, eh = rel_err(one(y), yr), rel_err(one(h), hr)
        log(f"  (b, h) = ({b}, {hh}): y {ey:.2e}, state {eh:.2e}")
        assert ey <= TOL and eh <= TOL, (b, hh, ey, eh)
    del x, Bm, Cm, h, dt, y
    torch.cuda.empty_cache()
