"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

None of these re-type the oracle's loop.  Each computes the expected value by a
different route -- an unrolled double sum with explicit products, a geometric
series, an exponential of a summed log-decay, the PAM page's quadratic dual
form, or a number the pages print -- so that a plausible slip in the oracle
(dropped term, wrong sign, conjugated operand, off-by-one in the decay, wrong
index) makes at least one of them fail.  ``test_oracle_mutants.py`` plants such
slips in copies of the oracle source and checks exactly that.

The discretisation a = exp(softplus(dt) A) is evaluated here with library
routines only: ``numpy.logaddexp(0, dt)`` for softplus and complex ``numpy.exp``.

Every pin takes the loaded oracle library (``lib``) and raises AssertionError
on failure.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def disc(dt, A):
    """exp(softplus(dt) * A) via library routines (broadcasting)."""
    return np.exp(np.logaddexp(0.0, np.asarray(dt, dtype=np.float64)) * A)


def crandn(rng, *shape, scale=math.sqrt(0.5)):
    return scale * (rng.standard_normal(shape) + 1j * rng.standard_normal(shape))


def rel_err(got, ref):
    got = np.asarray(got); ref = np.asarray(ref)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


# ---------------------------------------------------------------------------
# p1: brute-force unrolled double sum (T <= 8)
# ---------------------------------------------------------------------------
def bruteforce(x, Bm, Cm, dt, A, Dskip=None, h0=None):
    """Unrolled form of the recurrence (Mamba-3-Lite docs, "The Chunkwise Complex
    SSD Algorithm", section 3: with zero initial state the output is a sum over
    all earlier inputs, each weighted by the product of the decays after it and
    by the score C_t . B_s; the empty product is 1).  The initial-state term
    carries the product of all decays up to t.  Products are formed by explicit
    multiplication of the per-step factors, one pair (t, s) at a time."""
    Bsz, T, H, D = x.shape
    N = Bm.shape[-1]
    y = np.zeros((Bsz, T, H, D), dtype=np.complex128)
    hT = np.zeros((Bsz, H, N, D), dtype=np.complex128)
    for b in range(Bsz):
        for h in range(H):
            a = [complex(disc(dt[b, u, h], A[h])) for u in range(T)]

            def prod(lo, hi):
                p = 1.0 + 0.0j
                for u in range(lo, hi + 1):
                    p *= a[u]
                return p

            for t in range(T):
                acc = np.zeros(D, dtype=np.complex128)
                for s in range(t + 1):
                    score = np.sum(Cm[b, t, h, :] * Bm[b, s, h, :])
                    acc += prod(s + 1, t) * score * x[b, s, h, :]
                if h0 is not None:
                    acc += prod(0, t) * (Cm[b, t, h, :] @ h0[b, h])
                if Dskip is not None:
                    acc += Dskip[h] * x[b, t, h, :]
                y[b, t, h] = acc
            st = np.zeros((N, D), dtype=np.complex128)
            for s in range(T):
                st += prod(s + 1, T - 1) * np.outer(Bm[b, s, h], x[b, s, h])
            if h0 is not None:
                st += prod(0, T - 1) * h0[b, h]
            hT[b, h] = st
    return y, hT


def _rand_problem(rng, Bsz, T, H, D, N, with_h0=True, with_d=True):
    x = crandn(rng, Bsz, T, H, D)
    Bm = crandn(rng, Bsz, T, H, N)
    Cm = crandn(rng, Bsz, T, H, N)
    dt = rng.standard_normal((Bsz, T, H))
    A = -rng.uniform(0.1, 1.0, H) + 1j * rng.uniform(-math.pi, math.pi, H)
    Dk = rng.standard_normal(H) if with_d else None
    h0 = crandn(rng, Bsz, H, N, D) if with_h0 else None
    return x, Bm, Cm, dt, A, Dk, h0


def pin_bruteforce(lib):
    rng = np.random.default_rng(101)
    for (Bsz, T, H, D, N) in [(1, 1, 1, 1, 1), (2, 3, 2, 3, 2), (1, 5, 3, 2, 4), (2, 8, 2, 3, 5)]:
        for with_h0 in (False, True):
            prob = _rand_problem(rng, Bsz, T, H, D, N, with_h0=with_h0)
            y, hT = oracle.forward(*prob, lib=lib)
            yb, hb = bruteforce(*prob)
            assert rel_err(y, yb) < 1e-12, ("y", Bsz, T, H, D, N, with_h0, rel_err(y, yb))
            assert rel_err(hT, hb) < 1e-12, ("hT", Bsz, T, H, D, N, with_h0, rel_err(hT, hb))


# ---------------------------------------------------------------------------
# p2: impulse enumeration of the segment matrix
# ---------------------------------------------------------------------------
def pin_impulse(lib):
    """x one-hot at (s, p), B_t = C_t = e_n for all t, no skip, zero state:
    y_t[q] = exp(sum_{u=s+1}^{t} softplus(dt_u) A) if t >= s and q = p, else 0
    (Mamba-3-Lite docs, "SSD Theory" 4.3: the causal segment matrix with an
    inclusive diagonal of exactly 1).  Every (s, p) runs as one batch row."""
    rng = np.random.default_rng(202)
    T, D, N, n_hot = 7, 3, 2, 1
    A = np.array([-0.4 + 1.3j])
    dt_row = rng.standard_normal(T)
    Bsz = T * D
    x = np.zeros((Bsz, T, 1, D), dtype=np.complex128)
    for s in range(T):
        for p in range(D):
            x[s * D + p, s, 0, p] = 1.0
    Bm = np.zeros((Bsz, T, 1, N), dtype=np.complex128); Bm[..., n_hot] = 1.0
    Cm = Bm.copy()
    dt = np.broadcast_to(dt_row[None, :, None], (Bsz, T, 1)).copy()
    y, _ = oracle.forward(x, Bm, Cm, dt, A, None, None, lib=lib)
    logdec = np.logaddexp(0.0, dt_row) * A[0]
    for s in range(T):
        for p in range(D):
            got = y[s * D + p, :, 0, :]
            want = np.zeros((T, D), dtype=np.complex128)
            for t in range(s, T):
                want[t, p] = np.exp(np.sum(logdec[s + 1:t + 1]))
            assert np.max(np.abs(got - want)) < 1e-13, (s, p)


# ---------------------------------------------------------------------------
# p4/p5: constant input -- geometric series and its fixed point
# ---------------------------------------------------------------------------
def constant_closed_form(n, a, Bv, xv, Cv, d, h0):
    """State and output after n identical steps (burn-mamba step_constant: the
    n-step geometric series, here with no rotation operator, beta = 0, gamma = 1):
    h_n = a^n h0 + (1 - a^n)/(1 - a) B (x) x ;  y_n = C . h_n + d x."""
    an = np.exp(n * np.log(a))
    hn = an * h0 + (1.0 - an) / (1.0 - a) * np.outer(Bv, xv)
    return Cv @ hn + d * xv, hn


def _const_problem(rng, T, D, N, dt0, A0):
    Bv, Cv, xv = crandn(rng, N), crandn(rng, N), crandn(rng, D)
    h0 = crandn(rng, 1, 1, N, D)
    x = np.broadcast_to(xv, (1, T, 1, D)).copy()
    Bm = np.broadcast_to(Bv, (1, T, 1, N)).copy()
    Cm = np.broadcast_to(Cv, (1, T, 1, N)).copy()
    dt = np.full((1, T, 1), dt0)
    return x, Bm, Cm, dt, np.array([A0]), np.array([0.7]), h0, Bv, Cv, xv


def pin_constant_input(lib):
    rng = np.random.default_rng(303)
    T, D, N = 600, 3, 2
    x, Bm, Cm, dt, A, Dk, h0, Bv, Cv, xv = _const_problem(rng, T, D, N, 0.3, -0.05 + 2.1j)
    y, hT = oracle.forward(x, Bm, Cm, dt, A, Dk, h0, lib=lib)
    a = complex(disc(0.3, A[0]))
    for n in (1, 2, 3, 17, 256, T):
        yn, hn = constant_closed_form(n, a, Bv, xv, Cv, Dk[0], h0[0, 0])
        assert rel_err(y[0, n - 1, 0], yn) < 1e-10, ("y", n, rel_err(y[0, n - 1, 0], yn))
    _, hn = constant_closed_form(T, a, Bv, xv, Cv, Dk[0], h0[0, 0])
    assert rel_err(hT[0, 0], hn) < 1e-10


def pin_fixed_point(lib):
    """n -> infinity: y_inf = (C . B) x / (1 - a) + d x, independent of h0."""
    rng = np.random.default_rng(404)
    T, D, N = 4096, 2, 3
    x, Bm, Cm, dt, A, Dk, h0, Bv, Cv, xv = _const_problem(rng, T, D, N, -0.2, -0.06 - 0.8j)
    y, _ = oracle.forward(x, Bm, Cm, dt, A, Dk, h0, lib=lib)
    a = complex(disc(-0.2, A[0]))
    assert abs(a) ** T < 1e-20
    yinf = (Cv @ Bv) * xv / (1.0 - a) + Dk[0] * xv
    assert rel_err(y[0, -1, 0], yinf) < 1e-10


def pin_step_constant_input(lib):
    """The single-step entry point, iterated, against the same geometric series."""
    rng = np.random.default_rng(505)
    Bsz, H, D, N, n = 2, 2, 3, 2, 150
    Bv, Cv, xv = crandn(rng, Bsz, H, N), crandn(rng, Bsz, H, N), crandn(rng, Bsz, H, D)
    dt = rng.standard_normal((Bsz, H))
    A = np.array([-0.3 + 0.9j, -0.05 - 2.0j])
    Dk = np.array([0.4, -1.1])
    h = crandn(rng, Bsz, H, N, D)
    h_init = h.copy()
    for _ in range(n):
        y, h = oracle.step(xv, Bv, Cv, dt, A, Dk, h, lib=lib)
    for b in range(Bsz):
        for k in range(H):
            a = complex(disc(dt[b, k], A[k]))
            yn, hn = constant_closed_form(n, a, Bv[b, k], xv[b, k], Cv[b, k], Dk[k], h_init[b, k])
            assert rel_err(y[b, k], yn) < 1e-10, (b, k)
            assert rel_err(h[b, k], hn) < 1e-10, (b, k)


def pin_step_n_against_recurrence(lib):
    """The closed-form n-step entry point is the state and output after n calls
    of the one-step recurrence with the same input (burn-mamba step_constant).
    The heads cover |a| < 1, a pure rotation (|a| = 1, a != 1), a = 1 exactly
    (A = 0: h_n = h0 + n B (x) x) and a vanishing decay (h_n -> B (x) x)."""
    rng = np.random.default_rng(707)
    Bsz, H, D, N = 2, 4, 3, 5
    xv, Bv, Cv = crandn(rng, Bsz, H, D), crandn(rng, Bsz, H, N), crandn(rng, Bsz, H, N)
    dt = rng.uniform(-1.0, 1.0, (Bsz, H))
    A = np.array([-0.4 + 1.3j, 0.0 + 0.7j, 0.0 + 0.0j, -1e4 + 0.3j])
    Dk = np.array([0.5, -0.8, 1.2, 0.3])
    h0 = crandn(rng, Bsz, H, N, D)
    for n in (1, 2, 7, 40):
        h = h0.copy()
        for _ in range(n):
            y, h = oracle.step(xv, Bv, Cv, dt, A, Dk, h, lib=lib)
        yn, hn = oracle.step_n(xv, Bv, Cv, dt, A, Dk, h0, n, lib=lib)
        assert rel_err(hn, h) < 1e-12, ("h", n, rel_err(hn, h))
        assert rel_err(yn, y) < 1e-12, ("y", n, rel_err(yn, y))
    _, hn = oracle.step_n(xv, Bv, Cv, dt, A, Dk, h0, 9, lib=lib)
    outer = np.einsum("bhn,bhd->bhnd", Bv, xv)
    assert rel_err(hn[:, 2], h0[:, 2] + 9 * outer[:, 2]) < 1e-14   # a = 1
    assert rel_err(hn[:, 3], outer[:, 3]) < 1e-14                   # a -> 0


def pin_step_infinite_against_recurrence(lib):
    """The stationary output is what the recurrence settles to under an endless
    constant input, whatever the start state: iterate until |a|^n < 1e-18.  With a
    vanishing decay it is (C . B) x + D x."""
    rng = np.random.default_rng(808)
    Bsz, H, D, N = 2, 3, 4, 3
    xv, Bv, Cv = crandn(rng, Bsz, H, D), crandn(rng, Bsz, H, N), crandn(rng, Bsz, H, N)
    dt = rng.uniform(-1.0, 1.0, (Bsz, H))
    A = np.array([-0.5 + 2.0j, -0.2 - 0.6j, -1e4 + 1.0j])
    Dk = np.array([0.9, -0.4, 1.7])
    h = crandn(rng, Bsz, H, N, D)
    amax = float(np.max(np.abs(disc(dt, A[None, :]))))
    n = int(np.ceil(np.log(1e-18) / np.log(amax)))
    for _ in range(n):
        y, h = oracle.step(xv, Bv, Cv, dt, A, Dk, h, lib=lib)
    yinf = oracle.step_infinite(xv, Bv, Cv, dt, A, Dk, lib=lib)
    assert rel_err(yinf, y) < 1e-12, rel_err(yinf, y)
    score = np.einsum("bhn,bhn->bh", Cv, Bv)
    assert rel_err(yinf[:, 2], (score[:, 2, None] + Dk[2]) * xv[:, 2]) < 1e-14


# ---------------------------------------------------------------------------
# f1: gradients -- central finite differences of the forward oracle
# ---------------------------------------------------------------------------
def _fd_loss(lib, args, gy, ghT):
    """L = <dy, y> + <dhT, hT>, the real inner product of the re/im planes."""
    y, hT = oracle.forward(*args, lib=lib)
    return float(np.sum(gy.real * y.real + gy.imag * y.imag)
                 + np.sum(ghT.real * hT.real + ghT.imag * hT.imag))


def pin_backward_finite_differences(lib):
    """Every gradient entry of a small problem against a central difference of the
    forward oracle's loss (step 1e-6 in fp64): dt, A, Dskip and every re / im
    element of x, B, C and h0.  Independent of the reverse-mode code: it only
    calls the forward recurrence."""
    rng = np.random.default_rng(909)
    Bsz, T, H, D, N = 2, 5, 2, 3, 2
    x, Bm, Cm, dt, A, Dk, h0 = _rand_problem(rng, Bsz, T, H, D, N)
    gy, ghT = crandn(rng, Bsz, T, H, D), crandn(rng, Bsz, H, N, D)
    g = oracle.backward(x, Bm, Cm, dt, A, Dk, h0, gy, ghT, lib=lib)
    base = {"x": x, "Bm": Bm, "Cm": Cm, "dt": dt, "A": A, "Dk": Dk, "h0": h0}
    order = ("x", "Bm", "Cm", "dt", "A", "Dk", "h0")
    want = {"x": g["dx"], "Bm": g["dB"], "Cm": g["dC"], "dt": g["ddt"], "A": g["dA"],
            "Dk": g["dD"], "h0": g["dh0"]}
    eps = 1e-6
    for name in order:
        v = base[name]
        parts = (1.0, 1j) if np.iscomplexobj(v) else (1.0,)
        fd = np.zeros(v.shape, dtype=np.complex128)
        for idx in np.ndindex(v.shape):
            for unit in parts:
                vals = []
                for sign in (1.0, -1.0):
                    w = v.copy()
                    w[idx] += sign * eps * unit
                    args = tuple(w if k == name else base[k] for k in order)
                    vals.append(_fd_loss(lib, args, gy, ghT))
                fd[idx] += (vals[0] - vals[1]) / (2 * eps) * (1.0 if unit == 1.0 else 1j)
        got = want[name]
        err = float(np.max(np.abs(fd - got)) / max(np.max(np.abs(fd)), 1e-30))
        assert err < 1e-7, (name, err)


def pin_backward_without_initial_state(lib):
    """With no initial state and no final-state gradient, the same check on the
    inputs that remain (the oracle's NULL paths); B = C = 0 leaves only the skip:
    dx = D dy."""
    rng = np.random.default_rng(910)
    Bsz, T, H, D, N = 1, 4, 2, 2, 3
    x, Bm, Cm, dt, A, Dk, _ = _rand_problem(rng, Bsz, T, H, D, N, with_h0=False)
    gy = crandn(rng, Bsz, T, H, D)
    zero_hT = np.zeros((Bsz, H, N, D), dtype=np.complex128)
    g = oracle.backward(x, Bm, Cm, dt, A, Dk, None, gy, None, lib=lib)
    eps = 1e-6
    for k in np.ndindex(dt.shape):
        w = dt.copy(); w[k] += eps
        lp = _fd_loss(lib, (x, Bm, Cm, w, A, Dk, None), gy, zero_hT)
        w[k] -= 2 * eps
        lm = _fd_loss(lib, (x, Bm, Cm, w, A, Dk, None), gy, zero_hT)
        assert abs((lp - lm) / (2 * eps) - g["ddt"][k]) < 1e-7 * max(1.0, np.max(np.abs(g["ddt"])))
    zB = np.zeros_like(Bm)
    g0 = oracle.backward(x, zB, zB, dt, A, Dk, None, gy, None, lib=lib)
    assert rel_err(g0["dx"], Dk[None, None, :, None] * gy) < 1e-15
    assert np.max(np.abs(g0["dB"])) == 0 and np.max(np.abs(g0["ddt"])) == 0


# ---------------------------------------------------------------------------
# p6: decay zero -- the scan reduces to per-step outer products
# ---------------------------------------------------------------------------
def pin_decay_zero(lib):
    rng = np.random.default_rng(606)
    Bsz, T, H, D, N = 2, 9, 2, 3, 4
    x, Bm, Cm, _, _, Dk, h0 = _rand_problem(rng, Bsz, T, H, D, N)
    A = np.array([-1e4 + 0.5j, -1e4 - 2.0j])
    dt = np.zeros((Bsz, T, H))
    assert np.all(disc(0.0, A) == 0)
    y, hT = oracle.forward(x, Bm, Cm, dt, A, Dk, h0, lib=lib)
    score = np.einsum("bthn,bthn->bth", Cm, Bm)
    want = score[..., None] * x + Dk[None, None, :, None] * x
    assert rel_err(y, want) < 1e-13
    want_h = np.einsum("bhn,bhd->bhnd", Bm[:, -1], x[:, -1])
    assert rel_err(hT, want_h) < 1e-13


# ---------------------------------------------------------------------------
# p7: homogeneous recurrence -- exact transport of phase (Lemma 6.2)
# ---------------------------------------------------------------------------
def pin_homogeneous(lib):
    """x = 0, h0 != 0: h_T = (prod a_u) h0, so |h_T| = |h0| prod |a_u| and
    arg h_T = arg h0 + sum_u s_u Im A (mod 2 pi) ("Complex Phase-State Dynamics
    Reduce the Optimization Steps of Sequence Models", Lemma 6.2 / eq. 7,
    specialised to one coordinate); y_t = (prod_{u<=t} a_u) C_t . h0."""
    rng = np.random.default_rng(707)
    T, D, N = 4096, 2, 2
    A = np.array([-0.002 + 2.7j])
    dt = rng.standard_normal((1, T, 1)) * 0.5 - 1.0
    h0 = crandn(rng, 1, 1, N, D)
    Cm = crandn(rng, 1, T, 1, N)
    x = np.zeros((1, T, 1, D), dtype=np.complex128)
    Bm = crandn(rng, 1, T, 1, N)
    y, hT = oracle.forward(x, Bm, Cm, dt, A, None, h0, lib=lib)
    s = np.logaddexp(0.0, dt[0, :, 0])
    log_mag = math.fsum(s * A[0].real)
    phase = math.fsum(s * A[0].imag)
    got = hT[0, 0] / h0[0, 0]
    assert np.max(np.abs(np.log(np.abs(got)) - log_mag)) < 1e-9
    dphi = np.angle(got * np.exp(-1j * phase))
    assert np.max(np.abs(dphi)) < 1e-8
    cum = np.cumsum(s * A[0])
    for t in (0, 1, 100, T - 1):
        want = np.exp(cum[t]) * (Cm[0, t, 0] @ h0[0, 0])
        assert rel_err(y[0, t, 0], want) < 1e-8, t


# ---------------------------------------------------------------------------
# p9: linearity and the skip term
# ---------------------------------------------------------------------------
def pin_linearity_and_skip(lib):
    rng = np.random.default_rng(909)
    Bsz, T, H, D, N = 2, 12, 3, 4, 3
    x1, Bm, Cm, dt, A, Dk, _ = _rand_problem(rng, Bsz, T, H, D, N, with_h0=False)
    x2 = crandn(rng, Bsz, T, H, D)
    al, be = 0.3 - 1.2j, -0.7 + 0.4j
    y1, _ = oracle.forward(x1, Bm, Cm, dt, A, Dk, None, lib=lib)
    y2, _ = oracle.forward(x2, Bm, Cm, dt, A, Dk, None, lib=lib)
    y12, _ = oracle.forward(al * x1 + be * x2, Bm, Cm, dt, A, Dk, None, lib=lib)
    assert rel_err(y12, al * y1 + be * y2) < 1e-12
    y0, h0 = oracle.forward(x1, np.zeros_like(Bm), Cm, dt, A, Dk, None, lib=lib)
    assert np.array_equal(y0, Dk[None, None, :, None] * x1)
    assert np.all(h0 == 0)


# ---------------------------------------------------------------------------
# p10: PAM -- quadratic dual form and lossless retrieval with orthogonal keys
# ---------------------------------------------------------------------------
def pam_dual(K, Q, V, gamma, score):
    """Phase-Associative Memory eq. 7 evaluated in the page's O(T^2) dual form:
    decay matrix D[t,i] = gamma^(t-i) for i <= t (0 above the diagonal), score
    W = Q~ K^*T with Q~ = Q/sqrt(d), output Y = (W * D) V.  score="re" keeps
    Re(W) (the configuration's Re<K|Q>/sqrt(d) readout)."""
    Bsz, T, H, d = K.shape
    Y = np.zeros_like(V)
    t_idx = np.arange(T)
    expo = (t_idx[:, None] - t_idx[None, :]).astype(np.float64)
    for b in range(Bsz):
        for h in range(H):
            Dm = np.where(expo >= 0, gamma[h] ** np.maximum(expo, 0), 0.0)
            W = (Q[b, :, h, :] / math.sqrt(d)) @ np.conj(K[b, :, h, :]).T
            if score == "re":
                W = W.real
            Y[b, :, h, :] = (W * Dm) @ V[b, :, h, :]
    return Y


def pin_pam_dual_form(lib):
    import cssd_workloads as wl
    p = wl.pam_draw(77, 2, 40, 2, 8)
    for score in ("complex", "re"):
        inp = wl.pam_to_scan(p, chunk=16, score=score)
        x, Bm, Cm, dt, A, Dk, h0 = inp.complex()
        y, _ = oracle.forward(x, Bm, Cm, dt, A, Dk, h0, lib=lib)
        # the scan runs on fp32-rounded inputs; the dual form on the exact draws
        want = pam_dual(p.K, p.Q, p.V, p.gamma.astype(np.float32).astype(np.float64), score)
        assert rel_err(y, want) < 2e-6, (score, rel_err(y, want))


def pin_pam_orthogonal_keys(lib):
    """Orthonormal unit-phase keys (DFT rows / sqrt(d)), gamma = 1, queries
    Q_t = sqrt(d) K_{j(t)} with j(t) <= t: retrieval returns V_{j(t)} exactly
    (Phase-Associative Memory, the lossless-retrieval statement after eq. 7)."""
    import cssd_workloads as wl
    rng = np.random.default_rng(1010)
    d = T = 8
    k = np.arange(d)
    K = np.exp(2j * np.pi * np.outer(np.arange(T), k) / d) / math.sqrt(d)
    j = np.array([rng.integers(0, t + 1) for t in range(T)])
    Q = math.sqrt(d) * K[j]
    V = crandn(rng, T, d)
    p = wl.PamInputs(K[None, :, None, :], Q[None, :, None, :], V[None, :, None, :], np.array([1.0]))
    for score in ("complex", "re"):
        N = d if score == "complex" else 2 * d
        rs = 1.0 / math.sqrt(d)
        if score == "complex":
            Bm, Cm = np.conj(p.K), p.Q * rs
        else:
            Bm = np.concatenate([np.conj(p.K), p.K], -1)
            Cm = np.concatenate([p.Q, np.conj(p.Q)], -1) * (0.5 * rs)
        assert Bm.shape[-1] == N
        y, _ = oracle.forward(p.V, Bm, Cm, np.zeros((1, T, 1)), np.array([0.0 + 0.0j]), None, None,
                              lib=lib)
        assert np.max(np.abs(y[0, :, 0, :] - V[j])) < 1e-12, score


# ---------------------------------------------------------------------------
# golden values printed on the pages
# ---------------------------------------------------------------------------
def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pin_golden_modulus_drift(lib):
    """|h_T| / |h_0| after T homogeneous steps of modulus rho, rounded as printed."""
    g = _golden("modulus_drift.json")

    def drift(rho, T):
        # |a| = rho with dt = 0 (softplus(0) = ln 2): Re A = ln(rho) / ln 2
        A = np.array([math.log(rho) / math.log(2.0) + 0.37j])
        h0 = np.ones((1, 1, 1, 1), dtype=np.complex128)
        z = np.zeros((1, T, 1, 1), dtype=np.complex128)
        _, hT = oracle.forward(z, z, z, np.zeros((1, T, 1)), A, None, h0, lib=lib)
        return abs(hT[0, 0, 0, 0])

    for case in g["cases"]:
        got = drift(case["rho"], case["steps"])
        sig = case["printed_significant_digits"]
        assert float(f"{got:.{sig}g}") == case["printed"], (case, got)
    for case in g["bounds"]:
        got = drift(case["rho"], case["steps"])
        assert got < case["upper"], (case, got)


# ---------------------------------------------------------------------------
# f3: the per-coordinate phase-state scan (phase-state paper, section 5.2)
# ---------------------------------------------------------------------------
def _phase_coeff(phi, u):
    """a = sigmoid(u) exp(2i atan(phi)): the Cayley phase through its angle (the
    page's arg formula) and the gate through logaddexp -- a different route from
    the oracle's complex division."""
    return np.exp(-np.logaddexp(0.0, -np.asarray(u))) * np.exp(2j * np.arctan(phi))


def pin_phase_unrolled(lib):
    """psi_T = (prod_t a_t) psi_0 + sum_r (prod_{j>r} a_j) b_r for every prefix,
    products formed explicitly (section 5.3, eq. 4 unrolled)."""
    rng = np.random.default_rng(1111)
    Bsz, T, H, N = 2, 7, 2, 3
    phi = 2.0 * rng.standard_normal((Bsz, T, H, N))
    u = 2.0 * rng.standard_normal((Bsz, T, H, N))
    b = crandn(rng, Bsz, T, H, N)
    psi0 = crandn(rng, Bsz, H, N)
    psi, psiT = oracle.phase_scan(phi, u, b, psi0, lib=lib)
    a = _phase_coeff(phi, u)
    for t in range(T):
        want = psi0.copy()
        for j in range(t + 1):
            want = want * a[:, j]
        for r in range(t + 1):
            term = b[:, r].copy()
            for j in range(r + 1, t + 1):
                term = term * a[:, j]
            want = want + term
        assert rel_err(psi[:, t], want) < 1e-13, (t, rel_err(psi[:, t], want))
    assert rel_err(psiT, psi[:, -1]) == 0.0


def pin_phase_transport(lib):
    """Without input the phase is carried exactly (the paper's Lemma 6.2): |psi_T| =
    |psi_0| prod alpha_t and arg psi_T = arg psi_0 + sum 2 atan(phi_t) mod 2 pi; with
    the gate fully open the modulus stays |psi_0| over 4096 steps (exact unit
    modulus of the Cayley transform)."""
    rng = np.random.default_rng(1212)
    Bsz, T, H, N = 1, 1024, 2, 4
    phi = 3.0 * rng.standard_normal((Bsz, T, H, N))
    u = 4.0 + rng.standard_normal((Bsz, T, H, N))
    psi0 = crandn(rng, Bsz, H, N)
    zero = np.zeros((Bsz, T, H, N), dtype=np.complex128)
    _, psiT = oracle.phase_scan(phi, u, zero, psi0, lib=lib)
    alpha = np.exp(-np.logaddexp(0.0, -u))
    mod = np.abs(psi0) * np.prod(alpha, axis=1)
    assert np.max(np.abs(np.abs(psiT) - mod) / mod) < 1e-12
    ang = np.angle(psi0) + np.sum(2.0 * np.arctan(phi), axis=1)
    dang = np.angle(psiT * np.exp(-1j * ang))
    assert np.max(np.abs(dang)) < 1e-9
    T2 = 4096
    phi2 = rng.standard_normal((1, T2, 1, 2))
    _, psiT2 = oracle.phase_scan(phi2, np.full((1, T2, 1, 2), 60.0),
                                 np.zeros((1, T2, 1, 2), dtype=np.complex128),
                                 np.ones((1, 1, 2), dtype=np.complex128), lib=lib)
    assert np.max(np.abs(np.abs(psiT2) - 1.0)) < 1e-12


def pin_phase_golden_gain(lib):
    """The page's printed gain of a per-coordinate factor 0.99 over 1024 steps
    (3.4e-5), reached by the scan with gate 0.99 and no rotation."""
    g = _golden("modulus_drift.json")
    for case in g["cases"] + g["bounds"]:
        rho, T = case["rho"], case["steps"]
        u = np.full((1, T, 1, 1), math.log(rho / (1.0 - rho)))
        _, psiT = oracle.phase_scan(np.zeros((1, T, 1, 1)), u,
                                    np.zeros((1, T, 1, 1), dtype=np.complex128),
                                    np.ones((1, 1, 1), dtype=np.complex128), lib=lib)
        got = abs(psiT[0, 0, 0])
        if "printed" in case:
            sig = case["printed_significant_digits"]
            assert float(f"{got:.{sig}g}") == case["printed"], (case, got)
        else:
            assert got < case["upper"], (case, got)


# ---------------------------------------------------------------------------
# f4: causal Born attention (phase-state paper, section 5.5 eq. 5, Algorithm 3)
# ---------------------------------------------------------------------------
def _dft_keys(D):
    """Orthonormal keys with unit-modulus phases: row j of the D-point DFT / sqrt(D)."""
    n = np.arange(D)
    return np.exp(2j * np.pi * np.outer(n, n) / D) / math.sqrt(D)


def pin_born_orthogonal_keys(lib):
    """With orthonormal keys and each query a multiple of one earlier key, the
    Born score is nonzero only for that key, so the output is exactly that key's
    value (lossless retrieval).  Keys are DFT rows, whose complex phases differ
    coordinate by coordinate, so an overlap taken without the conjugate fails."""
    rng = np.random.default_rng(2121)
    for D in (8, 16):
        T, H, Bsz = D, 2, 2
        K = _dft_keys(D)
        k = np.broadcast_to(K[None, :, None, :], (Bsz, T, H, D)).copy()
        v = crandn(rng, Bsz, T, H, D)
        pick = np.array([[[rng.integers(0, i + 1) for _ in range(H)] for i in range(T)]
                         for _ in range(Bsz)])
        c = crandn(rng, Bsz, T, H) * 3.0
        q = c[..., None] * K[pick]
        tau = 0.5 + rng.random((Bsz, T, H))
        out = oracle.born_attention(q, k, v, tau, lib=lib)
        want = np.take_along_axis(v, pick[..., None], axis=1)
        assert np.max(np.abs(out - want)) < 1e-12, np.max(np.abs(out - want))


def pin_born_two_state_interference(lib):
    """The page's two-state computation (section 5.5): for a key
    (phi_1 + e^{i theta} phi_2)/sqrt 2 and the query (phi_1 + phi_2)/sqrt 2 the Born
    weight is (1 + cos theta)/2, falling to 0 at theta = pi; a second key phi_1 has
    weight 1/2.  So psi_1 = (p(theta) v_0 + v_1 / 2) / (p(theta) + 1/2), and the
    first key is extinguished by phase opposition at theta = pi."""
    D = 4
    phi1, phi2 = np.eye(D)[0].astype(complex), np.eye(D)[1].astype(complex)
    v = np.zeros((1, 2, 1, D), dtype=complex)
    v[0, 0, 0] = [1.0, 2.0j, -1.0, 0.5]
    v[0, 1, 0] = [0.0, 1.0, 1.0j, -2.0]
    for theta in np.linspace(0.0, math.pi, 9):
        k = np.zeros((1, 2, 1, D), dtype=complex)
        k[0, 0, 0] = (phi1 + np.exp(1j * theta) * phi2) / math.sqrt(2)
        k[0, 1, 0] = phi1
        q = np.zeros_like(k)
        q[0, 0, 0] = phi1
        q[0, 1, 0] = (phi1 + phi2) / math.sqrt(2)
        out = oracle.born_attention(q, k, v, None, lib=lib)
        p = 0.5 * (1.0 + math.cos(theta))
        want = (p * v[0, 0, 0] + 0.5 * v[0, 1, 0]) / (p + 0.5)
        assert np.max(np.abs(out[0, 1, 0] - want)) < 1e-14, (theta, out[0, 1, 0], want)
    assert np.max(np.abs(out[0, 1, 0] - v[0, 1, 0])) < 1e-14   # theta = pi
    assert np.max(np.abs(out[0, 0, 0] - v[0, 0, 0])) < 1e-14   # the first row sees only itself


def pin_born_density_matrix_form(lib):
    """Brute force through the density-matrix form the page gives for the Born
    score (section 5.5: the score is tr(M rho), linear in rho = |q><q|, here with
    M = |k><k|): tiny problems with the score formed as a trace of a matrix
    product and the causal normalisation written as explicit loops."""
    rng = np.random.default_rng(2222)
    Bsz, T, H, D = 2, 6, 2, 3
    q, k, v = crandn(rng, Bsz, T, H, D), crandn(rng, Bsz, T, H, D), crandn(rng, Bsz, T, H, D)
    tau = 0.3 + rng.random((Bsz, T, H))
    out = oracle.born_attention(q, k, v, tau, lib=lib)
    for b in range(Bsz):
        for h in range(H):
            for i in range(T):
                rho = np.outer(q[b, i, h], np.conj(q[b, i, h]))
                num = np.zeros(D, dtype=complex)
                den = 0.0
                for j in range(i + 1):
                    M = np.outer(k[b, j, h], np.conj(k[b, j, h]))
                    sij = np.trace(M @ rho).real / (D * tau[b, i, h])
                    num += sij * v[b, j, h]
                    den += sij
                assert np.max(np.abs(out[b, i, h] - num / den)) < 1e-13


def pin_born_invariances(lib):
    """Properties of eq. 5 at a random size: the temperature and the factor D cancel
    in the normalisation (rescaling tau per row changes nothing); a global phase on
    any query or key changes no squared modulus; row i ignores keys and values after
    i; equal values are returned unchanged; the first row returns its own value."""
    rng = np.random.default_rng(2323)
    Bsz, T, H, D = 2, 40, 3, 8
    q, k, v = crandn(rng, Bsz, T, H, D), crandn(rng, Bsz, T, H, D), crandn(rng, Bsz, T, H, D)
    tau = 0.5 + rng.random((Bsz, T, H))
    base = oracle.born_attention(q, k, v, tau, lib=lib)
    scaled = oracle.born_attention(q, k, v, tau * np.exp(3.0 * rng.standard_normal(tau.shape)),
                                   lib=lib)
    assert np.max(np.abs(scaled - base)) < 1e-12
    ph = lambda *s: np.exp(1j * rng.uniform(-math.pi, math.pi, s))
    rot = oracle.born_attention(q * ph(Bsz, T, H, 1), k * ph(Bsz, T, H, 1), v, tau, lib=lib)
    assert np.max(np.abs(rot - base)) < 1e-12
    i0 = 17
    k2, v2 = k.copy(), v.copy()
    k2[:, i0 + 1:] = crandn(rng, Bsz, T - i0 - 1, H, D)
    v2[:, i0 + 1:] = crandn(rng, Bsz, T - i0 - 1, H, D)
    causal = oracle.born_attention(q, k2, v2, tau, lib=lib)
    assert np.array_equal(causal[:, :i0 + 1], base[:, :i0 + 1])
    assert np.max(np.abs(causal[:, i0 + 1:] - base[:, i0 + 1:])) > 1e-3
    same = np.broadcast_to(crandn(rng, Bsz, 1, H, D), (Bsz, T, H, D))
    const = oracle.born_attention(q, k, same, tau, lib=lib)
    assert np.max(np.abs(const - same)) < 1e-13
    assert np.max(np.abs(base[:, 0] - v[:, 0])) < 1e-14



def pin_born_rows_match_full(lib):
    """The sampled-row form of Born attention returns, for each listed (b, i, h),
    exactly the row the full evaluation of eq. 5 gives there (the phase-state
    paper, section 5.5): each row's output depends only on that query and the
    keys and values up to it, so selecting rows after or before the evaluation
    must agree bit for bit.  Rows are random (b, i, h) triples with b, i and h
    drawn from ranges of different lengths, so that a decode that swaps any two
    of them reads the wrong row or leaves the problem; the first and last rows
    and repeated rows are included, in an order unrelated to memory order.  Both
    the complex and the (re, im) plane forms of the inputs are checked."""
    rng = np.random.default_rng(2424)
    Bsz, T, H, D = 3, 29, 5, 4
    q, k, v = crandn(rng, Bsz, T, H, D), crandn(rng, Bsz, T, H, D), crandn(rng, Bsz, T, H, D)
    tau = 0.5 + rng.random((Bsz, T, H))
    full = oracle.born_attention(q, k, v, tau, lib=lib)
    rows = np.stack([rng.integers(0, Bsz, 40), rng.integers(0, T, 40), rng.integers(0, H, 40)], 1)
    rows = np.concatenate([[[0, 0, 0], [Bsz - 1, T - 1, H - 1], [Bsz - 1, 0, H - 1],
                            [0, T - 1, 0]], rows, rows[:3]])
    want = full[rows[:, 0], rows[:, 1], rows[:, 2]]
    pl = lambda z: (z.real.copy(), z.imag.copy())
    for args in ((q, k, v), (pl(q), pl(k), pl(v))):
        try:
            got = oracle.born_attention_rows(*args, tau, rows, lib=lib)
        except RuntimeError as e:  # a decode that leaves the problem is a failure of the pin
            raise AssertionError(f"born_attention_rows rejected valid rows: {e}")
        assert got.shape == want.shape and np.array_equal(got, want), rel_err(got, want)
    # without a temperature: tau = 1 on every row
    full1 = oracle.born_attention(q, k, v, None, lib=lib)
    got1 = oracle.born_attention_rows(q, k, v, None, rows, lib=lib)
    assert np.array_equal(got1, full1[rows[:, 0], rows[:, 1], rows[:, 2]])

# ---------------------------------------------------------------------------
# empty sequences: a scan of no time steps
# ---------------------------------------------------------------------------
def pin_empty_sequence(lib):
    """With T = 0 the recurrence is never applied (Mamba-3-Lite docs, "Complex-Valued
    State Spaces", the naive scan): the final state is the initial one (zero
    without one), the gradient reaching h0 is the one given for hT, and the sums
    over time, dA and dDskip, are empty.  The phase scan keeps psi0 and Born
    attention has no rows."""
    rng = np.random.default_rng(77)
    Bsz, H, D, N = 2, 3, 4, 5
    x, Bm, Cm, dt, A, Dk, h0 = _rand_problem(rng, Bsz, 0, H, D, N)
    y, hT = oracle.forward(x, Bm, Cm, dt, A, Dk, h0, lib=lib)
    assert y.shape == (Bsz, 0, H, D) and np.array_equal(hT, h0)
    _, hz = oracle.forward(x, Bm, Cm, dt, A, Dk, None, lib=lib)
    assert hz.shape == (Bsz, H, N, D) and not np.any(hz)
    dhT = crandn(rng, Bsz, H, N, D)
    g = oracle.backward(x, Bm, Cm, dt, A, Dk, h0, np.zeros((Bsz, 0, H, D), complex), dhT, lib=lib)
    assert np.array_equal(g["dh0"], dhT)
    assert not np.any(g["dA"]) and not np.any(g["dD"])
    assert g["dx"].shape == (Bsz, 0, H, D) and g["ddt"].shape == (Bsz, 0, H)
    psi0 = crandn(rng, Bsz, H, N)
    z = np.zeros((Bsz, 0, H, N))
    psi, psiT = oracle.phase_scan(z, z, z.astype(complex), psi0, lib=lib)
    assert psi.shape == (Bsz, 0, H, N) and np.array_equal(psiT, psi0)
    e = np.zeros((Bsz, 0, H, D), complex)
    assert oracle.born_attention(e, e, e, lib=lib).shape == (Bsz, 0, H, D)


ALL_PINS = [pin_bruteforce, pin_empty_sequence, pin_impulse, pin_constant_input, pin_fixed_point,
            pin_phase_unrolled, pin_phase_transport, pin_phase_golden_gain,
            pin_born_orthogonal_keys, pin_born_two_state_interference,
            pin_born_density_matrix_form, pin_born_invariances, pin_born_rows_match_full,
            pin_step_n_against_recurrence, pin_step_infinite_against_recurrence,
            pin_backward_finite_differences, pin_backward_without_initial_state,
            pin_step_constant_input, pin_decay_zero, pin_homogeneous, pin_linearity_and_skip,
            pin_pam_dual_form, pin_pam_orthogonal_keys, pin_golden_modulus_drift]
