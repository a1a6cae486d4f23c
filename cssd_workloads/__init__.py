"""Seeded synthetic inputs for the complex diagonal state-space scan.

This module is shared by the GPU path's tests and benchmark and by the oracle's
callers.  It holds none of the scan's arithmetic: only random draws, casts to
the storage precision, and the input recipes of the workloads (distributions,
shapes, and the re-parameterisations that turn a recipe's target quantity into
the raw inputs the scan reads).

Recipe conventions
------------------
* Every tensor is drawn from its own stream
  ``numpy.random.default_rng(SeedSequence([seed, k]))`` where ``k`` is the
  tensor's index in ``TENSORS``; per-step decode inputs use
  ``SeedSequence([seed, step, k])``.
* Draws are made directly in float32 (``standard_normal(dtype=float32)``,
  ``random(dtype=float32)``) and scaled in float32; the arrays returned are the
  exact values handed to the GPU.  The oracle promotes them to fp64 exactly.
* "N(0, 1/2) per plane" means each of the real and imaginary planes is i.i.d.
  normal with variance 1/2, so E|z|^2 = 1.
* bf16 inputs are the float32 draws rounded to bfloat16 (round to nearest,
  ties to even); ``ForwardInputs.bits()`` gives the uint16 patterns and the
  float32 planes hold the rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

TENSORS = ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt", "A_re", "A_im", "Dskip")
_K = {name: i for i, name in enumerate(TENSORS)}
_HALF_STD = np.float32(math.sqrt(0.5))
_WORKERS = 8


def _rng(seed: int, k: int, step: Optional[int] = None) -> np.random.Generator:
    ent = [int(seed), int(k)] if step is None else [int(seed), int(step), int(k)]
    return np.random.default_rng(np.random.SeedSequence(ent))


def _normal(seed, k, shape, scale=None, step=None) -> np.ndarray:
    a = _rng(seed, k, step).standard_normal(shape, dtype=np.float32)
    if scale is not None:
        a *= np.float32(scale)
    return a


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint32(0x7FC00000)
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-representable; call round_bf16 first")
    return (u >> 16).astype(np.uint16)


@dataclasses.dataclass
class ForwardInputs:
    """Planar float32 inputs of one forward call (all arrays C-contiguous).

    x_*: (B,T,H,D); B_*, C_*: (B,T,H,N); dt: (B,T,H); A_*: (H,);
    Dskip: (H,) or None; h0_*: (B,H,N,D) or None.
    """
    x_re: np.ndarray
    x_im: np.ndarray
    B_re: np.ndarray
    B_im: np.ndarray
    C_re: np.ndarray
    C_im: np.ndarray
    dt: np.ndarray
    A_re: np.ndarray
    A_im: np.ndarray
    Dskip: Optional[np.ndarray]
    chunk: int
    h0_re: Optional[np.ndarray] = None
    h0_im: Optional[np.ndarray] = None
    in_dtype: str = "f32"          # "f32" or "bf16" (x, B, C planes only)
    name: str = ""

    @property
    def shape(self):
        Bsz, T, H, D = self.x_re.shape
        return dict(B=Bsz, T=T, H=H, D=D, N=self.B_re.shape[-1], C=self.chunk)

    def complex(self):
        """complex128 views for the oracle: (x, Bm, Cm, dt, A, Dskip, h0)."""
        c = lambda r, i: r.astype(np.float64) + 1j * i.astype(np.float64)
        h0 = None if self.h0_re is None else c(self.h0_re, self.h0_im)
        ds = None if self.Dskip is None else self.Dskip.astype(np.float64)
        return (c(self.x_re, self.x_im), c(self.B_re, self.B_im), c(self.C_re, self.C_im),
                self.dt.astype(np.float64), c(self.A_re, self.A_im), ds, h0)

    def bits(self, name: str) -> np.ndarray:
        """uint16 bf16 patterns of an x/B/C plane (in_dtype == 'bf16' only)."""
        if self.in_dtype != "bf16":
            raise ValueError("bits() is only meaningful for bf16 inputs")
        return bf16_bits(getattr(self, name))

    def slice_bh(self, b: int, h: int) -> "ForwardInputs":
        """The single sequence (b, h) as a B=1, H=1 problem (for sampled checks)."""
        s = lambda a: np.ascontiguousarray(a[b:b + 1, :, h:h + 1])
        h0r = None if self.h0_re is None else np.ascontiguousarray(self.h0_re[b:b + 1, h:h + 1])
        h0i = None if self.h0_im is None else np.ascontiguousarray(self.h0_im[b:b + 1, h:h + 1])
        return ForwardInputs(s(self.x_re), s(self.x_im), s(self.B_re), s(self.B_im),
                             s(self.C_re), s(self.C_im),
                             np.ascontiguousarray(self.dt[b:b + 1, :, h:h + 1]),
                             self.A_re[h:h + 1].copy(), self.A_im[h:h + 1].copy(),
                             None if self.Dskip is None else self.Dskip[h:h + 1].copy(),
                             self.chunk, h0r, h0i, self.in_dtype, self.name)


def _to_bf16(inp: ForwardInputs) -> ForwardInputs:
    for name in ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im"):
        setattr(inp, name, round_bf16(getattr(inp, name)))
    inp.in_dtype = "bf16"
    return inp


def random_forward(seed: int, B: int, T: int, H: int, D: int, N: int, chunk: int, *,
                   dt_std: float = 1.0, with_h0: bool = False, with_dskip: bool = True,
                   in_dtype: str = "f32", name: str = "") -> ForwardInputs:
    """The config-0 distributions at an arbitrary shape.

    x, B_t, C_t: N(0, 1/2) per plane; dt ~ N(0, dt_std^2) raw (softplus is applied
    by the scan); A_re = -U(0.1, 1), A_im = U(-pi, pi) per head; Dskip ~ N(0, 1)
    per head; h0 = 0 unless ``with_h0`` (then N(0, 1/2) per plane, streams 10, 11).
    """
    jobs = {
        "x_re": ((B, T, H, D), _HALF_STD), "x_im": ((B, T, H, D), _HALF_STD),
        "B_re": ((B, T, H, N), _HALF_STD), "B_im": ((B, T, H, N), _HALF_STD),
        "C_re": ((B, T, H, N), _HALF_STD), "C_im": ((B, T, H, N), _HALF_STD),
        "dt": ((B, T, H), dt_std if dt_std != 1.0 else None),
    }
    with ThreadPoolExecutor(_WORKERS) as ex:
        futs = {k: ex.submit(_normal, seed, _K[k], shp, sc) for k, (shp, sc) in jobs.items()}
        out = {k: f.result() for k, f in futs.items()}
    a_re = -(np.float32(0.1) + np.float32(0.9) * _rng(seed, _K["A_re"]).random(H, dtype=np.float32))
    a_im = (np.float32(2 * math.pi) * _rng(seed, _K["A_im"]).random(H, dtype=np.float32)
            - np.float32(math.pi))
    dskip = _normal(seed, _K["Dskip"], (H,)) if with_dskip else None
    h0r = h0i = None
    if with_h0:
        h0r = _normal(seed, 10, (B, H, N, D), _HALF_STD)
        h0i = _normal(seed, 11, (B, H, N, D), _HALF_STD)
    inp = ForwardInputs(out["x_re"], out["x_im"], out["B_re"], out["B_im"], out["C_re"],
                        out["C_im"], out["dt"], a_re.astype(np.float32), a_im.astype(np.float32),
                        dskip, chunk, h0r, h0i, "f32", name)
    return _to_bf16(inp) if in_dtype == "bf16" else inp


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------
CONFIG_SHAPES = {
    0: dict(B=1, T=64, H=2, D=16, N=16, C=16),
    1: dict(B=8, T=2048, H=48, D=64, N=64, C=64),
    2: dict(B=1, T=16384, H=48, D=64, N=128, C=128),
    3: dict(B=16, T=1024, H=12, D=64, N=128, C=64),   # PAM, Re-score mapping (N = 2d)
    4: dict(B=256, H=48, D=64, N=128, steps=512),     # decode
}


def config0() -> ForwardInputs:
    """Tiny: B1 H2 T64 D16 N16 C16, seed 0."""
    s = CONFIG_SHAPES[0]
    return random_forward(0, s["B"], s["T"], s["H"], s["D"], s["N"], s["C"], name="cfg0_tiny")


def config1(in_dtype: str = "f32") -> ForwardInputs:
    """Mamba-style layer: B8 T2048 H48 D64 N64 C64, seed 1 (fp32 or bf16 inputs)."""
    s = CONFIG_SHAPES[1]
    return random_forward(1, s["B"], s["T"], s["H"], s["D"], s["N"], s["C"], in_dtype=in_dtype,
                          name=f"cfg1_mamba_{in_dtype}")


def long_decay_dt(seed: int, shape, a_re: np.ndarray) -> np.ndarray:
    """Raw dt such that |exp(softplus(dt) A)| = r with log10(1 - r) ~ U(-4, log10 0.5).

    The decay-magnitude target r spans [0.5, 0.9999] log-uniformly in its time
    constant; dt is the raw value whose softplus equals ln(r) / Re A[h] (head is
    the last axis of ``shape``).  Computed in float64, stored as float32.
    """
    u = _rng(seed, _K["dt"]).random(shape)  # float64 in [0, 1)
    lo, hi = -4.0, math.log10(0.5)
    one_minus_r = 10.0 ** (lo + (hi - lo) * u)
    r = 1.0 - one_minus_r
    step = np.log(r) / a_re.astype(np.float64)           # target softplus(dt) > 0
    return np.log(np.expm1(step)).astype(np.float32)      # inverse softplus


def config2() -> ForwardInputs:
    """Long sequence: B1 T16384 H48 D64 N128 C128, seed 2, |Abar| in [0.5, 0.9999]."""
    s = CONFIG_SHAPES[2]
    inp = random_forward(2, s["B"], s["T"], s["H"], s["D"], s["N"], s["C"], name="cfg2_long")
    inp.dt = long_decay_dt(2, (s["B"], s["T"], s["H"]), inp.A_re)
    return inp


@dataclasses.dataclass
class PamInputs:
    """Phase-associative-memory draws (complex128 views of float32 values)."""
    K: np.ndarray      # (B,T,H,d) keys, unit phase, amplitude 1/sqrt(d)
    Q: np.ndarray      # (B,T,H,d) queries
    V: np.ndarray      # (B,T,H,d) values
    gamma: np.ndarray  # (H,) per-head constant decay


def pam_draw(seed: int, B: int, T: int, H: int, d: int) -> PamInputs:
    """K, Q, V = exp(i phi)/sqrt(d), phi ~ U(-pi, pi) (streams 0, 1, 2); gamma ~ U(0.9, 0.999)."""
    amp = 1.0 / math.sqrt(d)

    def unit(k):
        phi = (2 * math.pi) * _rng(seed, k).random((B, T, H, d)) - math.pi
        z = amp * np.exp(1j * phi)
        return (z.real.astype(np.float32).astype(np.float64)
                + 1j * z.imag.astype(np.float32).astype(np.float64))

    gamma = (0.9 + 0.099 * _rng(seed, 3).random(H)).astype(np.float32).astype(np.float64)
    return PamInputs(unit(0), unit(1), unit(2), gamma)


UNIT_STEP_DT = np.float32(math.log(math.e - 1.0))  # raw dt whose softplus is 1 (to fp32 rounding)


def pam_to_scan(p: PamInputs, chunk: int = 64, score: str = "re") -> ForwardInputs:
    """Express the PAM recurrence S_t = gamma S_{t-1} + V_t (x) conj(K_t), read out
    through the query, as the diagonal scan's inputs.

    score="complex": N = d, B_t = conj(K_t), C_t = Q_t / sqrt(d), x_t = V_t.
    score="re":      N = 2d, B_t = [conj(K_t), K_t], C_t = [Q_t, conj(Q_t)] / (2 sqrt(d)),
                     so that sum_n C_t[n] B_i[n] = Re(conj(K_i) . Q_t) / sqrt(d).
    A = ln(gamma) + 0i, dt = ln(e - 1) (softplus(dt) = 1), no skip, zero initial state.
    """
    B, T, H, d = p.K.shape
    rs = 1.0 / math.sqrt(d)
    if score == "complex":
        Bm = np.conj(p.K)
        Cm = p.Q * rs
    elif score == "re":
        Bm = np.concatenate([np.conj(p.K), p.K], axis=-1)
        Cm = np.concatenate([p.Q, np.conj(p.Q)], axis=-1) * (0.5 * rs)
    else:
        raise ValueError(score)
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return ForwardInputs(f(p.V.real), f(p.V.imag), f(Bm.real), f(Bm.imag), f(Cm.real), f(Cm.imag),
                         np.full((B, T, H), UNIT_STEP_DT, dtype=np.float32),
                         f(np.log(p.gamma)), np.zeros(H, dtype=np.float32), None, chunk,
                         name=f"cfg3_pam_{score}")


def config3(score: str = "re") -> ForwardInputs:
    """PAM: B16 T1024 H12 d64, seed 3, mapped per ``pam_to_scan`` with C = 64."""
    return pam_to_scan(pam_draw(3, 16, 1024, 12, 64), 64, score)


# ---------------------------------------------------------------------------
# Decode (config 4)
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class StepInputs:
    """One decode token for all (batch, head): x (B,H,D); B, C (B,H,N); dt (B,H)."""
    x_re: np.ndarray
    x_im: np.ndarray
    B_re: np.ndarray
    B_im: np.ndarray
    C_re: np.ndarray
    C_im: np.ndarray
    dt: np.ndarray

    def complex(self):
        c = lambda r, i: r.astype(np.float64) + 1j * i.astype(np.float64)
        return (c(self.x_re, self.x_im), c(self.B_re, self.B_im), c(self.C_re, self.C_im),
                self.dt.astype(np.float64))


def decode_params(seed: int, H: int):
    """Per-head A (re, im) and Dskip, drawn once as in config 0."""
    a_re = -(np.float32(0.1) + np.float32(0.9) * _rng(seed, _K["A_re"]).random(H, dtype=np.float32))
    a_im = (np.float32(2 * math.pi) * _rng(seed, _K["A_im"]).random(H, dtype=np.float32)
            - np.float32(math.pi))
    return a_re.astype(np.float32), a_im.astype(np.float32), _normal(seed, _K["Dskip"], (H,))


def decode_step(seed: int, step: int, B: int, H: int, D: int, N: int) -> StepInputs:
    """Token ``step``: config-0 distributions from streams SeedSequence([seed, step, k])."""
    def g(k, shp, sc):
        return _normal(seed, _K[k], shp, sc, step=step)
    return StepInputs(g("x_re", (B, H, D), _HALF_STD), g("x_im", (B, H, D), _HALF_STD),
                      g("B_re", (B, H, N), _HALF_STD), g("B_im", (B, H, N), _HALF_STD),
                      g("C_re", (B, H, N), _HALF_STD), g("C_im", (B, H, N), _HALF_STD),
                      g("dt", (B, H), None))


def decode_steps(seed: int, steps: int, B: int, H: int, D: int, N: int):
    """``steps`` consecutive tokens, stacked on a leading axis (generated in parallel)."""
    with ThreadPoolExecutor(_WORKERS) as ex:
        toks = list(ex.map(lambda s: decode_step(seed, s, B, H, D, N), range(steps)))
    return StepInputs(*[np.stack([getattr(t, f.name) for t in toks])
                        for f in dataclasses.fields(StepInputs)])


# ---------------------------------------------------------------------------
# The per-coordinate phase scan (the phase-state paper's H-Mamba layer)
# ---------------------------------------------------------------------------
PHASE_TENSORS = ("phi", "u", "b_re", "b_im", "psi0_re", "psi0_im", "dt", "delta")
_KP = {name: 100 + i for i, name in enumerate(PHASE_TENSORS)}


@dataclasses.dataclass
class PhaseInputs:
    """phi, u, b (B,T,H,N) float32 planes; psi0 (B,H,N) float32 planes."""
    phi: np.ndarray
    u: np.ndarray
    b_re: np.ndarray
    b_im: np.ndarray
    psi0_re: np.ndarray
    psi0_im: np.ndarray

    @property
    def shape(self):
        return self.phi.shape

    def b(self):
        return self.b_re.astype(np.float64) + 1j * self.b_im.astype(np.float64)

    def psi0(self):
        return self.psi0_re.astype(np.float64) + 1j * self.psi0_im.astype(np.float64)


def phase_frequencies(H: int, N: int) -> np.ndarray:
    """Per-coordinate base frequencies (H, N): magnitudes on a geometric grid from
    0.1 to 10 over the N coordinates of a head, signs alternating."""
    n = np.arange(N, dtype=np.float64)
    mag = 0.1 * 100.0 ** (n / max(N - 1, 1))
    sign = np.where(n % 2 == 0, 1.0, -1.0)
    return np.broadcast_to((sign * mag).astype(np.float32), (H, N)).copy()


def phase_inputs(seed: int, B: int, T: int, H: int, N: int) -> PhaseInputs:
    """Seeded inputs shaped like the phase-state paper's H-Mamba layer (sections
    5.2, 5.6, 5.7): the phase parameter is half a step size times a shift plus a
    base frequency, with the step size per (b, t, h) log-uniform on [1e-3, 1e-1]
    (the page caps it at 0.1), the shift N(0, 1) per coordinate and the base
    frequencies of ``phase_frequencies``; gate logits u ~ N(1.5, 2^2) (gates from
    about 0.1 to 0.99); b ~ N(0, 1/2) per plane; psi0 a complex normal draw per
    (h, n), scaled to unit norm per head and shared by every batch row."""
    shp = (B, T, H, N)
    with ThreadPoolExecutor(_WORKERS) as ex:
        fut = {
            "delta": ex.submit(_normal, seed, _KP["delta"], shp),
            "u": ex.submit(_normal, seed, _KP["u"], shp, 2.0),
            "b_re": ex.submit(_normal, seed, _KP["b_re"], shp, _HALF_STD),
            "b_im": ex.submit(_normal, seed, _KP["b_im"], shp, _HALF_STD),
        }
        r = {k: f.result() for k, f in fut.items()}
    lg = _rng(seed, _KP["dt"]).random((B, T, H, 1), dtype=np.float32)
    step = np.power(np.float32(10.0), np.float32(-3.0) + np.float32(2.0) * lg)
    phi = np.float32(0.5) * step * (r["delta"] + phase_frequencies(H, N)[None, None])
    u = r["u"] + np.float32(1.5)
    z_re = _normal(seed, _KP["psi0_re"], (H, N))
    z_im = _normal(seed, _KP["psi0_im"], (H, N))
    nrm = np.sqrt(np.sum(z_re.astype(np.float64) ** 2 + z_im.astype(np.float64) ** 2, axis=1,
                         keepdims=True))
    p_re = np.broadcast_to((z_re / nrm).astype(np.float32), (B, H, N)).copy()
    p_im = np.broadcast_to((z_im / nrm).astype(np.float32), (B, H, N)).copy()
    return PhaseInputs(phi.astype(np.float32), u.astype(np.float32), r["b_re"], r["b_im"],
                       p_re, p_im)


# ---------------------------------------------------------------------------
# Causal Born attention (the phase-state paper's H-Transformer layer)
# ---------------------------------------------------------------------------
BORN_TENSORS = ("q_re", "q_im", "k_re", "k_im", "v_re", "v_im", "tau")
_KB = {name: 200 + i for i, name in enumerate(BORN_TENSORS)}


@dataclasses.dataclass
class BornInputs:
    """q, k, v (B,T,H,D) float32 planes; tau (B,T,H) float32."""
    q_re: np.ndarray
    q_im: np.ndarray
    k_re: np.ndarray
    k_im: np.ndarray
    v_re: np.ndarray
    v_im: np.ndarray
    tau: np.ndarray

    def complex(self):
        c = lambda r, i: r.astype(np.float64) + 1j * i.astype(np.float64)
        return (c(self.q_re, self.q_im), c(self.k_re, self.k_im), c(self.v_re, self.v_im),
                self.tau.astype(np.float64))


def born_inputs(seed: int, B: int, T: int, H: int, D: int) -> BornInputs:
    """Seeded inputs shaped like the phase-state paper's H-Transformer layer
    (sections 5.5, 5.7): complex queries, keys and values N(0, 1/2) per plane,
    and a temperature per (b, t, h) uniform on [0.5, 2)."""
    shp = (B, T, H, D)
    with ThreadPoolExecutor(_WORKERS) as ex:
        fut = {n: ex.submit(_normal, seed, _KB[n], shp, _HALF_STD) for n in BORN_TENSORS[:6]}
        r = {k: f.result() for k, f in fut.items()}
    tau = np.float32(0.5) + np.float32(1.5) * _rng(seed, _KB["tau"]).random((B, T, H),
                                                                          dtype=np.float32)
    return BornInputs(r["q_re"], r["q_im"], r["k_re"], r["k_im"], r["v_re"], r["v_im"], tau)
