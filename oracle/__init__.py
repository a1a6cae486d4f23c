"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle for the complex diagonal scan.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library and its Python
binding never import it, and the two share no code: the only module both sides
use is the seeded input generator ``cssd_workloads``, which holds none of the
method's arithmetic.

The arithmetic lives in ``cssd_oracle.c`` (plain C, fp64, serial in time,
OpenMP over independent (batch, head) sequences).  This file only compiles it
with gcc, loads it with ctypes, and converts numpy arrays to the planar fp64
layout the C code reads.  What is computed, and from which passages, is written
at the top of ``cssd_oracle.c``:

    a_t = exp(softplus(dt_t) * A)            (Mamba-3-Lite docs, "Complex-Valued
                                              State Spaces", Discretization)
    h_t = a_t h_{t-1} + B_t (x) x_t          (Mamba-3-Lite docs, "SSD Theory",
    y_t = sum_n C_t[n] h_t[n,:] + D x_t       section 2; skip term from the
                                              burn-mamba step_constant module)

with its constant-input forms, its gradients, the phase-state paper's
per-coordinate Cayley-phase scan (section 5.2) and its causal Born attention
(section 5.5, eq. 5).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cssd_oracle.c")
_LIB = os.path.join(_HERE, "libcssd_oracle.so")
_lock = threading.Lock()
_lib = None

_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math).  Returns the path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str | None = None, rebuild: bool = False):
    """Load (building first if needed) the oracle shared library."""
    global _lib
    with _lock:
        if path is not None:
            return _bind(ctypes.CDLL(path))
        if _lib is None or rebuild:
            if rebuild or not os.path.exists(_LIB) or (
                    os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                build()
            _lib = _bind(ctypes.CDLL(_LIB))
        return _lib


def _bind(lib):
    lib.oracle_forward_f64.restype = ctypes.c_int
    lib.oracle_forward_f64.argtypes = [_i64] * 5 + [_d] * 10 + [_d] * 2 + [_d] * 4 + [ctypes.c_int]
    lib.oracle_step_f64.restype = ctypes.c_int
    lib.oracle_step_f64.argtypes = [_i64] * 4 + [_d] * 10 + [_d] * 4 + [ctypes.c_int]
    lib.oracle_step_n_f64.restype = ctypes.c_int
    lib.oracle_step_n_f64.argtypes = [_i64] * 5 + [_d] * 10 + [_d] * 4 + [ctypes.c_int]
    lib.oracle_step_infinite_f64.restype = ctypes.c_int
    lib.oracle_step_infinite_f64.argtypes = [_i64] * 4 + [_d] * 10 + [_d] * 2 + [ctypes.c_int]
    lib.oracle_backward_f64.restype = ctypes.c_int
    lib.oracle_backward_f64.argtypes = [_i64] * 5 + [_d] * 10 + [_d] * 2 + [_d] * 4 + [_d] * 6 \
        + [_d] * 1 + [_d] * 3 + [_d] * 2 + [ctypes.c_int]
    lib.oracle_phase_scan_f64.restype = ctypes.c_int
    lib.oracle_phase_scan_f64.argtypes = [_i64] * 4 + [_d] * 6 + [_d] * 4 + [ctypes.c_int]
    lib.oracle_born_attention_f64.argtypes = [_i64] * 4 + [_d] * 7 + [_d] * 2 + [ctypes.c_int]
    lib.oracle_born_attention_rows_f64.argtypes = [_i64] * 4 + [_d] * 7 + [_i64,
                                                  ctypes.POINTER(_i64)] + [_d] * 2 + [ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    return lib


def _planes(z, shape=None):
    z = np.asarray(z)
    if shape is not None and z.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {z.shape}")
    re = np.ascontiguousarray(z.real, dtype=np.float64)
    im = np.ascontiguousarray(z.imag if np.iscomplexobj(z) else np.zeros(z.shape), dtype=np.float64)
    return re, im


def _real(a, shape):
    a = np.ascontiguousarray(np.asarray(a), dtype=np.float64)
    if a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _p(a):
    return a.ctypes.data_as(_d) if a is not None else None


def forward(x, Bm, Cm, dt, A, Dskip=None, h0=None, nthreads: int = 0, lib=None):
    """Sequential fp64 recurrence over the whole sequence.

    x: (B,T,H,D) complex; Bm, Cm: (B,T,H,N) complex; dt: (B,T,H) real;
    A: (H,) complex; Dskip: (H,) real or None; h0: (B,H,N,D) complex or None.
    Returns (y (B,T,H,D) complex128, hT (B,H,N,D) complex128).
    """
    lib = lib or load()
    x = np.asarray(x)
    Bsz, T, H, D = x.shape
    N = np.asarray(Bm).shape[-1]
    xr, xi = _planes(x)
    br, bi = _planes(Bm, (Bsz, T, H, N))
    cr, ci = _planes(Cm, (Bsz, T, H, N))
    dtv = _real(dt, (Bsz, T, H))
    ar, ai = _planes(np.asarray(A, dtype=np.complex128), (H,))
    ds = _real(Dskip, (H,)) if Dskip is not None else None
    if h0 is not None:
        h0r, h0i = _planes(h0, (Bsz, H, N, D))
    else:
        h0r = h0i = None
    yr = np.empty((Bsz, T, H, D)); yi = np.empty_like(yr)
    hr = np.empty((Bsz, H, N, D)); hi = np.empty_like(hr)
    rc = lib.oracle_forward_f64(Bsz, T, H, D, N, _p(xr), _p(xi), _p(br), _p(bi), _p(cr), _p(ci),
                                _p(dtv), _p(ar), _p(ai), _p(ds), _p(h0r), _p(h0i),
                                _p(yr), _p(yi), _p(hr), _p(hi), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_forward_f64 failed")
    return yr + 1j * yi, hr + 1j * hi


def step(x, Bm, Cm, dt, A, Dskip, h, nthreads: int = 0, lib=None):
    """One decode step for all (batch, head).  h (B,H,N,D) complex is NOT modified;
    returns (y (B,H,D) complex128, h_new (B,H,N,D) complex128)."""
    lib = lib or load()
    x = np.asarray(x)
    Bsz, H, D = x.shape
    N = np.asarray(Bm).shape[-1]
    xr, xi = _planes(x)
    br, bi = _planes(Bm, (Bsz, H, N))
    cr, ci = _planes(Cm, (Bsz, H, N))
    dtv = _real(dt, (Bsz, H))
    ar, ai = _planes(np.asarray(A, dtype=np.complex128), (H,))
    ds = _real(Dskip, (H,)) if Dskip is not None else None
    hr, hi = _planes(h, (Bsz, H, N, D))
    hr = hr.copy(); hi = hi.copy()
    yr = np.empty((Bsz, H, D)); yi = np.empty_like(yr)
    rc = lib.oracle_step_f64(Bsz, H, D, N, _p(xr), _p(xi), _p(br), _p(bi), _p(cr), _p(ci),
                             _p(dtv), _p(ar), _p(ai), _p(ds), _p(hr), _p(hi), _p(yr), _p(yi),
                             int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_step_f64 failed")
    return yr + 1j * yi, hr + 1j * hi


def step_n(x, Bm, Cm, dt, A, Dskip, h, n: int, nthreads: int = 0, lib=None):
    """The same input held for n steps, in closed form.  h (B,H,N,D) complex is
    NOT modified; returns (y_n (B,H,D) complex128, h_n (B,H,N,D) complex128)."""
    lib = lib or load()
    x = np.asarray(x)
    Bsz, H, D = x.shape
    N = np.asarray(Bm).shape[-1]
    xr, xi = _planes(x)
    br, bi = _planes(Bm, (Bsz, H, N))
    cr, ci = _planes(Cm, (Bsz, H, N))
    dtv = _real(dt, (Bsz, H))
    ar, ai = _planes(np.asarray(A, dtype=np.complex128), (H,))
    ds = _real(Dskip, (H,)) if Dskip is not None else None
    hr, hi = _planes(h, (Bsz, H, N, D))
    hr = hr.copy(); hi = hi.copy()
    yr = np.empty((Bsz, H, D)); yi = np.empty_like(yr)
    rc = lib.oracle_step_n_f64(Bsz, H, D, N, int(n), _p(xr), _p(xi), _p(br), _p(bi), _p(cr),
                               _p(ci), _p(dtv), _p(ar), _p(ai), _p(ds), _p(hr), _p(hi), _p(yr),
                               _p(yi), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_step_n_f64 failed")
    return yr + 1j * yi, hr + 1j * hi


def step_infinite(x, Bm, Cm, dt, A, Dskip, nthreads: int = 0, lib=None):
    """The stationary output of an endless constant input; returns y (B,H,D) complex128."""
    lib = lib or load()
    x = np.asarray(x)
    Bsz, H, D = x.shape
    N = np.asarray(Bm).shape[-1]
    xr, xi = _planes(x)
    br, bi = _planes(Bm, (Bsz, H, N))
    cr, ci = _planes(Cm, (Bsz, H, N))
    dtv = _real(dt, (Bsz, H))
    ar, ai = _planes(np.asarray(A, dtype=np.complex128), (H,))
    ds = _real(Dskip, (H,)) if Dskip is not None else None
    yr = np.empty((Bsz, H, D)); yi = np.empty_like(yr)
    rc = lib.oracle_step_infinite_f64(Bsz, H, D, N, _p(xr), _p(xi), _p(br), _p(bi), _p(cr),
                                      _p(ci), _p(dtv), _p(ar), _p(ai), _p(ds), _p(yr), _p(yi),
                                      int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_step_infinite_f64 failed")
    return yr + 1j * yi


def backward(x, Bm, Cm, dt, A, Dskip, h0, dy, dhT=None, nthreads: int = 0, lib=None):
    """Gradients of the forward recurrence for upstream dy (B,T,H,D) complex and
    dhT (B,H,N,D) complex or None, as complex numbers dL/dRe + i dL/dIm.
    Returns a dict with dx, dB, dC (input shapes, complex128), ddt (B,T,H),
    dA (H,) complex, dD (H,) real and dh0 (B,H,N,D) complex."""
    lib = lib or load()
    x = np.asarray(x)
    Bsz, T, H, D = x.shape
    N = np.asarray(Bm).shape[-1]
    xr, xi = _planes(x)
    br, bi = _planes(Bm, (Bsz, T, H, N))
    cr, ci = _planes(Cm, (Bsz, T, H, N))
    dtv = _real(dt, (Bsz, T, H))
    ar, ai = _planes(np.asarray(A, dtype=np.complex128), (H,))
    ds = _real(Dskip, (H,)) if Dskip is not None else None
    h0r, h0i = _planes(h0, (Bsz, H, N, D)) if h0 is not None else (None, None)
    gyr, gyi = _planes(dy, (Bsz, T, H, D))
    ghr, ghi = _planes(dhT, (Bsz, H, N, D)) if dhT is not None else (None, None)
    out = {k: np.empty(shp) for k, shp in (("dxr", (Bsz, T, H, D)), ("dxi", (Bsz, T, H, D)),
                                            ("dbr", (Bsz, T, H, N)), ("dbi", (Bsz, T, H, N)),
                                            ("dcr", (Bsz, T, H, N)), ("dci", (Bsz, T, H, N)),
                                            ("ddt", (Bsz, T, H)), ("dar", (H,)), ("dai", (H,)),
                                            ("dd", (H,)), ("dh0r", (Bsz, H, N, D)),
                                            ("dh0i", (Bsz, H, N, D)))}
    rc = lib.oracle_backward_f64(Bsz, T, H, D, N, _p(xr), _p(xi), _p(br), _p(bi), _p(cr), _p(ci),
                                 _p(dtv), _p(ar), _p(ai), _p(ds), _p(h0r), _p(h0i), _p(gyr),
                                 _p(gyi), _p(ghr), _p(ghi), _p(out["dxr"]), _p(out["dxi"]),
                                 _p(out["dbr"]), _p(out["dbi"]), _p(out["dcr"]), _p(out["dci"]),
                                 _p(out["ddt"]), _p(out["dar"]), _p(out["dai"]), _p(out["dd"]),
                                 _p(out["dh0r"]), _p(out["dh0i"]), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_backward_f64 failed")
    return {"dx": out["dxr"] + 1j * out["dxi"], "dB": out["dbr"] + 1j * out["dbi"],
            "dC": out["dcr"] + 1j * out["dci"], "ddt": out["ddt"],
            "dA": out["dar"] + 1j * out["dai"], "dD": out["dd"],
            "dh0": out["dh0r"] + 1j * out["dh0i"]}


def phase_scan(phi, u, b, psi0=None, nthreads: int = 0, lib=None):
    """Per-coordinate scan psi_t = sigmoid(u_t) cayley(phi_t) psi_{t-1} + b_t.
    phi, u: (B,T,H,N) real; b: (B,T,H,N) complex; psi0: (B,H,N) complex or None.
    Returns (psi (B,T,H,N) complex128, psiT (B,H,N) complex128)."""
    lib = lib or load()
    phi = _real(phi, np.shape(phi))
    Bsz, T, H, N = phi.shape
    uv = _real(u, (Bsz, T, H, N))
    br, bi = _planes(b, (Bsz, T, H, N))
    p0r, p0i = _planes(psi0, (Bsz, H, N)) if psi0 is not None else (None, None)
    pr = np.empty((Bsz, T, H, N)); pi = np.empty_like(pr)
    tr = np.empty((Bsz, H, N)); ti = np.empty_like(tr)
    rc = lib.oracle_phase_scan_f64(Bsz, T, H, N, _p(phi), _p(uv), _p(br), _p(bi), _p(p0r),
                                   _p(p0i), _p(pr), _p(pi), _p(tr), _p(ti), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_phase_scan_f64 failed")
    return pr + 1j * pi, tr + 1j * ti


def born_attention(q, k, v, tau=None, nthreads: int = 0, lib=None):
    """Causal Born attention psi_i = sum_{j<=i} s_ij v_j / sum_{j<=i} s_ij with
    s_ij = |<q_i|k_j>|^2 / (D tau_i).  q, k, v: (B,T,H,D) complex; tau: (B,T,H)
    real or None.  Returns psi (B,T,H,D) complex128."""
    lib = lib or load()
    q = np.asarray(q)
    Bsz, T, H, D = q.shape
    qr, qi = _planes(q)
    kr, ki = _planes(k, (Bsz, T, H, D))
    vr, vi = _planes(v, (Bsz, T, H, D))
    tv = _real(tau, (Bsz, T, H)) if tau is not None else None
    outr = np.empty((Bsz, T, H, D)); outi = np.empty_like(outr)
    rc = lib.oracle_born_attention_f64(Bsz, T, H, D, _p(qr), _p(qi), _p(kr), _p(ki), _p(vr), _p(vi),
                                       _p(tv), _p(outr), _p(outi), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_born_attention_f64 failed")
    return outr + 1j * outi


def born_attention_rows(q, k, v, tau, rows, nthreads: int = 0, lib=None):
    """born_attention for the listed rows only: rows is an (M, 3) integer array
    of (b, t, h); returns (M, D) complex128.  The planes may be given as
    (re, im) pairs of float arrays to avoid forming complex copies."""
    lib = lib or load()
    pl = lambda z: tuple(np.ascontiguousarray(a, dtype=np.float64) for a in z) \
        if isinstance(z, tuple) else _planes(z)
    qr, qi = pl(q)
    Bsz, T, H, D = qr.shape
    kr, ki = pl(k)
    vr, vi = pl(v)
    for a in (qi, kr, ki, vr, vi):
        if a.shape != (Bsz, T, H, D):
            raise ValueError("q, k, v planes must share one (B,T,H,D) shape")
    tv = _real(tau, (Bsz, T, H)) if tau is not None else None
    rw = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    M = rw.shape[0]
    outr = np.empty((M, D)); outi = np.empty_like(outr)
    rc = lib.oracle_born_attention_rows_f64(Bsz, T, H, D, _p(qr), _p(qi), _p(kr), _p(ki), _p(vr),
                                            _p(vi), _p(tv), M,
                                            rw.ctypes.data_as(ctypes.POINTER(_i64)), _p(outr),
                                            _p(outi), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_born_attention_rows_f64 failed")
    return outr + 1j * outi


def max_threads(lib=None) -> int:
    return (lib or load()).oracle_max_threads()
