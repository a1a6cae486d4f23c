"""Helpers for the GPU tests: move seeded inputs to the device, run the HIP path
through the binding, run the oracle on the same values, compare."""
from __future__ import annotations

import sys

import numpy as np

import cssd_workloads as wl


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_inputs(inp: wl.ForwardInputs, device="cuda:0"):
    import torch
    io = torch.bfloat16 if inp.in_dtype == "bf16" else torch.float32

    def t(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)

    d = dict(x_re=t(inp.x_re, io), x_im=t(inp.x_im, io), B_re=t(inp.B_re, io), B_im=t(inp.B_im, io),
             C_re=t(inp.C_re, io), C_im=t(inp.C_im, io), dt=t(inp.dt), A_re=t(inp.A_re),
             A_im=t(inp.A_im), Dskip=None if inp.Dskip is None else t(inp.Dskip))
    d["h0"] = None if inp.h0_re is None else (t(inp.h0_re), t(inp.h0_im))
    return d


def gpu_forward(inp: wl.ForwardInputs, chunk=None, device="cuda:0"):
    """Run cssd_forward; returns (y, hT) as complex128 numpy arrays."""
    import torch
    import complex_valued_state_amd as cssd
    d = dev_inputs(inp, device)
    y_re, y_im, h_re, h_im = cssd.cssd_forward(
        d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"], d["dt"], d["A_re"],
        d["A_im"], d["Dskip"], d["h0"], chunk=chunk or inp.chunk)
    torch.cuda.synchronize()
    to = lambda r, i: r.double().cpu().numpy() + 1j * i.double().cpu().numpy()
    return to(y_re, y_im), to(h_re, h_im)


def oracle_forward(inp: wl.ForwardInputs, nthreads: int = 0):
    import oracle
    x, Bm, Cm, dt, A, Dk, h0 = inp.complex()
    return oracle.forward(x, Bm, Cm, dt, A, Dk, h0, nthreads=nthreads)


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over all elements (complex modulus)."""
    got = np.asarray(got); ref = np.asarray(ref)
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (den if den > 0 else 1.0)


def sampled_oracle(inp: wl.ForwardInputs, pairs, nthreads: int = 0):
    """Oracle on selected (b, h) sequences only: {(b, h): (y (T,D), hT (N,D))}."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    def one(bh):
        b, h = bh
        s = inp.slice_bh(b, h)
        x, Bm, Cm, dt, A, Dk, h0 = s.complex()
        y, hT = oracle.forward(x, Bm, Cm, dt, A, Dk, h0, nthreads=1)
        return bh, (y[0, :, 0, :], hT[0, 0])

    with ThreadPoolExecutor(max(1, min(len(pairs), nthreads or 8))) as ex:
        return dict(ex.map(one, pairs))
