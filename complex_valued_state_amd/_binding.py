"""ctypes binding of libcssd.so (include/cssd.h).

Argument marshalling only: shapes, dtypes, devices and contiguity are checked,
outputs and the workspace are allocated with torch (device memory plumbing),
raw pointers and the current HIP stream are handed to the C ABI, and a status
other than CSSD_OK raises CSSDError.  Every step of the computation runs in the
library's HIP kernels; there is no other code path.  If the library is not
built, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
import threading
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcssd.so")

CSSD_OK, CSSD_ERR_INVALID_ARG, CSSD_ERR_UNSUPPORTED, CSSD_ERR_WORKSPACE, CSSD_ERR_HIP = range(5)
CSSD_F32, CSSD_BF16 = 0, 1
KERNEL_NAMES = ("k_cumsum", "k_chunk_state", "k_state_pass", "k_chunk_scan", "k_step",
                "k_step_infinite", "k_bwd_dx", "k_bwd_dc", "k_bwd_dz",
                "k_phase_summary", "k_phase_carry", "k_phase_out", "k_born", "k_bwd_db",
                "k_state_scan", "k_state_scan_adj", "k_fill", "k_scan_fused", "k_widen")

_lock = threading.Lock()
_lib = None

_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t


class CSSDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load_library(path: Optional[str] = None):
    """Load libcssd.so and declare its C signatures.  Raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is not built: run `python -m complex_valued_state_amd.build` "
                               "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(p)
        lib.cssd_version.restype = ctypes.c_int
        lib.cssd_version.argtypes = []
        lib.cssd_status_string.restype = ctypes.c_char_p
        lib.cssd_status_string.argtypes = [ctypes.c_int]
        lib.cssd_forward_workspace_size.restype = ctypes.c_int
        lib.cssd_forward_workspace_size.argtypes = [_i64] * 6 + [ctypes.POINTER(_sz)]
        lib.cssd_forward.restype = ctypes.c_int
        lib.cssd_forward.argtypes = [_i64] * 6 + [_i32] + [_vp] * 6 + [_vp] * 4 + [_vp] * 2 \
            + [_vp] * 4 + [_vp, _sz, _vp]
        lib.cssd_forward_noalloc.restype = ctypes.c_int
        lib.cssd_forward_noalloc.argtypes = [_i64] * 6 + [_i32] + [_vp] * 6 + [_vp] * 4 \
            + [_vp] * 2 + [_vp] * 4 + [_vp]
        lib.cssd_backward_workspace_size.restype = ctypes.c_int
        lib.cssd_backward_workspace_size.argtypes = [_i64] * 6 + [ctypes.POINTER(_sz)]
        lib.cssd_backward_workspace_size_dtype.restype = ctypes.c_int
        lib.cssd_backward_workspace_size_dtype.argtypes = [_i64] * 6 + [_i32, ctypes.POINTER(_sz)]
        lib.cssd_backward.restype = ctypes.c_int
        lib.cssd_backward.argtypes = [_i64] * 6 + [_i32] + [_vp] * 6 + [_vp] * 4 + [_vp] * 2 \
            + [_vp] * 2 + [_vp] * 4 + [_vp] * 6 + [_vp] * 4 + [_vp] * 2 + [_vp, _sz, _vp]
        lib.cssd_backward_saved.restype = ctypes.c_int
        lib.cssd_backward_saved.argtypes = [_i64] * 6 + [_i32] + [_vp] * 6 + [_vp] * 4 \
            + [_vp] * 2 + [_vp] * 2 + [_vp] * 2 + [_vp] * 4 + [_vp] * 6 + [_vp] * 4 + [_vp] * 2 \
            + [_vp, _sz, _vp]
        lib.cssd_step.restype = ctypes.c_int
        lib.cssd_step.argtypes = [_i64] * 4 + [_vp] * 10 + [_vp] * 4 + [_vp]
        lib.cssd_step_n.restype = ctypes.c_int
        lib.cssd_step_n.argtypes = [_i64] * 5 + [_vp] * 10 + [_vp] * 4 + [_vp]
        lib.cssd_step_infinite.restype = ctypes.c_int
        lib.cssd_step_infinite.argtypes = [_i64] * 4 + [_vp] * 10 + [_vp] * 2 + [_vp]
        lib.cssd_phase_scan_workspace_size.restype = ctypes.c_int
        lib.cssd_phase_scan_workspace_size.argtypes = [_i64] * 5 + [ctypes.POINTER(_sz)]
        lib.cssd_phase_scan.restype = ctypes.c_int
        lib.cssd_phase_scan.argtypes = [_i64] * 5 + [_vp] * 10 + [_vp, _sz, _vp]
        lib.cssd_born_attention.restype = ctypes.c_int
        lib.cssd_born_attention.argtypes = [_i64] * 4 + [_i32] + [_vp] * 7 + [_vp] * 2 + [_vp]
        lib.cssd_profile_enable.restype = ctypes.c_int
        lib.cssd_profile_enable.argtypes = [ctypes.c_int]
        lib.cssd_profile_read.restype = ctypes.c_int
        lib.cssd_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
        lib.cssd_kernel_name.restype = ctypes.c_char_p
        lib.cssd_kernel_name.argtypes = [ctypes.c_int]
        if path is None:
            _lib = lib
        return lib


def status_string(status: int) -> str:
    try:
        return load_library().cssd_status_string(int(status)).decode()
    except RuntimeError:
        return f"status {status}"


def cssd_version() -> int:
    return load_library().cssd_version()


def cssd_forward_workspace_size(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                                chunk: int) -> int:
    out = _sz(0)
    st = load_library().cssd_forward_workspace_size(batch, seqlen, nheads, headdim, dstate, chunk,
                                                    ctypes.byref(out))
    if st != CSSD_OK:
        raise CSSDError(st, "cssd_forward_workspace_size")
    return int(out.value)


def cssd_backward_workspace_size(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                                 chunk: int, in_dtype: int = CSSD_F32) -> int:
    """Workspace bytes of cssd_backward with x, B, C of in_dtype (CSSD_F32 or
    CSSD_BF16: the latter adds the fp32 copies the inputs are widened into)."""
    out = _sz(0)
    st = load_library().cssd_backward_workspace_size_dtype(batch, seqlen, nheads, headdim, dstate,
                                                           chunk, in_dtype, ctypes.byref(out))
    if st != CSSD_OK:
        raise CSSDError(st, "cssd_backward_workspace_size_dtype")
    return int(out.value)


def cssd_phase_scan_workspace_size(batch: int, seqlen: int, nheads: int, dstate: int,
                                   chunk: int = 0) -> int:
    out = _sz(0)
    st = load_library().cssd_phase_scan_workspace_size(batch, seqlen, nheads, dstate, chunk,
                                                       ctypes.byref(out))
    if st != CSSD_OK:
        raise CSSDError(st, "cssd_phase_scan_workspace_size")
    return int(out.value)


# ---------------------------------------------------------------------------
# torch-facing helpers (torch is plumbing: device memory and streams)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _check(t, name, shape: Sequence[int], dtypes, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must live on the GPU device {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _on_stream(fn):
    """Run a binding call with `stream` (when given) as torch's current stream, so
    that the outputs and workspace the binding allocates come from that stream's
    pool of the caching allocator.  A block freed after the call is then reused
    only by later work on the same stream, which the kernels already enqueued
    there precede; allocated on another stream, it could be handed to new work
    there while the kernels still use it."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kwargs):
        ctx = contextlib.nullcontext() if stream is None else _torch().cuda.stream(stream)
        with ctx:
            return fn(*args, stream=stream, **kwargs)
    return call


def _stream_ptr(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(int(stream.cuda_stream))


@_on_stream
def cssd_forward(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip=None, h0=None, *,
                 chunk: int, return_state: bool = True, out=None, workspace=None, stream=None):
    """Chunkwise complex scan over a whole sequence (see include/cssd.h).

    x_*: (B,T,H,D); B_*, C_*: (B,T,H,N) -- float32, or all six bfloat16 for the
    bf16-input variant; dt: (B,T,H) float32; A_*: (H,) float32; Dskip: (H,)
    float32 or None; h0: (h0_re, h0_im) each (B,H,N,D) float32, or None.
    out: optional (y_re, y_im[, hT_re, hT_im]) preallocated outputs.
    Returns (y_re, y_im, hT_re, hT_im) (the last two None if not return_state).
    """
    return _forward(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0, chunk,
                    return_state, out, workspace, stream, noalloc=False)


@_on_stream
def cssd_forward_noalloc(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip=None,
                         h0=None, *, chunk: int, return_state: bool = True, out=None,
                         stream=None):
    """cssd_forward with its workspace in the library's fixed device array (see
    include/cssd.h): the library allocates nothing.  Arguments and result as
    cssd_forward, without a workspace; pass `out` as well for a call in which
    nothing at all is allocated.  Problems whose workspace exceeds
    CSSD_NOALLOC_SCRATCH_BYTES raise CSSDError (CSSD_ERR_TOO_LARGE)."""
    return _forward(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0, chunk,
                    return_state, out, None, stream, noalloc=True)


CSSD_NOALLOC_SCRATCH_BYTES = 64 << 20
CSSD_ERR_TOO_LARGE = 5


def _forward(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0, chunk, return_state,
             out, workspace, stream, noalloc):
    torch = _torch()
    lib = load_library()
    dev = x_re.device
    Bsz, T, H, D = x_re.shape
    N = B_re.shape[-1]
    in_dt = x_re.dtype
    if in_dt == torch.float32:
        code, okd = CSSD_F32, (torch.float32,)
    elif in_dt == torch.bfloat16:
        code, okd = CSSD_BF16, (torch.bfloat16,)
    else:
        raise TypeError("x/B/C planes must be float32 or bfloat16")
    f32 = (torch.float32,)
    p = {}
    for name, t, shp, dts in (("x_re", x_re, (Bsz, T, H, D), okd), ("x_im", x_im, (Bsz, T, H, D), okd),
                              ("B_re", B_re, (Bsz, T, H, N), okd), ("B_im", B_im, (Bsz, T, H, N), okd),
                              ("C_re", C_re, (Bsz, T, H, N), okd), ("C_im", C_im, (Bsz, T, H, N), okd),
                              ("dt", dt, (Bsz, T, H), f32), ("A_re", A_re, (H,), f32),
                              ("A_im", A_im, (H,), f32)):
        p[name] = _check(t, name, shp, dts, dev)
    p["Dskip"] = None if Dskip is None else _check(Dskip, "Dskip", (H,), f32, dev)
    if h0 is not None:
        p["h0_re"] = _check(h0[0], "h0_re", (Bsz, H, N, D), f32, dev)
        p["h0_im"] = _check(h0[1], "h0_im", (Bsz, H, N, D), f32, dev)
    else:
        p["h0_re"] = p["h0_im"] = None
    if out is not None:
        y_re, y_im = out[0], out[1]
        hT_re, hT_im = (out[2], out[3]) if (return_state and len(out) >= 4) else (None, None)
    else:
        y_re = torch.empty((Bsz, T, H, D), dtype=torch.float32, device=dev)
        y_im = torch.empty_like(y_re)
        hT_re = hT_im = None
    if return_state and hT_re is None:
        hT_re = torch.empty((Bsz, H, N, D), dtype=torch.float32, device=dev)
        hT_im = torch.empty_like(hT_re)
    p["y_re"] = _check(y_re, "y_re", (Bsz, T, H, D), f32, dev)
    p["y_im"] = _check(y_im, "y_im", (Bsz, T, H, D), f32, dev)
    p["hT_re"] = None if hT_re is None else _check(hT_re, "hT_re", (Bsz, H, N, D), f32, dev)
    p["hT_im"] = None if hT_im is None else _check(hT_im, "hT_im", (Bsz, H, N, D), f32, dev)
    args = (Bsz, T, H, D, N, int(chunk), code,
            p["x_re"], p["x_im"], p["B_re"], p["B_im"], p["C_re"], p["C_im"],
            p["dt"], p["A_re"], p["A_im"], p["Dskip"], p["h0_re"], p["h0_im"],
            p["y_re"], p["y_im"], p["hT_re"], p["hT_im"])
    if noalloc:
        st = lib.cssd_forward_noalloc(*args, _stream_ptr(stream, dev))
        if st != CSSD_OK:
            raise CSSDError(st, "cssd_forward_noalloc")
        return y_re, y_im, hT_re, hT_im
    need = cssd_forward_workspace_size(Bsz, T, H, D, N, chunk)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.cssd_forward(*args, workspace.data_ptr(), ws_bytes, _stream_ptr(stream, dev))
    if st != CSSD_OK:
        raise CSSDError(st, "cssd_forward")
    return y_re, y_im, hT_re, hT_im


@_on_stream
def cssd_backward(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0, y, dy, dhT=None,
                  *, chunk: int, want_dh0: bool = True, workspace=None, stream=None):
    """Gradients of cssd_forward (see include/cssd.h): planar (dL/dRe, dL/dIm) pairs.

    The first arguments are the forward inputs (x, B, C float32 or bfloat16, the
    rest float32; bfloat16 planes are widened once into the workspace); h0 as in
    cssd_forward;
    y = (y_re, y_im), the forward output, is not read and may be None (the
    gradients need only the inputs), dy = (dy_re, dy_im)
    its upstream gradient, dhT = (dhT_re, dhT_im) that of the final state or None.
    Returns a dict of float32 tensors: dx_re, dx_im, dB_re, dB_im, dC_re, dC_im,
    ddt, dA_re, dA_im, dD (None without Dskip), dh0_re, dh0_im (None unless
    want_dh0)."""
    return _backward(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0, y, dy, dhT,
                     chunk, want_dh0, workspace, stream, None)


@_on_stream
def cssd_backward_saved(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0, y, hT, dy,
                        dhT=None, *, chunk: int, workspace, want_dh0: bool = True, stream=None):
    """cssd_backward on the states a cssd_forward call left in `workspace` (a uint8
    tensor of at least cssd_backward_workspace_size bytes that was that call's
    workspace, untouched since); hT = (hT_re, hT_im) is that call's final state,
    needed when dhT is given, else may be None.  Same result as cssd_backward,
    without the forward recomputation."""
    if workspace is None:
        raise ValueError("cssd_backward_saved needs the forward call's workspace")
    return _backward(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0, y, dy, dhT,
                     chunk, want_dh0, workspace, stream, (hT,))


def _backward(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0, y, dy, dhT, chunk,
              want_dh0, workspace, stream, saved):
    torch = _torch()
    lib = load_library()
    dev = x_re.device
    Bsz, T, H, D = x_re.shape
    N = B_re.shape[-1]
    f32 = (torch.float32,)
    # bf16 x, B, C: cssd_backward widens them (cssd_backward_saved takes fp32 only)
    if x_re.dtype == torch.bfloat16 and saved is None:
        code, okd = CSSD_BF16, (torch.bfloat16,)
    else:
        code, okd = CSSD_F32, f32
    p = {}
    for name, t, shp, dts in (("x_re", x_re, (Bsz, T, H, D), okd), ("x_im", x_im, (Bsz, T, H, D), okd),
                              ("B_re", B_re, (Bsz, T, H, N), okd), ("B_im", B_im, (Bsz, T, H, N), okd),
                              ("C_re", C_re, (Bsz, T, H, N), okd), ("C_im", C_im, (Bsz, T, H, N), okd),
                              ("dt", dt, (Bsz, T, H), f32), ("A_re", A_re, (H,), f32),
                              ("A_im", A_im, (H,), f32),
                              ("dy_re", dy[0], (Bsz, T, H, D), f32), ("dy_im", dy[1], (Bsz, T, H, D), f32)):
        p[name] = _check(t, name, shp, dts, dev)
    # y is not read by the library; a given y is still checked for its shape
    if y is None:
        p["y_re"] = p["y_im"] = None
    else:
        for name, t in (("y_re", y[0]), ("y_im", y[1])):
            p[name] = _check(t, name, (Bsz, T, H, D), f32, dev)
    p["Dskip"] = None if Dskip is None else _check(Dskip, "Dskip", (H,), f32, dev)
    hT = None if saved is None else saved[0]
    for key, pair, shp in (("h0", h0, (Bsz, H, N, D)), ("dhT", dhT, (Bsz, H, N, D)),
                           ("hT", hT, (Bsz, H, N, D))):
        p[key + "_re"] = None if pair is None else _check(pair[0], key + "_re", shp, f32, dev)
        p[key + "_im"] = None if pair is None else _check(pair[1], key + "_im", shp, f32, dev)
    e = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    g = {"dx_re": e(Bsz, T, H, D), "dx_im": e(Bsz, T, H, D), "dB_re": e(Bsz, T, H, N),
         "dB_im": e(Bsz, T, H, N), "dC_re": e(Bsz, T, H, N), "dC_im": e(Bsz, T, H, N),
         "ddt": e(Bsz, T, H), "dA_re": e(H), "dA_im": e(H),
         "dD": e(H) if Dskip is not None else None,
         "dh0_re": e(Bsz, H, N, D) if want_dh0 else None,
         "dh0_im": e(Bsz, H, N, D) if want_dh0 else None}
    need = cssd_backward_workspace_size(Bsz, T, H, D, N, chunk, code)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    ws_bytes = workspace.numel() * workspace.element_size()
    ptr = lambda t: None if t is None else t.data_ptr()
    head = (Bsz, T, H, D, N, int(chunk), code,
            p["x_re"], p["x_im"], p["B_re"], p["B_im"], p["C_re"], p["C_im"],
            p["dt"], p["A_re"], p["A_im"], p["Dskip"], p["h0_re"], p["h0_im"], p["y_re"], p["y_im"])
    tail = (p["dy_re"], p["dy_im"], p["dhT_re"], p["dhT_im"],
            *(ptr(g[k]) for k in ("dx_re", "dx_im", "dB_re", "dB_im", "dC_re", "dC_im", "ddt",
                                  "dA_re", "dA_im", "dD", "dh0_re", "dh0_im")),
            workspace.data_ptr(), ws_bytes, _stream_ptr(stream, dev))
    if saved is None:
        st, name = lib.cssd_backward(*head, *tail), "cssd_backward"
    else:
        st, name = lib.cssd_backward_saved(*head, p["hT_re"], p["hT_im"], *tail), "cssd_backward_saved"
    if st != CSSD_OK:
        raise CSSDError(st, name)
    return g


def _step_ptrs(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h, Bsz, H, N, D, out):
    """Checked pointers of the decode entry points (h = (h_re, h_im) or None)."""
    torch = _torch()
    dev = x_re.device
    f32 = (torch.float32,)
    p = {}
    items = [("x_re", x_re, (Bsz, H, D)), ("x_im", x_im, (Bsz, H, D)),
             ("B_re", B_re, (Bsz, H, N)), ("B_im", B_im, (Bsz, H, N)),
             ("C_re", C_re, (Bsz, H, N)), ("C_im", C_im, (Bsz, H, N)),
             ("dt", dt, (Bsz, H)), ("A_re", A_re, (H,)), ("A_im", A_im, (H,))]
    if h is not None:
        items += [("h_re", h[0], (Bsz, H, N, D)), ("h_im", h[1], (Bsz, H, N, D))]
    for name, t, shp in items:
        p[name] = _check(t, name, shp, f32, dev)
    p["Dskip"] = None if Dskip is None else _check(Dskip, "Dskip", (H,), f32, dev)
    if out is None:
        y_re = torch.empty((Bsz, H, D), dtype=torch.float32, device=dev)
        y_im = torch.empty_like(y_re)
    else:
        y_re, y_im = out
    p["y_re"] = _check(y_re, "y_re", (Bsz, H, D), f32, dev)
    p["y_im"] = _check(y_im, "y_im", (Bsz, H, D), f32, dev)
    return p, (y_re, y_im), dev


@_on_stream
def cssd_step(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h_re, h_im, *,
              out=None, stream=None):
    """One decode token for all (batch, head); the state (h_re, h_im) is updated
    in place.  x_*: (B,H,D); B_*, C_*: (B,H,N); dt: (B,H); A_*: (H,); Dskip: (H,)
    or None; h_*: (B,H,N,D).  All float32.  Returns (y_re, y_im), each (B,H,D)."""
    lib = load_library()
    Bsz, H, N, D = h_re.shape
    p, y, dev = _step_ptrs(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip,
                           (h_re, h_im), Bsz, H, N, D, out)
    st = lib.cssd_step(Bsz, H, D, N, p["x_re"], p["x_im"], p["B_re"], p["B_im"], p["C_re"],
                       p["C_im"], p["dt"], p["A_re"], p["A_im"], p["Dskip"], p["h_re"],
                       p["h_im"], p["y_re"], p["y_im"], _stream_ptr(stream, dev))
    if st != CSSD_OK:
        raise CSSDError(st, "cssd_step")
    return y


@_on_stream
def cssd_step_n(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, h_re, h_im, nsteps,
                *, out=None, stream=None):
    """nsteps decode steps that all receive the same input, applied at once; the
    state is updated in place and the nsteps-th output is returned.  Arguments
    as cssd_step, plus nsteps >= 1."""
    lib = load_library()
    Bsz, H, N, D = h_re.shape
    p, y, dev = _step_ptrs(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip,
                           (h_re, h_im), Bsz, H, N, D, out)
    st = lib.cssd_step_n(Bsz, H, D, N, int(nsteps), p["x_re"], p["x_im"], p["B_re"], p["B_im"],
                         p["C_re"], p["C_im"], p["dt"], p["A_re"], p["A_im"], p["Dskip"],
                         p["h_re"], p["h_im"], p["y_re"], p["y_im"], _stream_ptr(stream, dev))
    if st != CSSD_OK:
        raise CSSDError(st, "cssd_step_n")
    return y


@_on_stream
def cssd_step_infinite(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, *,
                       out=None, stream=None):
    """The stationary output of an endless constant input (no state).  Arguments
    as cssd_step without the state; returns (y_re, y_im), each (B,H,D)."""
    lib = load_library()
    Bsz, H, D = x_re.shape
    N = B_re.shape[-1]
    p, y, dev = _step_ptrs(x_re, x_im, B_re, B_im, C_re, C_im, dt, A_re, A_im, Dskip, None,
                           Bsz, H, N, D, out)
    st = lib.cssd_step_infinite(Bsz, H, D, N, p["x_re"], p["x_im"], p["B_re"], p["B_im"],
                                p["C_re"], p["C_im"], p["dt"], p["A_re"], p["A_im"], p["Dskip"],
                                p["y_re"], p["y_im"], _stream_ptr(stream, dev))
    if st != CSSD_OK:
        raise CSSDError(st, "cssd_step_infinite")
    return y


@_on_stream
def cssd_phase_scan(phi, u, b_re, b_im, psi0=None, *, chunk: int = 0, return_state: bool = True,
                    out=None, workspace=None, stream=None):
    """Per-coordinate scan psi_t = sigmoid(u_t) (1 + i phi_t) / (1 - i phi_t) psi_{t-1} + b_t
    (see include/cssd.h).

    phi, u, b_re, b_im: (B,T,H,N) float32; psi0: (psi0_re, psi0_im) each (B,H,N)
    float32, or None.  out: optional (psi_re, psi_im[, psiT_re, psiT_im]).  chunk:
    segment length, 0 = the library's choice.  Returns (psi_re, psi_im, psiT_re,
    psiT_im) (the last two None if not return_state)."""
    torch = _torch()
    lib = load_library()
    dev = phi.device
    Bsz, T, H, N = phi.shape
    f32 = (torch.float32,)
    p = {}
    for name, t in (("phi", phi), ("u", u), ("b_re", b_re), ("b_im", b_im)):
        p[name] = _check(t, name, (Bsz, T, H, N), f32, dev)
    if psi0 is not None:
        p["psi0_re"] = _check(psi0[0], "psi0_re", (Bsz, H, N), f32, dev)
        p["psi0_im"] = _check(psi0[1], "psi0_im", (Bsz, H, N), f32, dev)
    else:
        p["psi0_re"] = p["psi0_im"] = None
    if out is not None:
        psi_re, psi_im = out[0], out[1]
        psiT_re, psiT_im = (out[2], out[3]) if (return_state and len(out) >= 4) else (None, None)
    else:
        psi_re = torch.empty((Bsz, T, H, N), dtype=torch.float32, device=dev)
        psi_im = torch.empty_like(psi_re)
        psiT_re = psiT_im = None
    if return_state and psiT_re is None:
        psiT_re = torch.empty((Bsz, H, N), dtype=torch.float32, device=dev)
        psiT_im = torch.empty_like(psiT_re)
    p["psi_re"] = _check(psi_re, "psi_re", (Bsz, T, H, N), f32, dev)
    p["psi_im"] = _check(psi_im, "psi_im", (Bsz, T, H, N), f32, dev)
    p["psiT_re"] = None if psiT_re is None else _check(psiT_re, "psiT_re", (Bsz, H, N), f32, dev)
    p["psiT_im"] = None if psiT_im is None else _check(psiT_im, "psiT_im", (Bsz, H, N), f32, dev)
    need = cssd_phase_scan_workspace_size(Bsz, T, H, N, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.cssd_phase_scan(Bsz, T, H, N, int(chunk), p["phi"], p["u"], p["b_re"], p["b_im"],
                             p["psi0_re"], p["psi0_im"], p["psi_re"], p["psi_im"],
                             p["psiT_re"], p["psiT_im"], workspace.data_ptr(), ws_bytes,
                             _stream_ptr(stream, dev))
    if st != CSSD_OK:
        raise CSSDError(st, "cssd_phase_scan")
    return psi_re, psi_im, psiT_re, psiT_im


@_on_stream
def cssd_born_attention(q_re, q_im, k_re, k_im, v_re, v_im, tau=None, *, out=None, stream=None):
    """Causal Born attention (see include/cssd.h): psi_i = sum_{j<=i} s_ij v_j /
    sum_{j<=i} s_ij with s_ij = |<q_i|k_j>|^2 / (D tau_i).

    q_*, k_*, v_*: (B,T,H,D), all float32 or all bfloat16 (the bf16-input kernel);
    tau: (B,T,H) float32 or None.  out: optional (out_re, out_im) float32.
    Returns (out_re, out_im), each (B,T,H,D) float32."""
    torch = _torch()
    lib = load_library()
    dev = q_re.device
    Bsz, T, H, D = q_re.shape
    if q_re.dtype == torch.float32:
        code, okd = CSSD_F32, (torch.float32,)
    elif q_re.dtype == torch.bfloat16:
        code, okd = CSSD_BF16, (torch.bfloat16,)
    else:
        raise TypeError("q/k/v planes must be float32 or bfloat16")
    f32 = (torch.float32,)
    p = {}
    for name, t in (("q_re", q_re), ("q_im", q_im), ("k_re", k_re), ("k_im", k_im),
                    ("v_re", v_re), ("v_im", v_im)):
        p[name] = _check(t, name, (Bsz, T, H, D), okd, dev)
    p["tau"] = None if tau is None else _check(tau, "tau", (Bsz, T, H), f32, dev)
    if out is None:
        out = (torch.empty((Bsz, T, H, D), dtype=torch.float32, device=dev),
               torch.empty((Bsz, T, H, D), dtype=torch.float32, device=dev))
    p["out_re"] = _check(out[0], "out_re", (Bsz, T, H, D), f32, dev)
    p["out_im"] = _check(out[1], "out_im", (Bsz, T, H, D), f32, dev)
    st = lib.cssd_born_attention(Bsz, T, H, D, code, p["q_re"], p["q_im"], p["k_re"],
                                 p["k_im"], p["v_re"], p["v_im"], p["tau"], p["out_re"],
                                 p["out_im"], _stream_ptr(stream, dev))
    if st != CSSD_OK:
        raise CSSDError(st, "cssd_born_attention")
    return out[0], out[1]


class profile:
    """Context manager around the library's per-kernel event timing.

    with profile() as prof: ...;  prof.ms[name], prof.launches[name]
    (the events are recorded on the stream each kernel is launched on)."""

    def __enter__(self):
        lib = load_library()
        lib.cssd_profile_read(None, None, 0)  # drop anything pending
        lib.cssd_profile_enable(1)
        self.ms, self.launches = {}, {}
        return self

    def read(self):
        lib = load_library()
        n = len(KERNEL_NAMES)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        k = lib.cssd_profile_read(ms, cnt, n)
        if k < 0:
            raise CSSDError(-k, "cssd_profile_read")
        for i, name in enumerate(KERNEL_NAMES):
            self.ms[name] = self.ms.get(name, 0.0) + ms[i]
            self.launches[name] = self.launches.get(name, 0) + cnt[i]
        return self

    def __exit__(self, *exc):
        self.read()
        load_library().cssd_profile_enable(0)
        return False
