"""The C ABI of libcssd.so on the host (no GPU needed, no kernel launched).

Every call here fails validation before anything is enqueued, so none of them
touches a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cssd.h")


@pytest.fixture(scope="module")
def lib():
    import complex_valued_state_amd as cssd
    if not os.path.exists(cssd.LIB_PATH):
        from complex_valued_state_amd.build import build_library
        build_library()
    return cssd.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cssd_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("cssd_forward", "cssd_backward", "cssd_backward_saved",
                     "cssd_backward_workspace_size", "cssd_backward_workspace_size_dtype",
                     "cssd_step", "cssd_step_n", "cssd_step_infinite", "cssd_phase_scan",
                     "cssd_phase_scan_workspace_size", "cssd_born_attention",
                     "cssd_forward_workspace_size", "cssd_status_string", "cssd_version"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {lib._name}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_version_and_status_strings(lib):
    assert lib.cssd_version() == 108
    for st in range(6):
        assert lib.cssd_status_string(st)
    assert b"unknown" in lib.cssd_status_string(99)


def _ws(lib, *shape):
    n = ctypes.c_size_t(0)
    st = lib.cssd_forward_workspace_size(*shape, ctypes.byref(n))
    return st, n.value


def _align(v):
    return (v + 255) // 256 * 256


def test_workspace_size_layout(lib):
    # B, T, H, D, N, C with a partial last chunk
    B, T, H, D, N, C = 2, 100, 3, 32, 64, 16
    st, got = _ws(lib, B, T, H, D, N, C)
    assert st == 0
    nC = -(-T // C)
    P = B * H * nC * C
    want = 0
    for nbytes in (8 * P, 8 * P, 4 * P, 4 * P, 4 * P, 4 * P, 4 * B * H * nC, 4 * B * H * nC,
                   4 * B * H * nC * N * D, 4 * B * H * nC * N * D):  # acs, e, w, cd, S_c/H_c
        want = _align(want + nbytes)
    assert got == want


def test_workspace_never_holds_the_segment_matrix(lib):
    """A materialised C x C segment matrix would cost 8*B*T*H*C bytes and grow
    with C ("SSD Theory", section 5: 268 MB at B16 T2048 H16 C64); the
    workspace instead shrinks as C grows (one state per chunk)."""
    assert 8 * 16 * 2048 * 16 * 64 == 268435456
    sizes = [_ws(lib, 16, 2048, 16, 64, 64, c)[1] for c in (16, 32, 64, 128)]
    assert sizes == sorted(sizes, reverse=True)


@pytest.mark.parametrize("shape,status", [
    ((-1, 64, 2, 16, 16, 16), 1), ((1, -1, 2, 16, 16, 16), 1), ((1, 64, -1, 16, 16, 16), 1),
    ((0, 64, 2, 24, 16, 16), 2), ((1, 0, 2, 16, 16, 0), 1),
    ((1, 64, 2, 24, 16, 16), 2), ((1, 64, 2, 16, 256, 16), 2), ((1, 64, 2, 16, 16, 48), 2),
    ((1, 64, 2, 16, 16, 8), 2), ((1 << 20, 1 << 20, 64, 128, 128, 64), 2),
    # under 2^31 elements in all, but one chunk's rows of a plane span more than 4 GB
    ((1, 64, 300000, 64, 64, 64), 2),
])
def test_workspace_size_rejects(lib, shape, status):
    assert _ws(lib, *shape)[0] == status


@pytest.mark.parametrize("shape", [(0, 64, 2, 16, 16, 16), (2, 0, 3, 32, 64, 16),
                                   (2, 100, 0, 32, 64, 16), (0, 0, 0, 128, 128, 128)])
def test_empty_problems_need_no_workspace(lib, shape):
    assert _ws(lib, *shape) == (0, 0)
    n = ctypes.c_size_t(7)
    assert lib.cssd_backward_workspace_size(*shape, ctypes.byref(n)) == 0 and n.value == 0


def _fwd(lib, shape=(1, 64, 2, 16, 16, 16), dtype=0, ptrs=None, ws=None, ws_bytes=1 << 30):
    # fake, aligned, never-dereferenced addresses; validation fails before any launch
    base = 0x10000000
    p = {k: base + 0x100000 * i for i, k in enumerate(
        ["x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt", "A_re", "A_im", "D",
         "h0_re", "h0_im", "y_re", "y_im", "hT_re", "hT_im"])}
    p.update(ptrs or {})
    return lib.cssd_forward(*shape, dtype, p["x_re"], p["x_im"], p["B_re"], p["B_im"], p["C_re"],
                            p["C_im"], p["dt"], p["A_re"], p["A_im"], p["D"], p["h0_re"],
                            p["h0_im"], p["y_re"], p["y_im"], p["hT_re"], p["hT_im"],
                            ws, ws_bytes, None)


def test_forward_validation(lib):
    # missing workspace (all pointers otherwise plausible) -> workspace error, no launch
    assert _fwd(lib, ws=None) == 3
    assert _fwd(lib, ws=0x20000000, ws_bytes=16) == 3
    assert _fwd(lib, ws=0x20000010) == 3                      # misaligned workspace
    assert _fwd(lib, ptrs={"x_re": None}, ws=0x20000000) == 1
    assert _fwd(lib, ptrs={"y_im": None}, ws=0x20000000) == 1
    assert _fwd(lib, ptrs={"B_im": 0x10000004}, ws=0x20000000) == 1  # misaligned vector operand
    assert _fwd(lib, ptrs={"dt": 0x10000002}, ws=0x20000000) == 1    # misaligned scalar operand
    assert _fwd(lib, ptrs={"h0_re": 0x10000008}, ws=0x20000000) == 1
    assert _fwd(lib, ptrs={"h0_im": None}, ws=0x20000000) == 1     # half an initial state
    assert _fwd(lib, ptrs={"hT_re": None}, ws=0x20000000) == 1     # half a final state
    assert _fwd(lib, ptrs={"y_re": 0x10000000}, ws=0x20000000) == 1  # y aliases x
    assert _fwd(lib, dtype=7, ws=0x20000000) == 1
    assert _fwd(lib, shape=(1, 64, 2, 16, 16, 48), ws=0x20000000) == 2
    assert _fwd(lib, shape=(1, 64, 2, 0, 16, 16), ws=0x20000000) == 1


def test_step_validation(lib):
    base = 0x10000000
    ptrs = [base + 0x100000 * i for i in range(14)]
    args = ptrs[:10] + ptrs[10:14]
    assert lib.cssd_step(-1, 2, 16, 16, *args, None) == 1
    assert lib.cssd_step(1, 2, 20, 16, *args, None) == 2
    bad = list(args); bad[0] = None
    assert lib.cssd_step(1, 2, 16, 16, *bad, None) == 1
    bad = list(args); bad[12] = bad[10]      # y_re aliases h_re
    assert lib.cssd_step(1, 2, 16, 16, *bad, None) == 1
    bad = list(args); bad[10] = bad[0]       # state aliases x
    assert lib.cssd_step(1, 2, 16, 16, *bad, None) == 1


def test_step_n_and_infinite_validation(lib):
    base = 0x10000000
    ptrs = [base + 0x100000 * i for i in range(14)]
    ins, h, y = ptrs[:10], ptrs[10:12], ptrs[12:14]
    assert lib.cssd_step_n(1, 2, 16, 16, 0, *ins, *h, *y, None) == 1      # nsteps < 1
    assert lib.cssd_step_n(1, 2, 16, 16, -5, *ins, *h, *y, None) == 1
    assert lib.cssd_step_n(1, 2, 16, 24, 3, *ins, *h, *y, None) == 2      # N not supported
    assert lib.cssd_step_n(1, 2, 16, 16, 3, *ins, None, h[1], *y, None) == 1
    assert lib.cssd_step_infinite(-1, 2, 16, 16, *ins, *y, None) == 1
    assert lib.cssd_step_infinite(1, 2, 16, 48, *ins, *y, None) == 2
    bad = list(ins); bad[6] = None                                         # dt missing
    assert lib.cssd_step_infinite(1, 2, 16, 16, *bad, *y, None) == 1
    assert lib.cssd_step_infinite(1, 2, 16, 16, *ins, y[0], y[0], None) == 1  # y_re is y_im
    assert lib.cssd_step_infinite(1, 2, 16, 16, *ins, ins[0], y[1], None) == 1  # y aliases x
    misaligned = list(y); misaligned[0] = y[0] + 4
    assert lib.cssd_step_infinite(1, 2, 16, 16, *ins, *misaligned, None) == 1


def test_backward_validation(lib):
    import ctypes
    fw, bw = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.cssd_forward_workspace_size(2, 100, 3, 32, 64, 16, ctypes.byref(fw)) == 0
    assert lib.cssd_backward_workspace_size(2, 100, 3, 32, 64, 16, ctypes.byref(bw)) == 0
    assert bw.value > fw.value and bw.value % 256 == 0
    assert lib.cssd_backward_workspace_size(2, 100, 3, 32, 48, 16, ctypes.byref(bw)) == 2
    base = 0x10000000
    p = [base + 0x100000 * i for i in range(40)]
    ins = p[:10] + [None, None] + p[12:16]          # x..Dskip, h0 NULL, y, dy
    grads = p[20:30] + [p[30], None]                # dx..dD, dh0 half-NULL (bad)
    ws = 0x20000000
    args = lambda g, dt=0, shape=(1, 64, 2, 16, 16, 16): (
        *shape, dt, *ins, None, None, *g, ws, 1 << 30, None)
    assert lib.cssd_backward(*args(grads)) == 1          # dh0_re without dh0_im
    good = p[20:30] + [None, None]
    # bf16 inputs need the widened copies in the workspace: a workspace of exactly
    # the fp32 size is refused before anything is launched
    fsz, bsz = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.cssd_backward_workspace_size_dtype(1, 64, 2, 16, 16, 16, 0, ctypes.byref(fsz)) == 0
    assert lib.cssd_backward_workspace_size_dtype(1, 64, 2, 16, 16, 16, 1, ctypes.byref(bsz)) == 0
    assert lib.cssd_backward_workspace_size_dtype(1, 64, 2, 16, 16, 16, 2, ctypes.byref(bsz)) == 1
    short = lambda g: (1, 64, 2, 16, 16, 16, 1, *ins, None, None, *g, ws, fsz.value, None)
    assert lib.cssd_backward(*short(good)) == 3           # CSSD_ERR_WORKSPACE
    # y is not read and may be NULL: the pointer checks pass and the short
    # workspace is what is refused (nothing launched)
    noy = ins[:12] + [None, None] + ins[14:]
    for dt in (0, 1):
        assert lib.cssd_backward(1, 64, 2, 16, 16, 16, dt, *noy, None, None, *good, ws, 256,
                                 None) == 3
    assert lib.cssd_backward(*args(good, shape=(1, 64, 2, 16, 24, 16))) == 2
    bad = list(good); bad[0] = ins[0]                     # dx aliases x
    assert lib.cssd_backward(*args(bad)) == 1
    bad = list(good); bad[2] = bad[0]                     # dB aliases dx
    assert lib.cssd_backward(*args(bad)) == 1
    # the saved-state form: the forward's hT is needed with dhT, and may alias no output
    hT = [p[32], p[33]]
    sargs = lambda g, hT=hT, dhT=(None, None), shape=(1, 64, 2, 16, 16, 16): (
        *shape, 0, *ins[:14], *hT, *ins[14:], *dhT, *g, ws, 1 << 30, None)
    assert lib.cssd_backward_saved(*sargs(grads)) == 1
    assert lib.cssd_backward_saved(*sargs(good, hT=(None, None), dhT=(p[34], p[35]))) == 1
    assert lib.cssd_backward_saved(*sargs(good, hT=(p[32], None))) == 1
    assert lib.cssd_backward_saved(*sargs(good, hT=(p[32] + 4, p[33]))) == 1
    bad = list(good); bad[0] = hT[0]                      # dx aliases hT
    assert lib.cssd_backward_saved(*sargs(bad)) == 1
    assert lib.cssd_backward_saved(*sargs(good, shape=(1, 64, 2, 16, 24, 16))) == 2
    bf = lambda g: (1, 64, 2, 16, 16, 16, 1, *ins[:14], *hT, *ins[14:], None, None, *g, ws,
                    1 << 30, None)
    assert lib.cssd_backward_saved(*bf(good)) == 2        # bf16: no saved chunk states


def test_backward_workspace_size_dtype(lib):
    """bf16 inputs add the fp32 copies of x, B, C (two planes each, each rounded
    up to 256 bytes) to the fp32 workspace."""
    up = lambda v: (v + 255) // 256 * 256
    for shape in ((1, 64, 2, 16, 16, 16), (2, 100, 3, 32, 64, 16), (1, 257, 2, 64, 128, 64)):
        B, T, H, D, N, C = shape
        f, b, plain = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
        assert lib.cssd_backward_workspace_size(*shape, ctypes.byref(plain)) == 0
        assert lib.cssd_backward_workspace_size_dtype(*shape, 0, ctypes.byref(f)) == 0
        assert lib.cssd_backward_workspace_size_dtype(*shape, 1, ctypes.byref(b)) == 0
        assert f.value == plain.value
        assert b.value == f.value + 2 * up(4 * B * T * H * D) + 4 * up(4 * B * T * H * N)
    z = ctypes.c_size_t(7)
    assert lib.cssd_backward_workspace_size_dtype(0, 64, 2, 16, 16, 16, 1, ctypes.byref(z)) == 0
    assert z.value == 0                                  # an empty problem needs none
    assert lib.cssd_backward_workspace_size_dtype(1, 64, 2, 16, 16, 16, 1, None) == 1


def _phase_ws(lib, *shape):
    n = ctypes.c_size_t(0)
    st = lib.cssd_phase_scan_workspace_size(*shape, ctypes.byref(n))
    return st, n.value


def test_phase_scan_workspace_size(lib):
    # one pass over the sequence needs no workspace: batch x coordinates fill the chip
    assert _phase_ws(lib, 256, 1024, 16, 16, 0) == (0, 0)
    assert _phase_ws(lib, 4, 100, 3, 16, 200) == (0, 0)          # chunk >= seqlen
    # explicit segments of 16 steps: 7 segments, six fp32 planes of (B, 7, H*N)
    assert _phase_ws(lib, 2, 100, 4, 16, 16) == (0, 6 * _align(2 * 7 * 64 * 4))
    # automatic segments for a small batch are a multiple of 16 steps
    st, n = _phase_ws(lib, 1, 4096, 2, 8, 0)
    assert st == 0 and n > 0 and n % (6 * 256) == 0
    assert _phase_ws(lib, -1, 10, 1, 1, 0)[0] == 1
    assert _phase_ws(lib, 1, 10, 1, 0, 0)[0] == 1                # dstate 0
    assert _phase_ws(lib, 0, 10, 1, 1, 0) == (0, 0)              # empty problems
    assert _phase_ws(lib, 3, 0, 2, 4, 16) == (0, 0)
    assert _phase_ws(lib, 1, 10, 1, 1, -1)[0] == 1
    assert _phase_ws(lib, 1 << 20, 1 << 20, 1, 2, 0)[0] == 2     # 2^41 elements per plane
    assert lib.cssd_phase_scan_workspace_size(1, 10, 1, 1, 0, None) == 1


def test_phase_scan_validation(lib):
    base = 0x10000000
    p = [base + 0x100000 * i for i in range(12)]
    ins, psi0, psi, psiT = p[:4], p[4:6], p[6:8], p[8:10]
    ws = 0x20000000
    call = lambda ins=ins, psi0=psi0, psi=psi, psiT=psiT, shape=(2, 64, 2, 16, 16), wsb=1 << 30, w=ws: \
        lib.cssd_phase_scan(*shape, *ins, *psi0, *psi, *psiT, w, wsb, None)
    assert call(shape=(-1, 64, 2, 16, 16)) == 1
    assert call(shape=(2, 64, 2, 16, -1)) == 1
    bad = list(ins); bad[1] = None                                  # u missing
    assert call(ins=bad) == 1
    bad = list(ins); bad[0] += 2                                    # phi misaligned
    assert call(ins=bad) == 1
    assert call(psi0=[psi0[0], None]) == 1                          # half a state
    assert call(psiT=[None, psiT[1]]) == 1
    assert call(psi=[ins[2], psi[1]]) == 1                          # psi aliases b
    assert call(psi=[psi[0], psi[0]]) == 1
    assert call(psi=[psi0[1], psi[1]]) == 1                         # psi aliases psi0
    assert call(psiT=[ins[0], psiT[1]]) == 1                        # psiT aliases phi
    assert call(psiT=[psi0[1], psi0[0]]) == 1                       # planes swapped
    assert call(psiT=[psi[0], psiT[1]]) == 1
    assert call(w=None) == 3                                        # segments need workspace
    assert call(wsb=16) == 3
    assert call(w=ws + 64) == 3


def test_born_attention_validation(lib):
    base = 0x10000000
    p = [base + 0x100000 * i for i in range(10)]
    ins, tau, out = p[:6], p[6], p[7:9]
    call = lambda shape=(2, 100, 3, 16), dt=0, ins=ins, tau=tau, out=out: \
        lib.cssd_born_attention(*shape, dt, *ins, tau, *out, None)
    assert call(shape=(-1, 100, 3, 16)) == 1
    assert call(shape=(2, -1, 3, 16)) == 1
    assert call(shape=(2, 100, 3, 24)) == 2                  # D not supported
    assert call(shape=(2, 100, 3, 128)) == 2
    assert call(dt=7) == 1
    bad = list(ins); bad[3] = None                           # k_im missing
    assert call(ins=bad) == 1
    bad = list(ins); bad[0] += 4                             # q_re misaligned
    assert call(ins=bad) == 1
    assert call(tau=tau + 2) == 1                            # tau misaligned
    assert call(out=[ins[4], out[1]]) == 1                   # out aliases v
    assert call(out=[out[0], tau]) == 1                      # out aliases tau
    assert call(out=[out[0], out[0]]) == 1
    assert call(out=[None, out[1]]) == 1


def test_profiler_without_launches(lib):
    import complex_valued_state_amd as cssd
    with cssd.profile() as prof:
        pass
    assert set(prof.ms) == set(cssd.KERNEL_NAMES)
    assert all(v == 0 for v in prof.launches.values())
    assert lib.cssd_kernel_name(3) == b"k_chunk_scan" and lib.cssd_kernel_name(19) is None
    assert lib.cssd_kernel_name(17) == b"k_scan_fused" and lib.cssd_kernel_name(18) == b"k_widen"
    assert lib.cssd_kernel_name(16) == b"k_fill"
    assert lib.cssd_kernel_name(14) == b"k_state_scan"
    assert lib.cssd_kernel_name(15) == b"k_state_scan_adj"
    assert lib.cssd_kernel_name(13) == b"k_bwd_db" and lib.cssd_kernel_name(6) == b"k_bwd_dx"
    assert lib.cssd_kernel_name(12) == b"k_born"
    assert lib.cssd_kernel_name(5) == b"k_step_infinite"
    assert lib.cssd_kernel_name(11) == b"k_phase_out"


def test_empty_problems_validate_and_enqueue_nothing(lib):
    """Empty problems (batch, seqlen or nheads 0): arrays with a zero extent may be
    NULL.  The calls below have nothing non-empty to write, so they return CSSD_OK
    without a launch (which is why they run without a GPU); bad pairs of the
    state pointers are still rejected."""
    n = None
    # forward: all 16 arrays NULL, no workspace
    for shape in [(0, 64, 2, 16, 16, 16), (2, 0, 3, 32, 64, 16), (2, 64, 0, 16, 16, 16)]:
        assert lib.cssd_forward(*shape, 0, *[n] * 16, n, 0, n) == 0
        assert lib.cssd_forward(*shape, 1, *[n] * 16, n, 0, n) == 0
        assert lib.cssd_forward(*shape, 5, *[n] * 16, n, 0, n) == 1      # bad dtype
    base = 0x10000000
    h0, hT = [base, base + 0x100000], [base + 0x200000, base + 0x300000]
    # T = 0 with hT requested launches the copy; here only the validation is run
    shape = (2, 0, 3, 32, 64, 16)
    assert lib.cssd_forward(*shape, 0, *[n] * 10, h0[0], n, *[n] * 2, *hT, n, 0, n) == 1
    assert lib.cssd_forward(*shape, 0, *[n] * 10, *h0, *[n] * 2, hT[0], n, n, 0, n) == 1
    assert lib.cssd_forward(*shape, 0, *[n] * 10, *h0, *[n] * 2, h0[0], hT[1], n, 0, n) == 1
    assert lib.cssd_forward(*shape, 0, *[n] * 10, *h0, *[n] * 2, hT[0] + 8, hT[1], n, 0, n) == 1
    # with batch 0 the state planes are empty too: nothing to launch
    assert lib.cssd_forward(0, 64, 2, 16, 16, 16, 0, *[n] * 10, *h0, *[n] * 2, *hT, n, 0, n) == 0
    # backward: no heads -> nothing at all; heads but no dA -> invalid
    assert lib.cssd_backward(2, 64, 0, 16, 16, 16, 0, *[n] * 18, *[n] * 12, n, 0, n) == 0
    assert lib.cssd_backward(2, 0, 3, 16, 16, 16, 0, *[n] * 18, *[n] * 12, n, 0, n) == 1
    assert lib.cssd_backward(2, 0, 3, 16, 16, 16, 1, *[n] * 18, *[n] * 12, n, 0, n) == 1  # bf16 alike
    # decode with no rows or heads; nsteps is still checked
    assert lib.cssd_step(0, 2, 16, 16, *[n] * 14, n) == 0
    assert lib.cssd_step_n(3, 0, 16, 16, 4, *[n] * 14, n) == 0
    assert lib.cssd_step_n(0, 2, 16, 16, 0, *[n] * 14, n) == 1
    assert lib.cssd_step_infinite(0, 2, 16, 16, *[n] * 12, n) == 0
    assert lib.cssd_step(0, 2, 16, 24, *[n] * 14, n) == 2
    # phase scan with batch 0 (empty psiT), Born attention of nothing
    assert lib.cssd_phase_scan(0, 64, 2, 16, 0, *[n] * 10, n, 0, n) == 0
    assert lib.cssd_phase_scan(0, 64, 2, 16, 0, *[n] * 4, base, n, *[n] * 4, n, 0, n) == 1
    for shape in [(0, 100, 3, 16), (2, 0, 3, 32), (2, 100, 0, 64)]:
        assert lib.cssd_born_attention(*shape, 0, *[n] * 7, n, n, n) == 0
    assert lib.cssd_born_attention(2, 0, 3, 24, 0, *[n] * 7, n, n, n) == 2


def test_missing_library_raises(tmp_path, monkeypatch):
    """No fallback: without the built library every call fails loudly."""
    import complex_valued_state_amd._binding as bd
    monkeypatch.setattr(bd, "_lib", None)
    monkeypatch.setattr(bd, "LIB_PATH", str(tmp_path / "libcssd.so"))
    with pytest.raises(RuntimeError, match="not built"):
        bd.cssd_forward_workspace_size(1, 64, 2, 16, 16, 16)


def test_product_never_reaches_the_oracle():
    """The package (binding and HIP sources) neither imports, includes nor names the
    CPU oracle: it is test infrastructure only."""
    import ast
    import glob
    pkg = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "complex_valued_state_amd")
    for f in glob.glob(os.path.join(pkg, "*.py")):
        tree = ast.parse(open(f).read())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                assert not any(a.name.split(".")[0] == "oracle" for a in node.names), f
            if isinstance(node, ast.ImportFrom):
                assert (node.module or "").split(".")[0] != "oracle", f
    for f in glob.glob(os.path.join(pkg, "csrc", "*")):
        assert "oracle" not in open(f).read().lower(), f
