"""HIP graph capture of the library's calls (needs an MI355X).

The entry points never allocate, copy, clear or synchronise: each enqueues its
kernels on the caller's stream.  So a caller may capture them in a graph and
replay it.  Each test captures once, replays several times with the program's
own eager work (overwriting the outputs, resetting the state) and a
synchronisation between replays, and checks every replay bit for bit against
the eager result.
"""
import numpy as np
import pytest

import cssd_workloads as wl
from gpu_util import dev_inputs, log

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def test_training_step_graph_replays():
    """Forward on a backward-sized workspace, then the backward on the states it
    saved: one captured graph, replayed."""
    import torch
    import complex_valued_state_amd as cssd
    Bsz, T, H, D, N, C = 2, 300, 3, 64, 64, 64
    log("graph: forward + backward_saved")
    inp = wl.random_forward(81, Bsz, T, H, D, N, C, with_h0=True)
    d = dev_inputs(inp)
    ins = (d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"], d["dt"], d["A_re"],
           d["A_im"], d["Dskip"], d["h0"])
    g = torch.Generator(device="cuda:0").manual_seed(82)
    dy = [torch.randn((Bsz, T, H, D), generator=g, device="cuda:0") for _ in range(2)]
    dhT = [torch.randn((Bsz, H, N, D), generator=g, device="cuda:0") for _ in range(2)]
    ws = torch.empty(cssd.cssd_backward_workspace_size(Bsz, T, H, D, N, C), dtype=torch.uint8,
                     device="cuda:0")
    y = [torch.empty((Bsz, T, H, D), device="cuda:0") for _ in range(2)]
    hT = [torch.empty((Bsz, H, N, D), device="cuda:0") for _ in range(2)]

    def step():
        cssd.cssd_forward(*ins, chunk=C, out=(*y, *hT), workspace=ws)
        return cssd.cssd_backward_saved(*ins, tuple(y), tuple(hT), dy, dhT, chunk=C,
                                        workspace=ws)

    ref_g = step()
    torch.cuda.synchronize()
    ref = {"y_re": y[0].clone(), "y_im": y[1].clone(), "hT_re": hT[0].clone(),
           "hT_im": hT[1].clone(), **{k: v.clone() for k, v in ref_g.items() if v is not None}}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gg = step()
    for rep in range(REPLAYS):
        for t in (*y, *hT, *(v for v in gg.values() if v is not None)):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {"y_re": y[0], "y_im": y[1], "hT_re": hT[0], "hT_im": hT[1],
               **{k: v for k, v in gg.items() if v is not None}}
        for k, v in ref.items():
            assert torch.equal(got[k], v), (rep, k)


def test_bf16_training_step_graph_replays():
    """bf16 x, B, C: the one-kernel forward, then the backward, which widens the
    bf16 planes in its workspace and reads no y: one captured graph, replayed."""
    import torch
    import complex_valued_state_amd as cssd
    Bsz, T, H, D, N, C = 2, 300, 3, 64, 64, 64
    log("graph: bf16 forward + backward")
    inp = wl.random_forward(83, Bsz, T, H, D, N, C, with_h0=True, in_dtype="bf16")
    d = dev_inputs(inp)
    ins = (d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"], d["dt"], d["A_re"],
           d["A_im"], d["Dskip"], d["h0"])
    g = torch.Generator(device="cuda:0").manual_seed(84)
    dy = [torch.randn((Bsz, T, H, D), generator=g, device="cuda:0") for _ in range(2)]
    dhT = [torch.randn((Bsz, H, N, D), generator=g, device="cuda:0") for _ in range(2)]
    ws_f = torch.empty(cssd.cssd_forward_workspace_size(Bsz, T, H, D, N, C), dtype=torch.uint8,
                       device="cuda:0")
    ws_b = torch.empty(cssd.cssd_backward_workspace_size(Bsz, T, H, D, N, C, cssd.CSSD_BF16),
                       dtype=torch.uint8, device="cuda:0")
    y = [torch.empty((Bsz, T, H, D), device="cuda:0") for _ in range(2)]
    hT = [torch.empty((Bsz, H, N, D), device="cuda:0") for _ in range(2)]

    def step():
        cssd.cssd_forward(*ins, chunk=C, out=(*y, *hT), workspace=ws_f)
        return cssd.cssd_backward(*ins, None, dy, dhT, chunk=C, workspace=ws_b)

    ref_g = step()
    torch.cuda.synchronize()
    ref = {"y_re": y[0].clone(), "y_im": y[1].clone(), "hT_re": hT[0].clone(),
           "hT_im": hT[1].clone(), **{k: v.clone() for k, v in ref_g.items() if v is not None}}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gg = step()
    for rep in range(REPLAYS):
        for t in (*y, *hT, *(v for v in gg.values() if v is not None)):
            t.fill_(float("nan"))
        ws_b.fill_(255)  # the widened planes are rewritten by every replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {"y_re": y[0], "y_im": y[1], "hT_re": hT[0], "hT_im": hT[1],
               **{k: v for k, v in gg.items() if v is not None}}
        for k, v in ref.items():
            assert torch.equal(got[k], v), (rep, k)


def test_bf16_forward_two_stream_split_graph_replays():
    """bf16 inputs with more sequences than CUs (and at most twice as many): the
    forward runs whole and half-width workgroups on the caller's stream and a
    second stream joined through events.  Captured into a graph and replayed, it
    gives the eager result bit for bit, and the eager result meets the oracle."""
    import torch
    import complex_valued_state_amd as cssd
    from gpu_util import oracle_forward, rel_err
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Bsz, T, H, D, N, C = 1, 100, cus + 9, 64, 64, 64
    log(f"graph: bf16 forward, {Bsz * H} sequences on {cus} CUs")
    inp = wl.random_forward(85, Bsz, T, H, D, N, C, with_h0=True, in_dtype="bf16")
    d = dev_inputs(inp)
    ins = (d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"], d["dt"], d["A_re"],
           d["A_im"], d["Dskip"], d["h0"])
    ws = torch.empty(cssd.cssd_forward_workspace_size(Bsz, T, H, D, N, C), dtype=torch.uint8,
                     device="cuda:0")
    y = [torch.empty((Bsz, T, H, D), device="cuda:0") for _ in range(2)]
    hT = [torch.empty((Bsz, H, N, D), device="cuda:0") for _ in range(2)]

    def step():
        cssd.cssd_forward(*ins, chunk=C, out=(*y, *hT), workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (*y, *hT)]
    yr, hr = oracle_forward(inp)
    to = lambda a, b: a.double().cpu().numpy() + 1j * b.double().cpu().numpy()
    assert rel_err(to(y[0], y[1]), yr) <= 2e-2 and rel_err(to(hT[0], hT[1]), hr) <= 2e-2
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(REPLAYS):
        for t in (*y, *hT):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip((*y, *hT), ref):
            assert torch.equal(t, r), rep


def test_decode_step_graph_replays():
    """cssd_step updates its state in place: the state is reset eagerly before
    each replay, and the replay must give the eager step's state and output."""
    import torch
    import complex_valued_state_amd as cssd
    B, H, D, N = 8, 6, 64, 128
    log("graph: decode step")
    st = wl.decode_step(83, 0, B, H, D, N)
    a_re, a_im, dk = (_dev(v) for v in wl.decode_params(83, H))
    args = [_dev(getattr(st, f)) for f in ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt")]
    rng = np.random.default_rng(84)
    h0 = [_dev(rng.standard_normal((B, H, N, D)).astype(np.float32)) for _ in range(2)]
    h = [t.clone() for t in h0]
    y = [torch.empty((B, H, D), device="cuda:0") for _ in range(2)]

    def step():
        cssd.cssd_step(*args, a_re, a_im, dk, h[0], h[1], out=tuple(y))

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (*h, *y)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(REPLAYS):
        h[0].copy_(h0[0])
        h[1].copy_(h0[1])
        y[0].fill_(float("nan"))
        y[1].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (got, want) in enumerate(zip((*h, *y), ref)):
            assert torch.equal(got, want), (rep, k)


def test_profiler_on_during_capture_counts_eager_launches_only():
    """With the per-kernel profiler on, a forward captured into a graph gets no
    event brackets: the replays are neither timed nor counted, the captured graph
    replays bit-identically to an eager call, and the read afterwards succeeds
    and counts exactly the eager calls made while profiling."""
    import torch
    import complex_valued_state_amd as cssd
    Bsz, T, H, D, N, C = 2, 200, 3, 64, 64, 64
    log("graph: forward captured with the profiler on")
    inp = wl.random_forward(85, Bsz, T, H, D, N, C, with_h0=True)
    d = dev_inputs(inp)
    ins = (d["x_re"], d["x_im"], d["B_re"], d["B_im"], d["C_re"], d["C_im"], d["dt"], d["A_re"],
           d["A_im"], d["Dskip"], d["h0"])
    ws = torch.empty(cssd.cssd_forward_workspace_size(Bsz, T, H, D, N, C), dtype=torch.uint8,
                     device="cuda:0")
    out = [torch.empty((Bsz, T, H, D), device="cuda:0") for _ in range(2)] + \
          [torch.empty((Bsz, H, N, D), device="cuda:0") for _ in range(2)]
    call = lambda: cssd.cssd_forward(*ins, chunk=C, out=tuple(out), workspace=ws)
    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in out]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with cssd.profile() as prof:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        for rep in range(REPLAYS):
            for t in out:
                t.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for k, (got, want) in enumerate(zip(out, ref)):
                assert torch.equal(got, want), (rep, k)
        call()
        call()
        torch.cuda.synchronize()
    log(f"  launches counted: {prof.launches['k_cumsum']}, {prof.launches['k_state_scan']}, "
        f"{prof.launches['k_chunk_scan']}")
    for k in ("k_cumsum", "k_state_scan", "k_chunk_scan"):
        assert prof.launches[k] == 2, (k, prof.launches[k])
        assert prof.ms[k] > 0.0
