"""Micro-kernels for the design's hardware assumptions (test infrastructure):
the achievable fp32 matrix-core rate and the issue of vector-ALU and matrix-core
instructions of one wave.  ``build()`` compiles ``mfma_probe.hip`` with hipcc for
gfx950 into ``libmfma_probe.so`` beside it; ``measure()`` runs it on cuda:0."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mfma_probe.hip")
LIB = os.path.join(HERE, "libmfma_probe.so")
PEAK_FP32_MFMA_TFLOPS = 157.3


def build() -> str:
    hipcc = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def measure(iters: int = 20000, reps: int = 3) -> dict:
    """Times the probes on cuda:0 with HIP events.  One workgroup of four waves
    per CU (one wave per SIMD); for the MFMA probe also two and four waves per
    SIMD; and two workgroups per CU, one of each mix.  Returns the rates and the
    ratios of the mixed runs to the separate ones."""
    import torch
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built: run tests/gpu_probes.build() first")
    lib = ctypes.CDLL(LIB)
    lib.probe_launch.restype = ctypes.c_int
    lib.probe_launch.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream(dev)

    def run(kind, blocks, threads=256):
        out = torch.empty(blocks * threads, device=dev)
        best = None
        for _ in range(reps + 1):  # the first run is a warm-up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.probe_launch(kind, blocks, threads, iters, out.data_ptr(),
                                  ctypes.c_void_p(stream.cuda_stream))
            e1.record(stream)
            if rc != 0:
                raise RuntimeError(f"probe_launch({kind}) returned {rc}")
            torch.cuda.synchronize(dev)
            t = e0.elapsed_time(e1)
            best = t if best is None else min(best, t)
        return best

    res = {"cus": cus, "iters": iters}
    for wps in (1, 2, 4):  # waves per SIMD
        blocks = cus * wps
        ms = run(0, blocks)
        flops = blocks * 4 * iters * 4 * 2048  # waves x MFMAs x flops per 16x16x4 MFMA
        res[f"mfma_tflops_{wps}_waves_per_simd"] = flops / (ms * 1e-3) / 1e12
    t_mfma, t_valu, t_mixed = run(0, cus), run(1, cus), run(2, cus)
    t_split = run(3, cus, 512)  # one MFMA wave and one VALU wave on every SIMD
    t_bf16 = run(4, cus)
    t_split16 = run(5, cus, 512)
    res["bf16_mfma_tflops_1_wave_per_simd"] = cus * 4 * iters * 4 * 16384 / (t_bf16 * 1e-3) / 1e12
    res.update({"ms_bf16_mfma_only": t_bf16, "ms_two_waves_bf16_and_valu": t_split16,
                "two_waves_bf16_over_sum": t_split16 / (t_bf16 + t_valu),
                "two_waves_bf16_over_max": t_split16 / max(t_bf16, t_valu)})
    res.update({"ms_mfma_only": t_mfma, "ms_valu_only": t_valu, "ms_mixed_one_wave": t_mixed,
                "mixed_over_sum": t_mixed / (t_mfma + t_valu),
                "mixed_over_max": t_mixed / max(t_mfma, t_valu),
                "ms_two_waves_one_each": t_split,
                "two_waves_over_max": t_split / max(t_mfma, t_valu)})
    return res
