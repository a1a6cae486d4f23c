"""The hardware figures the kernels' design rests on (needs an MI355X): the fp32
matrix-core rate a wave reaches with independent accumulator chains, against
the 157.3 TFLOP/s every roofline fraction here divides by; and whether one
wave's vector-ALU instructions overlap its matrix-core instructions, and whether
two waves' on one SIMD do.  For fp32 they do neither (the chip's fp32 matrix and
vector peaks are the same figure): every operand sum of the Gauss form (three
real MFMAs per complex product instead of four) and every other vector
instruction is paid in full.  The bf16 matrix instructions are measured the same
way, for information."""
import json
import os

import pytest

import gpu_probes
from gpu_util import log

pytestmark = pytest.mark.gpu


def test_fp32_mfma_peak_and_valu_issue():
    if not os.path.exists(gpu_probes.LIB):
        gpu_probes.build()
    r = gpu_probes.measure()
    log("  " + json.dumps({k: round(v, 4) if isinstance(v, float) else v for k, v in r.items()}))
    peak = gpu_probes.PEAK_FP32_MFMA_TFLOPS
    best = max(r[f"mfma_tflops_{w}_waves_per_simd"] for w in (1, 2, 4))
    assert 0.8 * peak <= best <= 1.02 * peak, best
    # fp32 VALU and fp32 MFMA work do not overlap, in one wave (1.15x the sum) or in
    # two waves of one SIMD (1.0x the sum): they share the SIMD's fp32 datapath
    assert 0.9 <= r["mixed_over_sum"] <= 1.4, r
    assert 0.85 <= r["ms_two_waves_one_each"] / (r["ms_mfma_only"] + r["ms_valu_only"]) <= 1.3, r
    assert r["bf16_mfma_tflops_1_wave_per_simd"] > 0.0 and r["two_waves_bf16_over_sum"] > 0.0
