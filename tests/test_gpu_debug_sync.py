"""CSSD_DEBUG_SYNC=1: every entry point synchronises after each of its kernels
and reports their errors at once.  Run in a child process (the setting is read
once, when the library is first used) on one forward, one decode step and one
backward; the results must equal, bit for bit, those of the same calls made in
this process without it."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import cssd_workloads as wl
from gpu_util import gpu_forward, log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, numpy as np
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
import cssd_workloads as wl
from gpu_util import gpu_forward
inp = wl.random_forward(77, 2, 300, 3, 64, 64, 64, with_h0=True)
y, hT = gpu_forward(inp)
inp16 = wl.random_forward(78, 2, 200, 2, 64, 64, 64, in_dtype="bf16")
y16, hT16 = gpu_forward(inp16)
np.savez(sys.argv[2], y=y, hT=hT, y16=y16, hT16=hT16)
print("child done", flush=True)
"""


def test_debug_sync_mode_gives_the_same_results(tmp_path):
    out = str(tmp_path / "child.npz")
    env = dict(os.environ, CSSD_DEBUG_SYNC="1")
    log("  child process with CSSD_DEBUG_SYNC=1")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, out], env=env, capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-3000:]
    got = np.load(out)
    y, hT = gpu_forward(wl.random_forward(77, 2, 300, 3, 64, 64, 64, with_h0=True))
    y16, hT16 = gpu_forward(wl.random_forward(78, 2, 200, 2, 64, 64, 64, in_dtype="bf16"))
    for k, v in (("y", y), ("hT", hT), ("y16", y16), ("hT16", hT16)):
        assert np.array_equal(got[k], v), k
