"""The C ABI's host layer under AddressSanitizer, on the CPU: validation,
workspace layout and kernel sequencing of every entry point, built from the
library's own source with the kernel launchers replaced by host-only stubs that
check each workspace region a launch would receive lies inside the workspace.
No device is touched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "complex_valued_state_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "asan")


def test_abi_host_layer_under_asan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    asan = ["-fsanitize=address", "-fno-omit-frame-pointer"]
    api = str(tmp_path / "api.o")
    # the HIP source: sanitizer on the host pass only
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *inc, "-c",
                    os.path.join(CSRC, "cssd_api.hip"), "-o", api], check=True,
                   capture_output=True)
    objs = [api]
    for src in ("launch_stubs.cpp", "abi_main.cpp"):
        obj = str(tmp_path / (src + ".o"))
        subprocess.run(["g++", "-O1", "-g", "-std=c++17", *asan, "-D__HIP_PLATFORM_AMD__",
                        "-I", "/opt/rocm/include", *inc, "-c", os.path.join(HERE, src), "-o", obj],
                       check=True, capture_output=True)
        objs.append(obj)
    exe = str(tmp_path / "abi_asan")
    subprocess.run(["g++", *asan, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "0 failed" in r.stdout
