"""The C-ABI layer (sla2_api.hip: argument checks, buffer sizes, workspace layouts, error
reporting) built for the host with AddressSanitizer and UndefinedBehaviorSanitizer and driven on
the CPU through every check (tests/host_sanitize/driver.cpp).  The launchers are stubs that
report a HIP error, so nothing reaches a GPU; the device side of sla2_api.hip (the no-alloc
router's scratch array) is compiled as usual."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "sparse_linear_attention_pool_amd", "csrc")
ROCM = "/opt/rocm"


def _tool(name):
    path = shutil.which(name) or os.path.join(ROCM, "bin", name)
    if not os.path.exists(path):
        pytest.skip(f"{name} not found")
    return path


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_api_layer_under_host_sanitizers(tmp_path):
    hipcc, clang = _tool("hipcc"), _tool("amdclang++")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    host_san = [x for f in san for x in ("-Xarch_host", f)]   # host code only: no GPU sanitizer
    api_o, stub_o, drv_o = (str(tmp_path / n) for n in ("api.o", "stub.o", "driver.o"))
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++20", "-fPIC", *host_san,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *inc,
          "-c", os.path.join(CSRC, "sla2_api.hip"), "-o", api_o])
    _run([clang, "-O1", "-g", "-std=c++20", "-fPIC", *san, "-D__HIP_PLATFORM_AMD__", "-I", f"{ROCM}/include", *inc,
          "-c", os.path.join(HERE, "stub_launch.cpp"), "-o", stub_o])
    _run([clang, "-O1", "-g", "-std=c++17", *san, "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(HERE, "driver.cpp"), "-o", drv_o])
    exe = str(tmp_path / "sanitize_driver")
    _run([clang, *san, api_o, stub_o, drv_o, "-L", f"{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "sanitize driver ok" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
