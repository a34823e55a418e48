"""The C ABI's host code built with AddressSanitizer and UBSan and run on the CPU.

tests/host_sanitize/abi_host_driver.cpp drives every host-only path of the
library -- shape validation, workspace sizing, argument rejection, the
persistent-head planner, status strings and the last-error buffer -- with
clo_api.cpp compiled by g++ under -fsanitize=address,undefined (the kernels
object is compiled as usual: its device code is not host code).  No GPU is
needed: nothing in the driver reaches a launch.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "top_sparse_attention_02_amd", "csrc")
ROCM = "/opt/rocm"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (shutil.which("g++") and os.path.exists(f"{ROCM}/bin/hipcc")), reason="needs g++ and hipcc")
def test_host_abi_under_address_and_undefined_sanitizers(tmp_path):
    from top_sparse_attention_02_amd import build

    kobjs = []
    for src in sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")):
        kobjs.append(str(tmp_path / (src + ".o")))
        _run([build.hipcc(), *build.HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", kobjs[-1]])
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
    common = ["-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}"]
    aobj, dobj = tmp_path / "api.o", tmp_path / "driver.o"
    _run(["g++", *common, *san, "-c", os.path.join(CSRC, "clo_api.cpp"), "-o", str(aobj)])
    _run(["g++", *common, *san, "-c", os.path.join(ROOT, "tests", "host_sanitize", "abi_host_driver.cpp"), "-o",
          str(dobj)])
    exe = tmp_path / "abi_host_driver"
    _run(["g++", *san, str(dobj), str(aobj), *kobjs, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib",
          "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host ABI checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
