"""The host half of the library (planner, reducer state machine, groups,
masks, failure handling) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, and driven by tests/native/host_fuzz.cpp: random
API sequences on host-only reducers, whose launches go to a callback. The
kernel launchers are stubbed out (a host-only reducer never launches one);
no GPU is needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bucketed_gradient_all_amd", "csrc")

STUB = r'''
#include "internal.h"
#include "static_area.h"
namespace ddp {
hipError_t launch_mean(int, int, bool, const Scale &, const KernelTables &, int32_t, int32_t, unsigned, bool,
                       hipStream_t)
{ return hipErrorInvalidValue; }
hipError_t launch_bf16_hook(int, int, bool, const Scale &, const KernelTables &, int32_t, int32_t, unsigned, bool,
                            hipStream_t)
{ return hipErrorInvalidValue; }
hipError_t launch_fp16_hook(int, int, bool, const Scale &, const KernelTables &, int32_t, int32_t, unsigned, bool,
                            hipStream_t)
{ return hipErrorInvalidValue; }
hipError_t static_table_area(int, void **, size_t *) { return hipErrorNoDevice; }
uint64_t claim_static_table_area(int) { return 0; }
uint64_t static_table_generation(int) { return 0; }
}
'''


SAN = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
       "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-static-libasan", "-static-libubsan",
       "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# operator new goes through tests/native/failing_new.h
WRAP_NEW = "-Wl,--wrap=_Znwm,--wrap=_Znam,--wrap=_ZnwmRKSt9nothrow_t,--wrap=_ZnamRKSt9nothrow_t"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _needs_toolchain():
    if shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("needs g++ and the ROCm headers")


def test_host_logic_under_sanitizers(tmp_path):
    _needs_toolchain()
    stub = tmp_path / "stub.cpp"
    stub.write_text(STUB)
    exe = tmp_path / "host_fuzz"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-static-libasan", "-static-libubsan",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "reducer.cpp"), str(stub), os.path.join(ROOT, "tests", "native", "host_fuzz.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", WRAP_NEW, "-o", str(exe)]
    subprocess.run(cmd, check=True, timeout=600)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    for args in (["300"], ["300", "oom"]):
        r = subprocess.run([str(exe), *args], capture_output=True, text=True, timeout=600, env=env)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
        assert "host_fuzz ok" in r.stdout
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_device_path_host_logic_under_sanitizers(tmp_path):
    """reducer.cpp's device path against a host-only stand-in for the HIP
    runtime (tests/native/fake_hip.cpp): the timing ring stays bounded and
    reads every launch's own events, a reduction on another stream is
    ordered around the mask upload, and failing host allocations give
    DDP_ERR_NOMEM without leaks or lost launches."""
    _needs_toolchain()
    exe = tmp_path / "device_host_checks"
    native = os.path.join(ROOT, "tests", "native")
    cmd = [*SAN, "-I", native, os.path.join(CSRC, "reducer.cpp"), os.path.join(native, "fake_hip.cpp"),
           os.path.join(native, "device_host_checks.cpp"), WRAP_NEW, "-o", str(exe)]
    subprocess.run(cmd, check=True, timeout=600)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=ENV)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "device_host_checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
