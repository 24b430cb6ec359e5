"""The C ABI's host code (argument validation, workspace layouts, the host-only entry points) built
with AddressSanitizer and UndefinedBehaviorSanitizer and run on the CPU: tests/host_sanitize/
abi_checks.cpp calls every device entry point with arguments its validation must reject (its
stand-in launchers abort if a launch is reached) and sweeps the workspace helpers, the fan-out, the
speedup model and the crossover up to the largest supported shapes. No GPU is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                    reason="needs g++ and the HIP runtime library")
def test_host_abi_code_is_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_checks")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include",
           f"-I{ROOT}/draft_verification_ssd_amd/csrc", os.path.join(ROOT, "tests", "host_sanitize", "abi_checks.cpp"),
           os.path.join(ROOT, "draft_verification_ssd_amd", "csrc", "ssd_api.cpp"), f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "abi checks ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
