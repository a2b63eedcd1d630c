"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
q4_api.hip built with the sanitizers on its host side only (-Xarch_host; the
kernels are compiled as usual and never launched) and linked with
tests/sanitize_abi_driver.cpp, which runs every entry point's argument
validation and the chain encoders (the temporal step, its dependent form, four
activation rows, the table limits, a short plan buffer, fused decoder layers)
on stand-in device addresses. No GPU is needed: nothing reaches a launch."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")


@pytest.mark.timeout(900)
@pytest.mark.skipif(shutil.which("hipcc") is None or not os.path.exists(CLANG), reason="needs hipcc and clang++")
def test_abi_host_code_under_address_and_ub_sanitizers(tmp_path):
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("q4_api.o", "driver.o", "abi_sanitized"))
    host_san = [a for f in san for a in ("-Xarch_host", f)]
    steps = [
        ["hipcc", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "--offload-arch=gfx950", *host_san,
         "-I", os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "bit_group_quantized_amd", "csrc", "q4_api.hip"),
         "-o", api_o],
        [CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *san, "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(HERE, "sanitize_abi_driver.cpp"),
         "-o", drv_o],
        [CLANG, *san[:2], api_o, drv_o, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
         "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, " ".join(cmd) + "\n" + r.stderr[-2000:]
    # (leak checking is off: the HIP runtime keeps its own allocations to the end)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi sanitized run: ok" in run.stdout
