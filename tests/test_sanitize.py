"""AddressSanitizer and UndefinedBehaviorSanitizer runs on the CPU.

The C oracle is built with gcc under -fsanitize=address,undefined together
with tests/sanitize/oracle_checks.c, which runs every oracle entry point on
small seeded inputs and every argument error.  The C ABI's host side (api.hip,
rebuilt with the sanitizers on its host code only) is linked with the other
library objects and tests/sanitize/abi_errors.cpp, which drives every argument
error path; those paths return before anything touches a device, so no GPU is
needed.  A sanitizer report fails the run (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OBJS = ["select", "gemv", "linear", "ffn", "attn"]
# every -fsanitize= of a hipcc compile applies to the host code only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def run(cmd, env=None, timeout=300):
    p = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    run(["gcc", "-std=c99", "-g", "-O1", "-fno-omit-frame-pointer", "-ffp-contract=off",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'oracle')}",
         os.path.join(ROOT, "oracle", "rmm_oracle.c"), os.path.join(HERE, "oracle_checks.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    p = run([exe], env=env)
    assert "oracle checks passed" in p.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_c_abi_host_validation_under_asan_ubsan(tmp_path):
    objs = [os.path.join(ROOT, "_build", o + ".o") for o in OBJS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (run __graft_entry__.build())")
    inc = os.path.join(ROOT, "include")
    api = str(tmp_path / "api.o")
    drv = str(tmp_path / "abi_errors.o")
    exe = str(tmp_path / "abi_errors")
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", *HOST_SAN, f"-I{inc}", "-c",
         os.path.join(ROOT, "input_adaptive_reduced_score_amd", "csrc", "api.hip"), "-o", api])
    run([HIPCC, "-O1", "-g", "-std=c++17", *HOST_SAN, f"-I{inc}", "-c", os.path.join(HERE, "abi_errors.cpp"),
         "-o", drv])
    run([HIPCC, "--offload-arch=gfx950", "-fsanitize=address,undefined", "-fno-gpu-sanitize", drv, api, *objs,
         "-o", exe])
    # the HIP runtime is not instrumented: leak reports from it are not this code's
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    p = run([exe], env=env)
    assert "abi checks passed" in p.stdout
