"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no kernel is launched).

api.hip (validation, error reporting, the size and plan queries) is rebuilt
with both sanitizers on its host code and linked, with the library's other
objects as built by the default build, into tests/abi_sanitized_driver.cpp.
The driver makes every entry point refuse invalid arguments (NULLs, bad
widths, shapes, group sizes, misalignment, extreme integers) and sweeps the
size and plan queries over ordinary and extreme shapes; any sanitizer report
aborts it (no recovery), any unexpected status fails it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))


def _tools():
    from weight_only_group_amd import build
    clangxx = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(clangxx) or not shutil.which(build.hipcc()):
        pytest.skip("ROCm's clang is not installed")
    return build, clangxx


def test_abi_validation_under_sanitizers(tmp_path):
    build, clangxx = _tools()
    objdir = os.path.join(build.HERE, "_build", "default")
    others = [os.path.join(objdir, s.replace(".hip", ".o")) for s in build.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in others):
        build.build()
    # Sanitizers on the host code only (each -fsanitize= behind -Xarch_host): the device code is as built.
    host_san = ["-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
                "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    api_o = str(tmp_path / "api_sanitized.o")
    cmd = [build.hipcc(), *build.compile_flags(), *host_san, "-c", os.path.join(build.CSRC, "api.hip"), "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "abi_sanitized_driver")
    link = [clangxx, "-g", "-O1", "-std=c++17", "-fsanitize=address", "-fsanitize=undefined",
            "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
            "-I", "/opt/rocm/include", os.path.join(HERE, "abi_sanitized_driver.cpp"), api_o, *others,
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "as expected" in r.stdout
