"""Build libqmm.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: ``python -m weight_only_group_amd.build`` or ``build()`` from Python.
Extra preprocessor definitions (tuning constants) can be passed with
``defines``; ``out`` names another output path.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ("api.hip", "pack.hip", "dequant.hip", "gemv.hip", "gemv_wave_b1.hip", "gemv_wave_b2.hip",
           "gemv_wave_b3.hip", "gemv_wave_b4.hip", "gemv_wave_b8.hip", "gemm.hip", "strips.hip")
LIB_NAME = "libqmm.so"
# Reference kernels for measurement (empty launch, streaming read, MFMA loop);
# a library of their own, outside the qmm ABI.
PROBE_SOURCES = ("probes.hip",)
PROBE_LIB_NAME = "libqmm_probes.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def compile_flags(defines=()) -> list[str]:
    flags = [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # Keep the compiler from emitting packed fp32 instructions.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wall", "-Wno-unused-result",
    ]
    flags += [f"-D{d}" for d in defines]
    return flags


def _compile_and_link(sources, out: str, defines, verbose: bool, jobs: int) -> str:
    cc = hipcc()
    tag = "default" if not defines else "_".join(str(d).replace("=", "-") for d in defines)
    objdir = os.path.join(HERE, "_build", tag)
    os.makedirs(objdir, exist_ok=True)
    flags = compile_flags(defines)

    def one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, sources))
    tmp = out + ".tmp"
    cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build(out: str | None = None, defines=(), verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libqmm.so (and, for the default build, the
    measurement probes library); returns the path of libqmm.so."""
    default = out is None and not defines
    path = _compile_and_link(SOURCES, out or os.path.join(HERE, LIB_NAME), defines, verbose, jobs)
    if default:
        _compile_and_link(PROBE_SOURCES, os.path.join(HERE, PROBE_LIB_NAME), (), verbose, jobs)
    return path


if __name__ == "__main__":
    defs = [a[2:] for a in sys.argv[1:] if a.startswith("-D")]
    outs = [a for a in sys.argv[1:] if not a.startswith("-D")]
    build(out=outs[0] if outs else None, defines=defs, verbose=True)
