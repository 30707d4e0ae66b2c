"""Build the HIP library in-tree: sparse_attention_video_da_amd/lib/libdecoupattn.so.

Compiles the attention sources under csrc/ for gfx950 with hipcc and links one shared library
exporting only the C ABI declared in include/decoupattn.h; the benchmark's peak probe
(csrc/peak_probe.hip) becomes lib/libdapeak.so, and the plain-C example that a GPU test runs
(tests/native/c_abi_example.c) becomes lib/c_abi_example, linked against the library.

    python sparse_attention_video_da_amd/build.py [--jobs N]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libdecoupattn.so")
SOURCES = ["api.cpp", "plan_lists.cpp", "forward.hip", "reassign.hip"]
PEAK_SOURCE = "peak_probe.hip"
PEAK_LIB = os.path.join(LIBDIR, "libdapeak.so")
C_EXAMPLE_SOURCE = os.path.join(ROOT, "tests", "native", "c_abi_example.c")
C_EXAMPLE = os.path.join(LIBDIR, "c_abi_example")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l)   # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({' '.join(cmd)}):\n{out}")
    return out


def build(jobs: int = 4, verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        out = _run([cc, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    # the benchmark's peak probe (not part of the attention library)
    probe = compile_one(PEAK_SOURCE)
    tmp = PEAK_LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, probe])
    os.replace(tmp, PEAK_LIB)
    build_c_example()
    return LIB


def build_c_example() -> str:
    """The C ABI from plain C: compile tests/native/c_abi_example.c with the system C compiler
    against lib/libdecoupattn.so (found next to the binary at run time)."""
    cc = next((c for c in (os.environ.get("CC"), shutil.which("cc"), shutil.which("gcc")) if c),
              None)
    if cc is None:
        raise RuntimeError("no C compiler found for the C ABI example")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = C_EXAMPLE + ".tmp"
    _run([cc, "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
          f"-I{os.path.join(ROOT, 'include')}", C_EXAMPLE_SOURCE, "-o", tmp, f"-L{LIBDIR}",
          "-ldecoupattn", f"-L{rocm}/lib", "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN",
          f"-Wl,-rpath,{rocm}/lib"])
    os.replace(tmp, C_EXAMPLE)
    return C_EXAMPLE


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
