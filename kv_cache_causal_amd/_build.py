"""Build the HIP library (libkvc.so, gfx950) and the host-only validation shim.

    python -m kv_cache_causal_amd._build

Compiles every source under csrc/ with hipcc for gfx950 (in parallel), links
lib/libkvc.so, builds lib/libkvc_probe.so (the benchmark's streaming-read helper, not
part of the library) and lib/libkvc_hostcheck.so (validate.cpp + hostcheck.cpp with g++,
no HIP) so the argument checks can be tested on a machine without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
OBJDIR = os.path.join(ROOT, "_build", "obj")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_SOURCES = ["k_rope.hip", "k_qkv.hip", "k_decode.hip", "k_prefill.hip", "kvc_api.cpp",
               "validate.cpp", "plan.cpp"]
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # Packed fp32 instructions are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
LIB = os.path.join(LIBDIR, "libkvc.so")
HOSTCHECK = os.path.join(LIBDIR, "libkvc_hostcheck.so")
PROBE = os.path.join(LIBDIR, "libkvc_probe.so")
ABI_DEMO = os.path.join(LIBDIR, "abi_demo")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {os.path.basename(cmd[-1])}")
    return r


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    _run([HIPCC, *HIP_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(HIP_SOURCES)))) as ex:
        objs = list(ex.map(_compile, HIP_SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    # The benchmark's measurement helper (read ceiling, cache flush): a library of its own.
    probe_obj = _compile("read_probe.hip")
    tmp = PROBE + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", probe_obj, "-o", tmp])
    os.replace(tmp, PROBE)
    tmp = HOSTCHECK + ".tmp"
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}",
          os.path.join(CSRC, "validate.cpp"), os.path.join(CSRC, "plan.cpp"),
          os.path.join(CSRC, "hostcheck.cpp"), "-o", tmp])
    os.replace(tmp, HOSTCHECK)
    # The ABI used from plain C (a GPU test runs it): gcc, C11, against the HIP runtime.
    tmp = ABI_DEMO + ".tmp"
    _run(["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
          f"-I{ROCM}/include", f"-I{INCLUDE}", os.path.join(ROOT, "tests", "c_abi", "abi_demo.c"),
          f"-L{LIBDIR}", "-lkvc", f"-L{ROCM}/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN",
          f"-Wl,-rpath,{ROCM}/lib", "-o", tmp])
    os.replace(tmp, ABI_DEMO)
    return LIB


if __name__ == "__main__":
    print(build())
