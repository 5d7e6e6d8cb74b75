"""Build the HIP library in-tree: ``kv_cache_compression_kvc_amd/libkvc.so``.

    python -m kv_cache_compression_kvc_amd.build [--jobs N] [--host-only]

Compiles for gfx950 only.  The four (head_dim, dtype) kernel sets are
separate objects so they compile in parallel.  ``--host-only`` builds just
``libkvc_host.so`` (the validation / sizing half, plain C++ with g++), which
the CPU tests use where hipcc is unavailable.
"""

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvc.so")
HOST_LIB = os.path.join(PKG, "libkvc_host.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU ops stay disabled in every device compile.
HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
INSTANCES = [(64, 0), (64, 1), (128, 0), (128, 1)]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if p.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build_host_only():
    cxx = shutil.which("g++") or shutil.which("c++")
    _run([cxx, "-std=c++17", "-O2", "-Wall", "-Wextra", "-fPIC", "-shared",
          os.path.join(CSRC, "kvc_host.cpp"), "-o", HOST_LIB])
    return HOST_LIB


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    tasks = []
    for d, dt in INSTANCES:
        obj = os.path.join(BUILD, "kvc_inst_d%d_t%d.o" % (d, dt))
        tasks.append([HIPCC] + HIP_FLAGS + ["-DKVC_D=%d" % d, "-DKVC_DT=%d" % dt, "-c",
                                            os.path.join(CSRC, "kvc_inst.hip"), "-o", obj])
    for name in ("kvc_launch.hip", "kvc_probe.hip", "kvc_unfused.hip", "kvc_pipeline.hip", "kvc_host.cpp"):
        obj = os.path.join(BUILD, name.split(".")[0] + ".o")
        src = os.path.join(CSRC, name)
        lang = ["-x", "hip"] if name.endswith(".hip") else []
        tasks.append([HIPCC] + HIP_FLAGS + lang + ["-c", src, "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, tasks):
            if verbose and out.strip():
                print(out)
    objs = [t[-1] for t in tasks]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp])
    os.replace(tmp, LIB)
    build_host_only()
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--host-only", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    if a.host_only:
        print(build_host_only())
    else:
        print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
