"""Build libkvevict.so in-tree with hipcc for gfx950.

Each HIP source is compiled to an object in ``_build/`` (in parallel), then
linked into ``learned_kv_cache_head_amd/_lib/libkvevict.so``. The benchmark's
read-bandwidth reference kernel is linked into its own ``libkvebench.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libkvevict.so")
BENCH_LIB = os.path.join(LIBDIR, "libkvebench.so")
BUILD = os.path.join(ROOT, "_build")
RESOURCE_REPORT = os.path.join(BUILD, "kernel_resource_usage.txt")
SOURCES = ["kvevict.hip", "attention.hip", "cache_ops.hip", "score.hip",
           "mlstm.hip", "prefill.hip"]
BENCH_SOURCES = ["bench_read.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # Packed FP32 instructions are left to no code path here.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature;
    # that line is expected and dropped.
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "is not a recognized feature" not in l)
    return p.returncode, out


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library. Returns its
    path. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [cc, *COMMON_FLAGS, *inc, "-c", os.path.join(CSRC, src),
               "-o", obj, "-Rpass-analysis=kernel-resource-usage"]
        rc, out = _run(cmd)
        return src, obj, rc, out, cmd

    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(compile_one, SOURCES + BENCH_SOURCES))
    usage = []
    for src, obj, rc, out, cmd in results:
        remarks = [l for l in out.splitlines()
                   if "kernel-resource-usage" in l]
        usage += remarks
        rest = "\n".join(l for l in out.splitlines()
                         if "kernel-resource-usage" not in l
                         and not l.lstrip().startswith(("|", "^"))
                         and not l.strip().isdigit())
        if verbose or rc != 0:
            sys.stderr.write(f"[build] {' '.join(cmd)}\n{rest}\n")
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}")
    # The compiler's per-kernel resource report (registers, scratch, LDS,
    # occupancy), kept for the check that no kernel spills to scratch.
    with open(RESOURCE_REPORT, "w") as f:
        f.write("\n".join(usage) + "\n")
    objs = {r[0]: r[1] for r in results}
    for lib, srcs in ((LIB, SOURCES), (BENCH_LIB, BENCH_SOURCES)):
        tmp = lib + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
               *[objs[x] for x in srcs]]
        rc, out = _run(cmd)
        if verbose or rc != 0:
            sys.stderr.write(f"[build] {' '.join(cmd)}\n{out}\n")
        if rc != 0:
            raise RuntimeError(f"link failed: {os.path.basename(lib)}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
