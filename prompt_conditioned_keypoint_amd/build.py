"""Build libgkdhead.so (the HIP kernels + C ABI) in-tree for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgkdhead.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-fvisibility=hidden",  # only the GKD_API entry points are exported
    # packed fp32 VALU ops (v_pk_*_f32) are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip (one hipcc per source, in parallel) and link
    them into libgkdhead.so (always recompiles)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tag = "%d" % os.getpid()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + "." + tag + ".o") for s in srcs]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = max(1, min(len(srcs), os.cpu_count() or 1, 8))
    try:
        with ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda so: _run([hipcc, *compile_flags, *inc, "-c", so[0], "-o", so[1]],
                                        verbose), zip(srcs, objs)))
        tmp = LIB + ".tmp" + tag
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
