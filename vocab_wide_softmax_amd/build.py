"""Build libvws.so (HIP kernels for gfx950 behind the C ABI of include/vws.h).

Usage: python -m vocab_wide_softmax_amd.build [-v]

Every .hip file under csrc/ is compiled with hipcc for gfx950 (in parallel) and
linked into vocab_wide_softmax_amd/libvws.so, next to this file. Packed fp32
VALU instructions are disabled for all device code.
"""

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvws.so")

ARCH = os.environ.get("VWS_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and "feature flag" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (r.returncode, " ".join(cmd), r.stdout))
    if verbose and out.strip():
        print(out, flush=True)


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libvws.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJDIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_run, [HIPCC] + COMMON + ["-c", s, "-o", o], verbose) for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
