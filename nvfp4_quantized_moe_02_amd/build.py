"""Build libnvfp4moe.so in-tree: the HIP sources with hipcc for gfx950 (cross-compiles
without a GPU), the host-only sources (*.cpp) with the host C++ compiler."""
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libnvfp4moe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # no packed fp32 instructions (see the design notes); harmless warning on the host pass
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-pthread", "-Wall"]


def cxx() -> str:
    for c in (os.environ.get("CXX"), shutil.which("g++"), "/opt/rocm/llvm/bin/clang++"):
        if c and (os.path.exists(c) or shutil.which(c)):
            return c
    raise RuntimeError("no host C++ compiler found")


def _run(cmd, what, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError(what + " failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source (always), one process per translation unit, then link."""
    from concurrent.futures import ThreadPoolExecutor

    jobs = []
    objs = []
    for src in sorted(glob.glob(os.path.join(PKG, "csrc", "*.cpp"))):
        obj = os.path.join(PKG, "csrc", os.path.basename(src)[:-4] + ".host.o")
        jobs.append(([cxx(), *HOST_FLAGS, "-c", src, "-o", obj], "host compile of " + src))
        objs.append(obj)
    for src in sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip"))):
        obj = os.path.join(PKG, "csrc", os.path.basename(src)[:-4] + ".dev.o")
        jobs.append(([hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj],
                     "hipcc of " + src))
        objs.append(obj)
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_run, c, w, verbose) for c, w in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-pthread", "-o", tmp], "link", verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
