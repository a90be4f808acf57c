"""Build libpa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m paged_kv_cache_32_amd.build [--verbose]

Compiles every ``csrc/*.hip`` with hipcc for gfx950 only, and the host-only
``csrc/*.cpp`` (the block manager) with the host C++ compiler, and links them
into ``paged_kv_cache_32_amd/lib/libpa.so``.  Packed-fp32 VALU forms are
switched off for the device code (plain fp32 VALU and MFMA only).
"""

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libpa.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def flags(extra=()):
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-result", f"-I{INCLUDE}", *extra,
    ]


def host_cxx():
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no host C++ compiler found")


def host_flags():
    return ["-O2", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}"]


def build(verbose=False, extra=()):
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = []
    cc = hipcc()
    for src in srcs:
        obj = os.path.join(LIBDIR, os.path.basename(src) + ".o")
        if src.endswith(".cpp"):
            cmd = [host_cxx(), *host_flags(), "-c", src, "-o", obj]
        else:
            cmd = [cc, *flags(extra), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(line for line in (r.stderr or "").splitlines()
                         if "packed-fp32-ops" not in line)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
