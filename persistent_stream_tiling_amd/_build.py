"""Compile the gfx950 GEMM library (libgemmsk.so) in-tree with hipcc."""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgemmsk.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "api.hip")]
ARCH = "gfx950"


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libgemmsk.so")
    return path


def build(out=LIB, verbose=False, extra=()):
    """Compile every source for gfx950 into one shared library; returns its path."""
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           f"-I{INCLUDE}", f"-I{CSRC}",
           # packed fp32 VALU ops are kept out of the generated code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           *extra, *SOURCES, "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr[-8000:])
    if verbose:
        print(res.stderr)
    os.replace(out + ".tmp", out)
    return out


PROBES = os.path.join(PKG, "probes")


def build_probes(verbose=False):
    """Compile the measurement probes kept out of the library: the
    hardware-ceiling program (probes/ceilings.hip) and the phase-timing copy of
    the kernels (probes/libphase.so, see probes/phases.py); returns the
    ceiling program's path."""
    from .probes import phases
    phases.build()
    src = os.path.join(PROBES, "ceilings.hip")
    out = os.path.join(PROBES, "ceilings")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr[-8000:])
    if verbose:
        print(res.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=False))
