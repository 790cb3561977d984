"""Builds libbitsmoe.so (gfx950) in-tree with hipcc.

    python -m spectral_expert_gemv_amd.build

Host-only sources (packer, status strings) are compiled as plain C++ with
no floating-point contraction; the HIP source is compiled for gfx950 with
packed fp32 instructions disabled.  Objects go to ``_build/`` at the repo
root; the shared library lands next to this file.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libbitsmoe.so")
ARCH = "gfx950"

HOST_SOURCES = ["common.cpp", "pack.cpp"]
HIP_SOURCES = ["bitsmoe.hip", "fused.hip", "one.hip", "grouped.hip", "pack_gpu.hip", "fqcm.hip", "down.hip", "ssd.hip"]

HIP_FLAGS = [
    "-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-x", "c++", "-O2", "-std=c++17", "-fPIC", "-ffp-contract=off",
              "-fno-fast-math", "-Wall"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout)
        raise RuntimeError("command failed: " + " ".join(cmd))
    if verbose and r.stdout.strip():
        # keep warnings visible, but the host pass's note about the device
        # feature flag is expected
        lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            print("\n".join(lines), flush=True)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    inc = ["-I", INCLUDE, "-I", CSRC]
    for src in HOST_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        _run([hipcc] + HOST_FLAGS + inc + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        _run([hipcc] + HIP_FLAGS + inc + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = OUT + ".tmp"
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
