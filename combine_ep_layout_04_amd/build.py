"""Build libep.so (HIP, gfx950) in-tree with hipcc.

    python -m combine_ep_layout_04_amd.build

Flags: -O3; fp32 division and square root correctly rounded (the fp8 scale
and every quotient must match IEEE division bit for bit); fp32 denormals
kept; packed-fp32 instruction selection disabled.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libep.so")
ARCH = os.environ.get("EP_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


PROBE_SRC = os.path.join(PKG, "probes", "write_pattern.hip")
PROBE_LIB = os.path.join(PKG, "probes", "libep_probe.so")
DEMO_SRC = os.path.join(PKG, "examples", "c_abi_demo.c")
DEMO = os.path.join(PKG, "examples", "c_abi_demo")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into combine_ep_layout_04_amd/libep.so."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "--hip-link")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


def build_probe(verbose: bool = False) -> str:
    """Compile the measurement kernels (probes/write_pattern.hip) into
    probes/libep_probe.so, with the library's flags."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{CSRC}", "-o", tmp, PROBE_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on the probes:\n" + res.stdout + res.stderr)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build_demo(verbose: bool = False) -> str:
    """Compile the plain-C example (examples/c_abi_demo.c) with gcc against
    include/ep.h and libep.so: the C ABI used with no Python in the way."""
    cc = os.environ.get("CC") or shutil.which("gcc") or "cc"
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{INCLUDE}", f"-I{ROCM}/include", "-o", DEMO, DEMO_SRC, f"-L{PKG}", "-lep",
           f"-L{ROCM}/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN/..", f"-Wl,-rpath,{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the C example failed:\n" + res.stdout + res.stderr)
    return DEMO


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_demo(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
