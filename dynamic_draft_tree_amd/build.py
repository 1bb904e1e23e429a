"""Build libeagletree.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libeagletree.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


PROBES = os.path.join(HERE, "probes")


def build_probes(verbose: bool = False) -> list:
    """Measurement programs (probes/*.hip, one executable each beside its
    source): not part of the library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    out = []
    for src in sorted(glob.glob(os.path.join(PROBES, "*.hip"))):
        exe = src[:-len(".hip")]
        cmd = [hipcc, *flags, src, "-o", exe]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, capture_output=not verbose)
        out.append(exe)
    return out


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    # a kernel template whose host-side instantiation failed leaves its
    # launch stub undefined; refuse such a library here rather than at load
    und = subprocess.run(["nm", "-D", "--undefined-only", tmp], check=True,
                         capture_output=True, text=True).stdout
    missing = [ln.split()[-1] for ln in und.splitlines() if "_ZN2et" in ln]
    if missing:
        os.remove(tmp)
        raise RuntimeError("libeagletree: undefined symbols " + ", ".join(missing))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probes(verbose=True))
