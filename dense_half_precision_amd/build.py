"""Build libhgemm.so (the HIP kernels and their C ABI) for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhgemm.so")
SOURCES = ["hgemm_api.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-command-line-argument",
    # keep the backend from forming packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def asm(source: str = "hgemm_api.hip", out: str | None = None) -> str:
    """Device assembly of one source (for reading our own ISA)."""
    out = out or os.path.join(PKG, "_build", source.replace(".hip", ".s"))
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "-S", "--cuda-device-only",
           os.path.join(CSRC, source), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
