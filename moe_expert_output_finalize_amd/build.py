"""Build libmoe_finalize.so (gfx950) in-tree with hipcc.

    python moe_expert_output_finalize_amd/build.py [-o OUT] [-D MACRO=VALUE ...]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_finalize.so")
SOURCES = ["capi.hip", "finalize_kernels.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    # packed FP32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIB, defines: list[str] | None = None, verbose: bool = False) -> str:
    """Compile the HIP sources into `out` (always recompiles)."""
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmd += [f"-D{d}" for d in (defines or [])]
    tmp = out + f".tmp{os.getpid()}"
    cmd += ["-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that note
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msg = "\n".join(l for l in (p.stdout + p.stderr).splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed ({p.returncode}):\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libmoe_finalize.so for gfx950")
    ap.add_argument("-o", "--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[],
                    help="extra preprocessor definition, e.g. -D MF_MAX_VECS=8")
    ns = ap.parse_args()
    print(build(out=ns.out, defines=ns.defines, verbose=True))
