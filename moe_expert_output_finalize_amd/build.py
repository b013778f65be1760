"""Build libmoe_finalize.so (gfx950) in-tree with hipcc.

    python moe_expert_output_finalize_amd/build.py [-o OUT] [-D MACRO=VALUE ...]

Beside the library it writes ``<library>.sources``: a digest of every source
and header the library is built from, which the Python binding compares with
the tree it is imported from, so a library older than its sources is refused
instead of being tested or timed.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_finalize.so")
SOURCES = ["capi.cpp", "finalize_kernels.hip"]
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


PROBES_LIB = os.path.join(PKG, "libmf_probes.so")
PROBES_SOURCE = "bench_probes.hip"


def source_files(root: str = ROOT) -> list[str]:
    """Every file the library is compiled from, in a fixed order."""
    csrc = os.path.join(root, "moe_expert_output_finalize_amd", "csrc")
    inc = os.path.join(root, "include")
    files = [os.path.join(csrc, f) for f in SOURCES]
    files += [os.path.join(csrc, f) for f in sorted(os.listdir(csrc)) if f.endswith(".hpp")]
    files += [os.path.join(inc, f) for f in sorted(os.listdir(inc)) if f.endswith(".h")]
    return files


def code_text(text: str) -> str:
    """C/C++ source with its comments removed and blank lines dropped, so that
    an edit to a comment does not change what the digest says was built.
    String and character literals are kept as they are."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    lines = [line.rstrip() for line in "".join(out).splitlines()]
    return "\n".join(line for line in lines if line)


def source_digest(root: str = ROOT, defines: list[str] | None = None) -> str:
    """SHA-256 over the names and code (comments removed) of the library's
    sources, the compiler flags and any extra definitions."""
    h = hashlib.sha256()
    h.update(" ".join(HIPCC_FLAGS + sorted(defines or [])).encode())
    for path in source_files(root):
        h.update(os.path.relpath(path, root).encode() + b"\0")
        with open(path, encoding="utf-8") as f:
            h.update(code_text(f.read()).encode() + b"\0")
    return h.hexdigest()


def digest_path(lib: str) -> str:
    return lib + ".sources"


def build(out: str = LIB, defines: list[str] | None = None, verbose: bool = False) -> str:
    """Compile the HIP sources into `out` (always recompiles) and record the
    digest of what it was built from."""
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC]
    cmd += [f"-D{d}" for d in (defines or [])]
    tmp = out + f".tmp{os.getpid()}"
    cmd += ["-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    digest = source_digest(ROOT, defines)
    p = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that note
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msg = "\n".join(l for l in (p.stdout + p.stderr).splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed ({p.returncode}):\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    os.replace(tmp, out)
    with open(digest_path(out) + ".tmp", "w") as f:
        f.write(digest + "\n")
    os.replace(digest_path(out) + ".tmp", digest_path(out))
    return out


def build_probes(out: str = PROBES_LIB) -> str:
    """Compile the benchmark's memory probes (csrc/bench_probes.hip) into
    their own library, which the finalize ABI does not include."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, os.path.join(CSRC, PROBES_SOURCE)]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed ({p.returncode}):\n{p.stdout}{p.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libmoe_finalize.so for gfx950")
    ap.add_argument("-o", "--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[],
                    help="extra preprocessor definition, e.g. -D MF_MAX_VECS_INDEX_MAP=8")
    ns = ap.parse_args()
    print(build(out=ns.out, defines=ns.defines, verbose=True))
