"""Builds libmagi_attn.so (the HIP kernels and the C ABI) in-tree for gfx950."""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmagi_attn.so")
SOURCES = ["api.cpp", "plan.cpp", "fwd_bf16.hip", "fwd_fp32.hip", "bwd_bf16.hip", "bwd_fp32.hip", "noalloc.hip"]

# gfx950 only; packed-fp32 VALU forms are disabled on purpose (the compiler
# still emits scalar fp32); code object v5 for the HIP runtime shipped with torch.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-mcode-object-version=5",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    """Compiles every source and links the shared library; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIP_FLAGS + ["-shared", "-I" + INCLUDE, "-I" + CSRC, "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    errtext = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + errtext)
    if verbose and errtext.strip():
        print(errtext, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
    deps.append(os.path.join(INCLUDE, "magi_attn.h"))
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build(verbose=True))
