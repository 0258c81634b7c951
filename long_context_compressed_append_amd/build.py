"""Build liblcca.so and liblcca_debug.so (gfx950) in-tree with hipcc.

    python -m long_context_compressed_append_amd.build [--release-only]

Each source compiles to an object under _build/ (the debug library's under
_build/debug/) at the repository root, then everything links into
long_context_compressed_append_amd/liblcca.so.  The debug library is the same
sources built with LCCA_DEBUG: its kernels check every index they read from
device memory before forming an address (lcca_debug_check in lcca.h).
Device code is built with packed-fp32 instructions disabled.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblcca.so")
DEBUG_LIB = os.path.join(PKG, "liblcca_debug.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-I" + os.path.join(ROOT, "include")]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]


# Per-file device flags.  The attention kernels keep their MFMA accumulators
# in architectural VGPRs (the online-softmax rescale is VALU work on them);
# AGPRs then serve as spill space instead of scratch memory.
EXTRA = {"sparse_attn.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form=1"]}


def sources():
    out = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip"):
            out.append((os.path.join(CSRC, f), True))
        elif f.endswith(".cpp"):
            out.append((os.path.join(CSRC, f), False))
    return out


def _compile(item, verbose, debug):
    src, device = item
    obj = os.path.join(BUILD, "debug" if debug else "", os.path.basename(src) + ".o")
    cmd = [HIPCC] + (DEVICE if device else []) + EXTRA.get(os.path.basename(src), []) + COMMON + \
        (["-DLCCA_DEBUG"] if debug else []) + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (src, r.stdout, r.stderr))
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build_one(debug: bool, verbose: bool = False, jobs: int = 8) -> str:
    """Compile and link one of the two libraries; returns its path."""
    lib = DEBUG_LIB if debug else LIB
    os.makedirs(os.path.join(BUILD, "debug") if debug else BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda it: _compile(it, verbose, debug), sources()))
    for _, warn in results:
        if warn and verbose:
            print(warn, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, jobs: int = 8, debug: bool = True) -> str:
    """Build liblcca.so and (unless debug is False) liblcca_debug.so; returns
    the release library's path."""
    path = build_one(False, verbose, jobs)
    if debug:
        build_one(True, verbose, jobs)
    return path


if __name__ == "__main__":
    print(build(verbose=True, debug="--release-only" not in sys.argv))
