"""Build libattn.so (the gfx950 kernels and their C ABI) in-tree with hipcc,
and its debug sibling libattn_debug.so (the same sources compiled with
ATTN_DEBUG_TRACE: the per-tile softmax trace of include/attn_debug.h)."""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "attn.hip")
LIB = os.path.join(PKG, "libattn.so")
DEBUG_LIB = os.path.join(PKG, "libattn_debug.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-shared", "-fPIC",
    # keep the compiler from forming packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _command(out, extra_flags=(), debug=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = list(HIPCC_FLAGS) + list(extra_flags)
    if debug:
        flags.append("-DATTN_DEBUG_TRACE")
    return [hipcc, *flags, "-I", os.path.join(ROOT, "include"), SRC, "-o",
            out + ".tmp"]


def build(verbose=False, extra_flags=(), debug=False):
    """Compile one library (the release one, or the debug one)."""
    out = DEBUG_LIB if debug else LIB
    cmd = _command(out, extra_flags, debug)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    os.replace(out + ".tmp", out)
    return out


def build_all(verbose=False):
    """Compile both libraries, the two hipcc runs side by side."""
    jobs = []
    for debug in (False, True):
        out = DEBUG_LIB if debug else LIB
        cmd = _command(out, (), debug)
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                           stderr=subprocess.STDOUT,
                                           text=True)))
    failed = []
    for out, p in jobs:
        text = p.communicate()[0]
        if p.returncode != 0:
            sys.stderr.write(text)
            failed.append(os.path.basename(out))
        else:
            os.replace(out + ".tmp", out)
    if failed:
        raise RuntimeError(f"hipcc failed for {', '.join(failed)}")
    return LIB, DEBUG_LIB


if __name__ == "__main__":
    print(build_all(verbose=True))
