"""Builds libdecode_attn.so (the attention library) and libdecode_attn_probe.so
(an HBM read probe used by the benchmark) for gfx950 with hipcc, in-tree.

Usage: python -m decode_attention_amd.build [--verbose]
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "sliding.hip", "global.hip", "append.hip", "multiquery.hip"]
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


# Per-file flags. The global kernel's 6-step descriptor loop must unroll fully
# (its ring and descriptors live in registers only then); the pre-norm
# variant's body exceeds LLVM's default size limit for a requested unroll.
FILE_FLAGS = {"global.hip": ["-mllvm", "-pragma-unroll-threshold=60000"]}


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src, verbose, extra):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *HIP_FLAGS, *FILE_FLAGS.get(src, []), *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stderr or "").splitlines() if "not a recognized feature" not in l]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def _link(objs, name):
    out = os.path.join(LIBDIR, name)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link of {name} failed:\n" + res.stderr)
    os.replace(tmp, out)
    return out


def build(verbose=False, extra=()):
    """Compiles every source and links both libraries; returns the attention
    library's path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose, list(extra)), srcs)))
    _link([objs[s] for s in PROBE_SOURCES], "libdecode_attn_probe.so")
    return _link([objs[s] for s in SOURCES], "libdecode_attn.so")


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv,
                extra=["-Rpass-analysis=kernel-resource-usage"] if "--usage" in sys.argv else []))
