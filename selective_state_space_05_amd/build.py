"""Build libmssm.so (hipcc, gfx950) in this package directory.

Usage:  python -m selective_state_space_05_amd.build [--verbose]

Every HIP source is compiled with packed-FP32 instruction selection turned
off (the kernels are written for scalar v_*_f32 arithmetic) and linked into
one shared library exporting the C ABI of include/mssm.h.
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "libmssm")
LIB = os.path.join(PKG, "libmssm.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-fvisibility=hidden", "-DMSSM_BUILDING_LIBRARY",
    "-I" + INCLUDE, "-I" + CSRC,
]


def source_hash() -> str:
    """16 hex digits of a SHA-256 over every file under csrc/ and include/
    (names and contents, in sorted order) and the compile flags.  build()
    compiles it into the library (mssm_source_hash()), and the binding
    refuses a library whose hash differs from that of the sources beside
    it."""
    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            path = os.path.join(d, name)
            if os.path.isfile(path):
                h.update(name.encode() + b"\0")
                with open(path, "rb") as f:
                    h.update(f.read())
                h.update(b"\0")
    # the include paths are absolute: hash them relative to the repository,
    # so a copy of the tree elsewhere hashes the same
    flags = [f.replace(ROOT, "<root>") for f in COMMON]
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def sources():
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith(".hip") or name.endswith(".cpp"):
            out.append(os.path.join(CSRC, name))
    return out


def _compile(src, verbose, extra=()):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-x", "hip", "-c", src, "-o", obj] + COMMON + list(extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    noise = ("packed-fp32-ops", "not a recognized feature", "warning: unknown")
    msgs = [ln for ln in r.stderr.splitlines() if not any(n in ln for n in noise)]
    if verbose and msgs:
        print("\n".join(msgs))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libmssm.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    tag = ['-DMSSM_SOURCE_HASH="%s"' % source_hash()]

    def one(src):
        # the hash goes into the host front end only
        return _compile(src, verbose, tag if src.endswith("mssm_api.cpp") else ())

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
