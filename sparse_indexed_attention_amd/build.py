"""Build libdsa.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m sparse_indexed_attention_amd.build              # or build() from Python
    python -m sparse_indexed_attention_amd.build --timeline   # libdsa_timeline.so

The --timeline variant is the same sources compiled with -DDSA_TIMELINE: its kernels record
per-workgroup phase stamps into a buffer registered through include/dsa_timeline.h.  It is a
measurement tool (profile_counters.py timeline), never what the binding loads by default.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
LIB_TIMELINE = os.path.join(HERE, "libdsa_timeline.so")
# (source, object, extra flags): the indexer compiles as four parts, one per group of its
# kernel's instantiations, so that they build in parallel
SOURCES = [("api.cpp", "api", []), ("sfa.hip", "sfa", []), ("store.hip", "store", []),
           ("prolog.hip", "prolog", []), ("noalloc.hip", "noalloc", [])] + \
          [("indexer.hip", f"indexer_p{k}", [f"-DDSA_INDEXER_PART={k}"]) for k in range(4)]
LIBS = ["-L/opt/rocm/lib", "-lrocblas", "-Wl,-rpath,/opt/rocm/lib"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
        "-I", os.path.join(HERE, "..", "include"),
    ]


def _compile(cc, src, obj, extra, verbose):
    cmd = [cc, *flags(), *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def _quiet(stderr: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature name and says so; not an error
    return "\n".join(l for l in stderr.splitlines()
                     if "packed-fp32-ops" not in l or "error" in l.lower())


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Compile every source to an object in parallel (build/ next to this file), then link.
    timeline=True builds the stamp-recording variant libdsa_timeline.so (objects in
    build/timeline/)."""
    from concurrent.futures import ThreadPoolExecutor
    cc = hipcc()
    objdir = os.path.join(HERE, "build", "timeline") if timeline else os.path.join(HERE, "build")
    lib = LIB_TIMELINE if timeline else LIB
    macro = ["-DDSA_TIMELINE"] if timeline else []
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1, 16)) as ex:
        for s, o, extra in SOURCES:
            obj = os.path.join(objdir, o + ".o")
            jobs.append((o, ex.submit(_compile, cc, os.path.join(CSRC, s), obj, macro + extra, verbose)))
    for s, j in jobs:
        res = j.result()
        err = _quiet(res.stderr)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {s} ({res.returncode}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = lib + ".tmp"
    objs = [os.path.join(objdir, o + ".o") for _, o, _ in SOURCES]
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *LIBS, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{_quiet(res.stderr)}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, timeline="--timeline" in sys.argv[1:]))
