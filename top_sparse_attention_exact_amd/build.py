"""Build libatopk.so (HIP, gfx950) in-tree with hipcc.

    python -m top_sparse_attention_exact_amd.build
"""

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libatopk.so")
SOURCES = ["api.cpp", "select_bucket.hip", "select_exact.hip", "select_row.hip", "select_wide.hip", "decode.hip",
           "decode_fused.hip", "rerank.hip", "choose.cpp", "noalloc.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # hand-written float code must not be turned into packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# The streaming-read yardstick bench.py measures the kernels against (not
# part of the library).
CALIB = os.path.join(HERE, "libatopk_calib.so")
CALIB_SOURCES = [os.path.join(HERE, "calib", "stream_read.hip")]


OBJDIR = os.path.join(ROOT, "_build")


def _run(cmd, what, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + what)


def _source_key(src, includes, flags):
    """Hash of a source, every header next to it or in its include
    directories, and the flags: the name of its cached object."""
    h = hashlib.sha256(" ".join(flags).encode())
    dirs = sorted({os.path.dirname(src)} | set(includes))
    for d in dirs:
        for name in sorted(os.listdir(d)):
            if name.endswith(".h"):
                with open(os.path.join(d, name), "rb") as f:
                    h.update(name.encode() + f.read())
    with open(src, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:20]


def _compile(out, sources, includes, verbose):
    """Each source to an object (in parallel, one hipcc per source), then one
    link into the shared library.  Every source is compiled on every call;
    with ATOPK_BUILD_CACHE=1 an object whose source, headers and flags are
    unchanged is reused from the object directory instead."""
    os.makedirs(OBJDIR, exist_ok=True)
    inc = [a for d in includes for a in ("-I", d)]
    comp = [f for f in FLAGS if f != "-shared"]
    cache = os.environ.get("ATOPK_BUILD_CACHE") == "1"
    objs, todo = [], []
    for s in sources:
        if cache:
            o = os.path.join(OBJDIR, "%s.%s.o" % (os.path.basename(s), _source_key(s, includes, comp)))
            if not os.path.exists(o):
                todo.append((s, o))
        else:
            o = os.path.join(OBJDIR, "%s.%s.%d.o" % (os.path.basename(s), os.path.basename(out), os.getpid()))
            todo.append((s, o))
        objs.append(o)
    jobs = max(1, min(len(sources), int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 4)))
    try:
        with ThreadPoolExecutor(jobs) as pool:
            futs = [pool.submit(_compile_one, comp + inc, s, o, verbose) for s, o in todo]
            for f in futs:
                f.result()
        tmp = out + ".tmp%d" % os.getpid()
        _run([hipcc()] + FLAGS + objs + ["-o", tmp], os.path.basename(out), verbose)
        os.replace(tmp, out)
    finally:
        if not cache:
            for o in objs:
                if os.path.exists(o):
                    os.remove(o)


def _compile_one(flags, src, obj, verbose):
    tmp = obj + ".tmp%d" % os.getpid()
    _run([hipcc()] + flags + ["-c", src, "-o", tmp], os.path.basename(src), verbose)
    os.replace(tmp, obj)


def build(verbose=False):
    _compile(LIB, [os.path.join(CSRC, s) for s in SOURCES], [INCLUDE, CSRC], verbose)
    _compile(CALIB, CALIB_SOURCES, [], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
