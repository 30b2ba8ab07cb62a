"""Build libatopk.so (HIP, gfx950) in-tree with hipcc.

    python -m top_sparse_attention_exact_amd.build
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libatopk.so")
SOURCES = ["api.cpp", "select_bucket.hip", "select_exact.hip", "select_row.hip", "select_wide.hip", "decode.hip",
           "decode_fused.hip", "rerank.hip", "choose.cpp"]

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


def _compile(out, sources, includes, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + FLAGS + [a for inc in includes for a in ("-I", inc)] + sources + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    os.replace(tmp, out)


def build(verbose=False):
    _compile(LIB, [os.path.join(CSRC, s) for s in SOURCES], [INCLUDE, CSRC], verbose)
    _compile(CALIB, CALIB_SOURCES, [], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
