"""Build libfedavg.so (the HIP library for gfx950) in-tree with hipcc."""

import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libfedavg.so")
SOURCES = [os.path.join(HERE, "csrc", "fedavg_kernels.hip"),
           os.path.join(HERE, "csrc", "topk.hip"),
           os.path.join(HERE, "csrc", "fedavg_api.hip")]
HEADERS = [os.path.join(HERE, "csrc", "fedavg_internal.h"),
           os.path.join(ROOT, "include", "fedavg.h")]

# IEEE fp32 arithmetic: no fast-math, no FMA contraction beyond the explicit
# fmaf calls, denormals kept (the gfx950 default); packed fp32 instructions
# are switched off.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libfedavg.so")
    return path


# Measurement kernels for the benchmark's HBM ceilings (byte patterns of the
# aggregation kernels without their arithmetic); not part of the library.
CEILING_PATH = os.path.join(HERE, "libhbm_ceiling.so")
CEILING_SOURCES = [os.path.join(HERE, "csrc", "hbm_ceiling.hip")]


def _compile(sources, path, verbose):
    fd, tmp = tempfile.mkstemp(prefix=os.path.basename(path) + ".", suffix=".so.tmp", dir=HERE)
    os.close(fd)
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", tmp] + sources
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
        os.replace(tmp, path)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)


def build(verbose=False):
    """Compile the library and the benchmark's ceiling kernels; always
    rebuilds.  Returns the path of the library."""
    _compile(SOURCES, LIB_PATH, verbose)
    _compile(CEILING_SOURCES, CEILING_PATH, verbose)
    return LIB_PATH


def is_stale():
    """True when the library is missing or older than one of its sources."""
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
