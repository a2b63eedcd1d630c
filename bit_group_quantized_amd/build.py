"""Build libq4.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "q4_api.hip")
DEPS = [SRC, os.path.join(HERE, "csrc", "q4_kernels.h"), os.path.join(HERE, "csrc", "q4_chain.h"),
        os.path.join(HERE, "csrc", "q4_attn.h"),
        os.path.join(ROOT, "include", "q4.h")]
LIB = os.path.join(HERE, "libq4.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE division for the quantizer's (max-min)/15 and (w-b)/s
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    "-Wall",
]


# measurement support for the benchmark (a plain HBM stream-read kernel)
CEILING_SRC = os.path.join(HERE, "csrc", "q4_stream_ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libq4_ceiling.so")


def _hipcc(src: str, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["hipcc", *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile libq4.so (the library) and libq4_ceiling.so (the benchmark's
    stream-read ceiling kernel) for gfx950."""
    _hipcc(CEILING_SRC, CEILING_LIB, verbose)
    return _hipcc(SRC, LIB, verbose)


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
