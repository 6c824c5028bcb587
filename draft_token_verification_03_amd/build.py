"""Build libspecverify.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("sv_api.hip", "sv_verify.hip", "sv_outcome.hip", "sv_tree.hip")]
HEADERS = [os.path.join(HERE, "csrc", f) for f in ("sv_device.h", "sv_internal.h", "sv_accept.h", "sv_tile.h", "sv_stream.h")] + [
    os.path.join(ROOT, "include", "specverify.h")]
LIB = os.path.join(HERE, "libspecverify.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms stay off (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{os.path.join(ROOT, 'include')}",
           f"-I{os.path.join(HERE, 'csrc')}", *SOURCES, "-o", LIB + ".tmp", *(extra or [])]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
