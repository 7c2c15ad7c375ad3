"""Build libhta.so for gfx950 with hipcc, in the package directory."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["api.hip", "prefill.hip", "load.hip", "frame.hip", "stream.hip"]
HEADERS = ["device_common.h", "hta_internal.h"]
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
         # keep hipcc from emitting packed fp32 VALU ops
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "libhta.so")
    tmp = out + ".tmp"
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    cmd = [hipcc()] + FLAGS + ["-o", tmp] + srcs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout[-4000:] + res.stderr[-4000:])
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
