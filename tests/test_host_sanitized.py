"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's sources are compiled with both sanitizers on the host pass (the gfx950
device code is built as usual, without them; nothing here launches a kernel), linked with
tests/host_abi_check.cpp, and run.
The driver exercises un-delay, the streaming hand-off and its stop guard (200 random
utterances pushed and read in random pieces through exactly sized buffers, checked against
the one-shot un-delay), the workspace size rules on valid, unsupported and overflowing
shapes, context creation where no usable device exists, and the null-context checks of
every call that takes a context.  Any out-of-bounds access, use after free, leak in the
library's own code or undefined arithmetic fails the test.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "autoregressive_codebook_tts_amd", "csrc")
SOURCES = ["api.hip", "prefill.hip", "load.hip", "frame.hip", "stream.hip"]
# every sanitizer flag applies to the host pass only
FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-std=c++17", "-O1", "-g",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
         "-I", os.path.join(ROOT, "include")]
# allocations the HIP and HSA runtimes keep for the process lifetime are theirs, not the library's
SUPPRESSIONS = "leak:libamdhip64\nleak:libhsa-runtime64\nleak:libhsakmt\nleak:librocprofiler\nleak:libamd_comgr\n"


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_host_abi_under_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")

    def compile_one(src):
        path = os.path.join(CSRC, src) if src.endswith(".hip") else src
        obj = os.path.join(tmp_path, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "c++"]
        r = subprocess.run([hipcc] + lang + FLAGS + ["-c", path, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, f"compiling {src}:\n{r.stderr[-3000:]}"
        return obj

    srcs = SOURCES + [os.path.join(ROOT, "tests", "host_abi_check.cpp")]
    with ThreadPoolExecutor(max_workers=4) as pool:
        objs = list(pool.map(compile_one, srcs))
    exe = os.path.join(tmp_path, "host_abi_check")
    r = subprocess.run([hipcc] + FLAGS + objs + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, f"linking:\n{r.stderr[-3000:]}"

    supp = os.path.join(tmp_path, "lsan.supp")
    with open(supp, "w") as f:
        f.write(SUPPRESSIONS)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0:abort_on_error=0"
    env["LSAN_OPTIONS"] = f"suppressions={supp}:print_suppressions=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # never a device, also where one exists
    r = subprocess.run([exe, "--no-device"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"rc {r.returncode}\nstdout:\n{r.stdout[-2000:]}\nstderr:\n{r.stderr[-6000:]}"
    assert "host ABI checks passed" in r.stdout
