"""Builds the ABI layer of libidx (csrc/api.cpp, csrc/validate.cpp, unchanged) with the
host compiler under AddressSanitizer and UndefinedBehaviorSanitizer, linked against
host_stubs.cpp instead of the HIP runtime and the kernels. Host code only: no HIP
source is compiled here.

    python tests/host_asan/build.py OUT.so
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "sparse_attention_indexer_mxfp4_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SANITIZE = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer"]


def compiler() -> str | None:
    return shutil.which("g++")


def asan_runtime(cxx: str) -> str | None:
    """Path of the compiler's shared ASan runtime (preloaded into an uninstrumented
    Python), or None."""
    out = subprocess.run([cxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def build(out: str) -> str:
    cxx = compiler()
    if cxx is None:
        raise RuntimeError("g++ not found")
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "validate.cpp"), os.path.join(HERE, "host_stubs.cpp")]
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), *SANITIZE, *srcs, "-o", out, "-Wl,--no-undefined"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(HERE, "libidx_host_asan.so")))
