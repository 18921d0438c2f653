"""Build libidx.so (the indexer's C ABI and its gfx950 HIP kernels), libidx_debug.so
(the same sources with -DIDX_DEBUG: every clamped device-resident value is recorded
for idx_debug_flags) and libidx_calib.so (the measurement kernels of
include/idx_calib.h) in-tree with hipcc.

Every HIP source compiles for gfx950 only, with packed-fp32 instruction selection
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``; hipcc's host pass
warns that it does not know the feature, which is harmless). Objects go to
``_build/`` next to this file and the libraries beside it.

    python -m sparse_attention_indexer_mxfp4_amd.build [-v]
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libidx.so")
DEBUG_LIB = os.path.join(PKG, "libidx_debug.so")
CALIB_SRC = os.path.join(CSRC, "calib", "calib.hip")
CALIB_LIB = os.path.join(PKG, "libidx_calib.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Wall", "-Wno-unused-function"]
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-gpu-flush-denormals-to-zero"]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, extra: list[str], out_dir: str = BUILD) -> tuple[str, str]:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *extra]
    if src.endswith(".hip"):
        cmd += DEVICE + ["-x", "hip"]
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, extra: list[str] | None = None, jobs: int = 8, debug: bool = True) -> str:
    """Compile every source and link libidx.so, libidx_debug.so (unless debug is False)
    and libidx_calib.so; returns libidx.so's path. Always rebuilds."""
    debug_dir = os.path.join(BUILD, "debug")
    os.makedirs(debug_dir, exist_ok=True)
    extra = list(extra or [])
    release = sources() + [CALIB_SRC]
    jobs_list = [(s, extra, BUILD) for s in release]
    if debug:
        jobs_list += [(s, extra + ["-DIDX_DEBUG"], debug_dir) for s in sources()]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda j: _compile(*j), jobs_list))
    if verbose:
        for obj, err in results:
            noise = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln]
            if noise:
                print(obj, "\n".join(noise), file=sys.stderr)
    objs = [o for o, _ in results]
    n = len(release)
    _link(objs[:n - 1], LIB)
    _link(objs[n - 1:n], CALIB_LIB)
    if debug:
        _link(objs[n:], DEBUG_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
