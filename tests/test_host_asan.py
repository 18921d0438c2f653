"""The ABI layer (csrc/api.cpp and csrc/validate.cpp: every entry point's argument
checks, size arithmetic and launch dispatch) under AddressSanitizer and
UndefinedBehaviorSanitizer.

tests/host_asan/build.py builds those two files unchanged with the host compiler and
the sanitizers, linked against stand-ins for the HIP runtime and the kernel launchers
(tests/host_asan/host_stubs.cpp). tests/test_abi_cpu.py then runs against that build
in a child Python with the ASan runtime preloaded: the argument checks with no device,
and with a pretend gfx950, every valid call of every entry point reaching its
launchers with arguments the kernels can use. Any sanitizer report fails the run."""

import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _builder():
    spec = importlib.util.spec_from_file_location("host_asan_build", os.path.join(ROOT, "tests", "host_asan",
                                                                                   "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_layer_under_sanitizers(tmp_path):
    hb = _builder()
    cxx = hb.compiler()
    if cxx is None:
        pytest.skip("no host C++ compiler")
    runtime = hb.asan_runtime(cxx)
    if runtime is None:
        pytest.skip("the host compiler has no shared ASan runtime")
    so = hb.build(str(tmp_path / "libidx_host_asan.so"))
    syms = subprocess.run(["nm", "-D", so], capture_output=True, text=True).stdout
    assert "__asan_init" in syms and "__ubsan_handle" in syms, "the build is not instrumented"

    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(x for x in (runtime, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["IDX_TEST_LIB"] = so
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q", "-rs",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert "needs the host build" not in out, "the host-build tests were skipped"
