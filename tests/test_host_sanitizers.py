"""The library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, without a GPU.  libabs.so is rebuilt with both
sanitizers on its host pass only (each flag behind -Xarch_host; the device
code is the same), then
  1. tests/c/host_calls.c, built with the same sanitizers, calls every
     host-side function of abs.h with valid and invalid arguments;
  2. the binding's ABI tests and bench.py's host tests run in a subprocess
     with the sanitizer runtime preloaded and the binding pointed at this
     build (its gcc-linked C test is left to test_abi.py itself).
A sanitizer report, or any failure, fails the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from block_sparse_attention_abs_amd import build as B  # noqa: E402

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}
CLANG = "/opt/rocm/llvm/bin/clang"


def _runtime():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return rt[-1] if rt else None


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    if not os.path.exists(B.HIPCC) or not os.path.exists(CLANG) or _runtime() is None:
        pytest.skip("hipcc, clang or the clang sanitizer runtime not found")
    d = tmp_path_factory.mktemp("san")
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g", *HOST_SAN]
    procs, objs = [], []
    for src in B.SOURCES:
        obj = str(d / (src + ".o"))
        cmd = [B.HIPCC, *flags, "-I", B.CSRC, "-c", os.path.join(B.CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p in procs:
        log, _ = p.communicate(timeout=900)
        assert p.returncode == 0, log[-3000:]
    lib = str(d / "libabs.so")
    subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN[:4], "-shared-libasan",
                    "-o", lib, *objs], check=True, timeout=600)
    return lib


def _env(extra):
    env = dict(os.environ)
    env.update(ENV)
    env.update(extra)
    return env


def test_c_host_calls_under_sanitizers(san_lib, tmp_path):
    exe = str(tmp_path / "host_calls")
    lib_dir = os.path.dirname(san_lib)
    subprocess.run([CLANG, "-std=c11", "-Wall", "-Werror", "-g",
                    "-fsanitize=address,undefined", "-shared-libasan", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "host_calls.c"), "-L", lib_dir, "-labs",
                    f"-Wl,-rpath,{lib_dir}", "-o", exe], check=True, timeout=300)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env=_env({"LD_LIBRARY_PATH": os.path.dirname(_runtime())}))
    assert r.returncode == 0 and "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    assert r.stdout.count("\n") >= 10


def test_binding_host_tests_under_sanitizers(san_lib, tmp_path):
    plugin = tmp_path / "san_lib_plugin.py"
    plugin.write_text("import block_sparse_attention_abs_amd.abs as A\n"
                      f"A.LIB_PATH = {san_lib!r}\n")
    cmd = [sys.executable, "-m", "pytest", "-p", "san_lib_plugin", "-s", "-q", "-m", "not gpu",
           "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py"),
           os.path.join(ROOT, "tests", "test_bench_host.py"),
           "--deselect", "tests/test_abi.py::test_host_calls_from_plain_c"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900, cwd=ROOT,
                       env=_env({"LD_PRELOAD": _runtime(), "PYTHONPATH": f"{tmp_path}:{ROOT}"}))
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
