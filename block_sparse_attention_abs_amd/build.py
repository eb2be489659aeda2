"""Build libabs.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m block_sparse_attention_abs_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libabs.so")
SOURCES = ["centroid.hip", "select.hip", "decode.hip", "calibrate.hip", "gather.hip", "abs_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 math is kept off on this hardware
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division/sqrt: the INT4 quantizer's codes depend on it
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, out: str = LIB, defines=(), objdir: str = OBJ, csrc: str = CSRC) -> str:
    """Compile every source under `csrc` and link `out`; `defines` are extra -D tuning macros."""
    os.makedirs(objdir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC, *FLAGS, "-I", csrc, *[f"-D{d}" for d in defines], "-c", os.path.join(csrc, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                 text=True)))
    objs, errors = [], []
    for src, obj, p in procs:
        log, _ = p.communicate()
        if verbose or p.returncode != 0:
            txt = "\n".join(l for l in log.splitlines() if "packed-fp32-ops" not in l and l.strip())
            if txt:
                print(f"--- {src}\n{txt}", file=sys.stderr)
        if p.returncode != 0:
            errors.append(src)
        objs.append(obj)
    if errors:
        raise RuntimeError(f"hipcc failed for {errors}")
    tmp = out + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
