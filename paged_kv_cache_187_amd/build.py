"""Build libpagedattn.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc."""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# Read-bandwidth probes (bench.py's ceiling line only; not part of the C ABI above).
PROBE_SRC = os.path.join(PKG, "probe", "pa_probe.hip")
PROBE_PATH = os.path.join(PKG, "libpaprobe.so")
# (source, object, extra flags): the decode source is built twice, the second time for the
# kernels of the fused append + decode.
SOURCES = [("pa_append.hip", "pa_append.o", []), ("pa_copy.hip", "pa_copy.o", []),
           ("pa_decode.hip", "pa_decode.o", []),
           ("pa_decode.hip", "pa_decode_append.o", ["-DPA_DECODE_APPEND=1"]),
           ("pa_scratch.hip", "pa_scratch.o", []), ("pa_api.cpp", "pa_api.o", [])]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # Keep the compiler from forming packed-FP32 (v_pk_*_f32) instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)


def build(verbose=False, extra_flags=()):
    """Compile every source for gfx950 and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src, obj_name, flags in SOURCES:
        obj = os.path.join(BUILD, obj_name)
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *COMMON, *extra_flags, *flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    ptmp = PROBE_PATH + ".tmp"
    _run([HIPCC, *COMMON, *extra_flags, "-shared", "-x", "hip", PROBE_SRC, "-o", ptmp], verbose)
    os.replace(ptmp, PROBE_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
