"""Compile liblightning.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Every source under csrc/ is compiled on each call (hipcc cross-compiles
without a GPU) and linked into ``liblightning.so`` next to this file, except
``la_stream.hip``, the benchmark's HBM streaming references, which becomes
``libla_stream.so`` (C ABI in include/la_stream.h).
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "liblightning.so")
# Measurement helper for the benchmark (HBM streaming references), its own library.
STREAM_SOURCE = "la_stream.hip"
STREAM_LIB_PATH = os.path.join(HERE, "libla_stream.so")
SOURCES = ["la_api.cpp", "la_fwd_f32.hip", "la_fwd_bf16.hip", "la_bwd_bf16.hip", "la_bwd_f32.hip", "la_decode.hip",
           "la_noalloc.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions stay disabled: every float operation is scalar.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "unknown target feature" not in l
                    and "-packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    """Compile all sources and link liblightning.so (and the benchmark's
    streaming-reference library libla_stream.so); returns liblightning's path."""
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="la_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1, 8)) as ex:
            outs = list(ex.map(_run, cmds))
        tmp_lib = LIB_PATH + ".tmp"
        outs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]))
        os.replace(tmp_lib, LIB_PATH)
        tmp_stream = STREAM_LIB_PATH + ".tmp"
        outs.append(_run([hipcc, *HIP_FLAGS, "-shared", os.path.join(CSRC, STREAM_SOURCE), "-o", tmp_stream]))
        os.replace(tmp_stream, STREAM_LIB_PATH)
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
