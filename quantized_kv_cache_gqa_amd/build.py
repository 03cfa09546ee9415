"""Build the HIP library libkvq.so in-tree for gfx950 with hipcc.

Also builds libkvq_test.so: the same kernels with the host layer compiled
with -DKVQ_TEST_HOOKS, which adds kvq_test_set_team_hooks (a smaller team
wait budget and a silent team member, to force a run-out from the host).
Only the tests load it; the product library has no such hook.

Usage: python -m quantized_kv_cache_gqa_amd.build   (or call build()).
Every source is compiled on each call (the caller decides when to rebuild).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvq.so")
TEST_LIB = os.path.join(PKG, "libkvq_test.so")
SOURCES = ["kvq_api.cpp", "kvq_quantize.hip", "kvq_decode.hip", "kvq_decode_mfma.hip", "kvq_decode_two.hip"]
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-mcode-object-version=5",
    # packed FP32 instructions stay off (see the toolchain notes in the design doc)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{os.path.join(PKG, '..', 'include')}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src: str, obj: str, extra=()) -> None:
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = [os.path.join(out_dir, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    hooks_obj = os.path.join(out_dir, "kvq_api_test_hooks.o")
    jobs = [(s, o, ()) for s, o in zip(SOURCES, objs)] + [("kvq_api.cpp", hooks_obj, ("-DKVQ_TEST_HOOKS",))]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs, LIB)
    _link([hooks_obj] + objs[1:], TEST_LIB)
    if verbose:
        print(f"built {LIB} and {TEST_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
