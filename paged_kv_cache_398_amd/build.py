"""Build libpa.so (C ABI + gfx950 kernels) in-tree with hipcc.

``python -m paged_kv_cache_398_amd.build`` compiles every source under
``csrc/`` for gfx950 into ``lib/libpa.so`` next to this file.
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libpa.so")
SOURCES = ["pa_kernels.hip", "pa_cache_write.hip", "pa_chunk.hip", "pa_kivi.hip",
           "pa_api.cpp", "pa_block_manager.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled on purpose: the compiler would
# otherwise pair independent fp32 operations into v_pk_* instructions.
# MFMA accumulators are kept in arch VGPRs (-amdgpu-mfma-vgpr-form): in the
# chunk kernels the compiler otherwise places them in AGPRs and copies all
# of them to VGPRs and back on every loop iteration, for the rarely taken
# rescaling of the online softmax.  Only the MFMA kernels are affected.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source to an object (in parallel), then link libpa.so."""
    os.makedirs(LIB_DIR, exist_ok=True)
    obj_dir = tempfile.mkdtemp(prefix="pa_build_")
    try:
        inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
        objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[hipcc(), *HIP_FLAGS, *extra_flags, *inc, "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1, 8)) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB_PATH + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB_PATH)
    finally:
        shutil.rmtree(obj_dir, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
