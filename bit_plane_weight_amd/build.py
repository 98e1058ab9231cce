"""Build libbpw.so in-tree with hipcc for gfx950 (the only target): every source compiled to an object
(in parallel), then linked."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(_HERE, "csrc", f) for f in (
    "bpw_host.cpp", "bpw_gemv.hip", "bpw_gemv_tokens.hip", "bpw_bytelane.hip", "bpw_small_batch.hip", "bpw_dense_head.hip",
    "bpw_quantize.hip", "bpw_measure.hip", "bpw_trit.cpp", "bpw_bitcos.hip", "bpw_bitcos_host.cpp",
    "bpw_static.hip")]
OUT = os.path.join(_HERE, "libbpw.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",  # the dequantisation multiplies are rounded one at a time
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",  # no packed fp32 VALU ops
    "-Wall", "-Wno-unused-function",
]

# Kernel arguments preloaded into SGPRs (gfx950): a workgroup's first table read then waits for one
# scalar load instead of two (the argument, then the table entry). Measured in kernel traces of the
# grouped GEMV's small plans (one 640 x 2560 matrix to one layer): 0.28-0.32 us less per launch; the
# 210-matrix decode step is level. The code object keeps the compiler's fallback that loads the
# arguments itself where the firmware does not preload them. The quantiser is built without it: its
# trace median rose by 0.16-0.2 us with it.
KERNARG_PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
NO_PRELOAD = {"bpw_quantize.hip"}


def flags_for(src: str) -> list:
    name = os.path.basename(src)
    return HIPCC_FLAGS + (KERNARG_PRELOAD if name.endswith(".hip") and name not in NO_PRELOAD else [])


def build() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    work = tempfile.mkdtemp(prefix="bpw_build_")
    try:
        objs = [os.path.join(work, os.path.basename(s) + ".o") for s in SOURCES]

        def compile_one(i: int) -> None:
            subprocess.run([hipcc, *flags_for(SOURCES[i]), "-c", SOURCES[i], "-o", objs[i]], check=True)

        with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
            list(ex.map(compile_one, range(len(SOURCES))))
        tmp = OUT + ".tmp"
        subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
        os.replace(tmp, OUT)
    finally:
        shutil.rmtree(work, ignore_errors=True)
    return OUT


if __name__ == "__main__":
    print(build())
