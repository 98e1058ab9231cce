"""Build libbpw.so in-tree with hipcc for gfx950 (the only target)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(_HERE, "csrc", f) for f in (
    "bpw_host.cpp", "bpw_gemv.hip", "bpw_gemv_tokens.hip", "bpw_bytelane.hip", "bpw_small_batch.hip", "bpw_dense_head.hip",
    "bpw_quantize.hip", "bpw_measure.hip", "bpw_trit.cpp", "bpw_bitcos.hip", "bpw_bitcos_host.cpp",
    "bpw_static.hip")]
OUT = os.path.join(_HERE, "libbpw.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",  # the dequantisation multiplies are rounded one at a time
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",  # no packed fp32 VALU ops
    "-Wall", "-Wno-unused-function",
]


def build() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = OUT + ".tmp"
    subprocess.run([hipcc, *HIPCC_FLAGS, "-o", tmp, *SOURCES], check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
