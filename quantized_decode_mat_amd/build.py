"""Build libxq.so in-tree with hipcc for gfx950.

    python -m quantized_decode_mat_amd.build

Every HIP translation unit is compiled with packed-FP32 instructions turned
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``); the float code
here is plain scalar code. Code objects are emitted as version 5, which the
HIP runtime bundled with the PyTorch wheel (the runtime libxq shares with
torch in one process) loads.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libxq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [
    "q8k_quantize.hip",
    "gemv_q4k.hip",
    "gemv_iq4nl.hip",
    "gemm_q4k.hip",
    "repack_iq4nl.hip",
    "route_experts.hip",
    "stream_read.hip",
    "workspace.cpp",
    "xq_api.cpp",
]

FLAGS = [
    "--offload-arch=gfx950",
    "-mcode-object-version=5",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    """Compile every source and link libxq.so; returns its path."""
    with tempfile.TemporaryDirectory(prefix="xq_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".hip"):
                cmd[1:1] = ["-x", "hip"]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
            if r.returncode != 0:
                sys.stderr.write(r.stderr)
                raise RuntimeError("hipcc failed on %s" % src)
            objs.append(obj)
        tmp_lib = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-mcode-object-version=5", "-shared", "-fPIC",
               *objs, "-o", tmp_lib]
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
