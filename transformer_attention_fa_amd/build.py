"""Build libfa.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

    python -m transformer_attention_fa_amd.build

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection turned off, then linked into ``transformer_attention_fa_amd/libfa.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fwd_bf16.hip", "fwd_f32.hip", "decode.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-I", INCLUDE,
    "-I", CSRC,
    # never select packed fp32 instructions (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# per-source extras: the decode kernel rescales its accumulators in place, so
# its matrix-core products accumulate in ordinary VGPRs rather than AGPRs
# (which would need copies in and out on every rescale)
EXTRA_FLAGS = {
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, [])]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every source and link libfa.so; returns its path."""
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            list(ex.map(_compile, SOURCES, objs))
        out = LIB + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
        os.replace(out, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
