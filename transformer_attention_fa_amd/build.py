"""Build libfa.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

    python -m transformer_attention_fa_amd.build [--debug-barriers]

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection turned off, then linked into ``transformer_attention_fa_amd/libfa.so``.

``--debug-barriers`` builds ``libfa_debug_barriers.so`` instead: the same
library with FA_DEBUG_BARRIERS defined, which puts one more barrier (after a
full wait for the wave's memory operations) between the two phases of every
period of the prefill kernel.  Its arithmetic is the same, so its outputs must
match libfa.so bit for bit; a difference points at a race between the phases
of different waves.  Point ``FA_LIBRARY`` at it to run any caller against it.
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
DEBUG_LIB = os.path.join(PKG, "libfa_debug_barriers.so")
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
# (which would need copies in and out on every rescale); and its one-lane
# chunk-queue atomic stays a plain atomic (the atomic optimizer's wave
# reduction would wait for the result at once, before the chunk's loads)
EXTRA_FLAGS = {
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
}


def _compile(src: str, obj: str, defines=()) -> None:
    cmd = [HIPCC, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), *(f"-D{d}" for d in defines)]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False, debug_barriers: bool = False) -> str:
    """Compile every source and link libfa.so (or, with debug_barriers, the
    race-hunting libfa_debug_barriers.so); returns its path."""
    lib = DEBUG_LIB if debug_barriers else LIB
    defines = ("FA_DEBUG_BARRIERS",) if debug_barriers else ()
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            list(ex.map(lambda so: _compile(so[0], so[1], defines), zip(SOURCES, objs)))
        out = lib + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
        os.replace(out, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, debug_barriers="--debug-barriers" in sys.argv[1:])
    sys.exit(0)
