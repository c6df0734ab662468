"""Build step: compile the gfx950 HIP sources into the in-tree libfp8bs.so.

Run ``python -m fp8_block_scaled_05_amd.build`` (or ``__graft_entry__.build()``).
hipcc cross-compiles for gfx950 without a GPU present.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfp8bs.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["status.cpp", "quant.hip", "dequant.hip", "tensor_quant.hip", "gemm.hip"]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the generated code.
# Division and sqrt stay correctly rounded (hipcc's default); no fast-math.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8bs)")


def build(verbose=False, extra_flags=()):
    out_tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"libfp8bs build failed:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    os.replace(out_tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
