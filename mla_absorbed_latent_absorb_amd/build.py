"""Build the gfx950 HIP library libmla_absorb.so in-tree with hipcc.

    python -m mla_absorbed_latent_absorb_amd.build

compiles every kernel and the C-ABI host code for gfx950 and writes
``mla_absorbed_latent_absorb_amd/libmla_absorb.so``.  hipcc cross-compiles, so
this also runs on a machine without a GPU.
"""

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
REPO = os.path.dirname(PKG_DIR)
LIB_NAME = "libmla_absorb.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["decode_latent.hip", "decode_latent_wide.hip", "decode_latent_fp8.hip", "proj_combine.hip", "cache_append.hip", "decode_step_fused.hip",
           "naive_decode.hip", "noalloc_scratch.hip", "mla_absorb.cpp"]

# -packed-fp32-ops: plain fp32 code is compiled without v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def build(verbose=False):
    """Compile libmla_absorb.so for gfx950; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(REPO, "include")] + \
        [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
