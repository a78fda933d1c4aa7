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
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
REPO = os.path.dirname(PKG_DIR)
LIB_NAME = "libmla_absorb.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["decode_latent.hip", "decode_latent16.hip", "decode_latent_wide.hip", "decode_latent_fp8.hip",
           "proj_combine.hip", "cache_append.hip", "decode_step_fused.hip", "naive_decode.hip",
           "noalloc_scratch.hip", "mla_absorb.cpp"]

# -packed-fp32-ops: plain fp32 code is compiled without v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-source flags.  decode_latent16.hip: MFMA accumulators in ordinary VGPRs
# (its rare O rescale is plain VALU work on them; with AGPR accumulators the
# compiler copies all 128 of them to VGPRs and back on every tile).
EXTRA_FLAGS = {
    "decode_latent16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _check(res, what):
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({res.returncode}):\n{err}")
    return err


def build(verbose=False, csrc=CSRC, include=os.path.join(REPO, "include"), out=LIB_PATH):
    """Compile libmla_absorb.so for gfx950 (one object per source, compiled in
    parallel, then linked); returns its path."""
    with tempfile.TemporaryDirectory(prefix="mla_build_") as tmpdir:
        jobs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            cmd = [hipcc()] + HIPCC_FLAGS + EXTRA_FLAGS.get(src, []) + ["-I", include, "-c",
                                                                        os.path.join(csrc, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            jobs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        errs = []
        for src, obj, proc in jobs:
            stdout, stderr = proc.communicate()
            errs.append(_check(subprocess.CompletedProcess(proc.args, proc.returncode, stdout, stderr), src))
        tmp = out + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for _, o, _ in jobs] + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        errs.append(_check(subprocess.run(cmd, capture_output=True, text=True), "link"))
    if verbose and any(e.strip() for e in errs):
        print("\n".join(e for e in errs if e.strip()), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
