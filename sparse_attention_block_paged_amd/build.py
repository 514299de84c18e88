"""Build libmm3idx.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmm3idx.so")
ARCH = "gfx950"

# Packed-FP32 VALU forms are kept out of the generated code (-packed-fp32-ops).
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source additions.  decode_score: max() without NaN canonicalisation
# (block scores of rows whose q or keys hold NaN are unspecified) and MFMA
# results in ordinary VGPRs (no accumulator-register reads per tile); together
# they take ~8% of the vector instructions out of the NVFP4 scorer's loop.
SOURCE_FLAGS = {
    "decode_score.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    # prefill_score: its page copies set M0 in inline assembly, so no
    # compiler-generated code there may read M0; the wave-level combining of
    # the fused selection's counter atomics would (v_writelane with an M0
    # lane index), so atomics are left as written
    "prefill_score.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [cc, *HIP_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), "-I", INCLUDE, "-I", CSRC,
               "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write("\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed on: " + ", ".join(os.path.basename(f) for f in failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                          stderr=subprocess.DEVNULL if not verbose else None)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
