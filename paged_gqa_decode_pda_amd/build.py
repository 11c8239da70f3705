"""Build libpda.so (the gfx950 HIP kernels and the C ABI of include/pda.h) in-tree.

    python paged_gqa_decode_pda_amd/build.py

Run as a script (the package itself refuses to import until the library
exists).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libpda.so")
SOURCES = [os.path.join(HERE, "csrc", n) for n in ("pda_api.hip", "pda_kernels.hip", "pda_attend.hip", "pda_prefill.hip",
                                                  "pda_rope.hip")]
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for every HIP translation unit; hipcc's
# host pass warns that it does not know the feature, which is harmless.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
             # single-lane work-queue claims: keep the compiler from turning
             # them into wave reductions that read the result back at once
             "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


# Per-source extra flags.  The prefill kernel's scores never hold a NaN
# (finite bf16 inputs; masked scores are -inf), so its translation unit is
# built without NaN semantics: fmaxf on matrix-core results is then one
# v_max_f32 instead of two quieting maxima and the maximum (infinities are
# still honoured).  Forcing that kernel's MFMA results into VGPRs
# (-amdgpu-mfma-vgpr-form=1) removes the accumulator copies between AGPRs
# and VGPRs but measured slower at 64 rows per wave.
EXTRA_FLAGS = {"pda_prefill.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra=()) -> str:
    """Compiles every source to an object in parallel, then links libpda.so."""
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(HERE, "csrc", os.path.basename(src) + ".o")
        cmd = [hipcc(), *HIP_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), *extra, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
        objs.append(obj)
    failed = [p.args[-1] for p in procs if p.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    for obj in objs:
        os.remove(obj)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
