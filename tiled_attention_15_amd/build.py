"""Compile the HIP kernels and the C ABI into tiled_attention_15_amd/libfa_hip.so.

hipcc cross-compiles for gfx950 without a GPU present.  Packed-fp32 VALU
instructions are disabled for all device code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa_hip.so")
SOURCES = [os.path.join(CSRC, "fa_api.cpp"), os.path.join(CSRC, "fa_fwd_kernel.hip"),
           os.path.join(CSRC, "fa_naive.hip"), os.path.join(CSRC, "fa_bwd.hip"),
           os.path.join(CSRC, "fa_fwd_ext.hip"), os.path.join(CSRC, "fa_bwd256.hip"),
           os.path.join(CSRC, "fa_fwd_diag.hip"), os.path.join(CSRC, "fa_clock.hip"),
           os.path.join(CSRC, "fa_bwd_noalloc.hip"), os.path.join(CSRC, "fa_fwd_drop.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Kernels whose MFMA accumulators are also worked on by vector instructions:
# the VGPR form of the MFMA instructions keeps those accumulators in VGPRs
# instead of AGPRs, which removes the AGPR<->VGPR copies the compiler
# otherwise inserts around every softmax step (and lowers register use).
PER_SOURCE_FLAGS = {
    "fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "fa_fwd_ext.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}
ARCH = "gfx950"


def hipcc_flags(extra=()):
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", *extra]


def build(out=LIB, extra=(), verbose=False, jobs=None):
    """Build the shared library (always recompiles) and return its path.
    The sources compile in parallel (one hipcc process each)."""
    tmpdir = os.path.join(PKG, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    cmds = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        per = PER_SOURCE_FLAGS.get(os.path.basename(src), [])
        cmds.append((src, [HIPCC, *hipcc_flags(extra), *per, *lang, "-c", src, "-o", obj]))
        objs.append(obj)

    def compile_one(item):
        src, cmd = item
        if verbose:
            print(" ".join(cmd), flush=True)
        return src, subprocess.run(cmd, capture_output=True, text=True)

    if jobs is None:
        jobs = min(len(cmds), max(1, min(8, len(os.sched_getaffinity(0)))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, r in ex.map(compile_one, cmds):
            if r.returncode != 0:
                raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    tmp = out + ".tmp%d" % os.getpid()
    # --no-undefined: a kernel whose host stub failed to instantiate must fail the build
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
