"""Builds libprism.so (the HIP kernels and the C ABI of include/prism.h) for gfx950.

    python -m dynamic_block_sparse_stats_amd.build

Each .hip source is compiled with hipcc into an object, in parallel, then linked into
dynamic_block_sparse_stats_amd/libprism.so next to this file.  The build always runs (no
timestamp shortcut): callers decide when to rebuild.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libprism.so")
SOURCES = ["plan_kernels.hip", "select_kernels.hip", "attn_fwd.hip", "attn_bwd.hip",
           "attn_bwd_dkdv.hip", "a2v_norm.hip", "prism_api.hip"]
# The attention kernels never see NaN inputs; without IEEE-mode NaN quieting the compiler
# can feed MFMA results straight into v_max instead of canonicalising each one first.
# The forward and dQ kernels also keep their MFMA accumulators in ordinary VGPRs (no
# accvgpr copies around the softmax); dK/dV, with more live accumulators, does not.
_NAN = ["-fno-honor-nans", "-mno-amdgpu-ieee"]
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {"attn_fwd.hip": _NAN + _VGPR_MFMA, "attn_bwd.hip": _NAN + _VGPR_MFMA,
         "attn_bwd_dkdv.hip": _NAN}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libprism.so)")


def compile_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
            "-Wno-unused-variable", "-Wno-unused-function",
            # no packed-FP32 instructions anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(HERE, "..", "include")]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="prism_build_")
    try:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *compile_flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
                   "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            # the host pass does not know the packed-fp32 feature; that note is harmless
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if lines and (verbose or p.returncode):
                print(f"--- {src}\n" + "\n".join(lines), file=sys.stderr)
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        link = [cc, "-shared", f"--offload-arch={ARCH}", "-o", LIB + ".tmp", *objs]
        subprocess.check_call(link)
        os.replace(LIB + ".tmp", LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
