"""Build libmla_paged.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m mla_decode_attention_paged_amd.build

Compiles csrc/mla_decode.hip (FP8 decode kernels with their split merge,
csrc/split_merge.h, + launchers), csrc/mla_decode_rf.hip (the FP8 decode with
both contractions on the block-scaled FP8 MFMA),
csrc/mla_decode_bf16.hip (unquantized-cache decode kernel), csrc/kv_append.hip
(append-and-quantise kernel), csrc/noalloc.hip (the decode entry point with a
device-resident split scratch) and csrc/api.cpp (C ABI) into
mla_decode_attention_paged_amd/libmla_paged.so.  Packed-FP32 VALU
instructions are disabled for the device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libmla_paged.so")
ARCH = "gfx950"


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def device_flags(vgpr_mfma: bool = True) -> list[str]:
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
    if vgpr_mfma:
        # MFMA accumulators in ordinary VGPRs: the online softmax rescales
        # them with VALU ops, and AGPR accumulators would be copied to VGPRs
        # and back on every loop iteration.  (The one-wave-per-SIMD kernel of
        # mla_decode_rf.hip needs the AGPRs for its accumulators.)
        flags += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    return flags


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    hipcc = hipcc_path()
    with tempfile.TemporaryDirectory(prefix="mla_build_") as tmp:
        objs = []
        for src, lang in (("mla_decode.hip", "hip"), ("mla_decode_rf.hip", "hip"), ("mla_decode_bf16.hip", "hip"),
                          ("kv_append.hip", "hip"), ("noalloc.hip", "hip"), ("api.cpp", "c++")):
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc, *device_flags(src != "mla_decode_rf.hip"), "-x", lang, "-c", os.path.join(CSRC, src),
                   "-o", obj]
            if lang == "c++":
                # host-only source (HIP runtime calls, no kernels): hipcc still
                # treats it as HIP, so name the one target to skip its default
                cmd = [hipcc, f"--offload-arch={ARCH}", "-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
                       "-c", os.path.join(CSRC, src), "-o", obj]
            _run(cmd, verbose)
            objs.append(obj)
        tmp_out = os.path.join(tmp, "libmla_paged.so")
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_out], verbose)
        shutil.copyfile(tmp_out, OUT + ".tmp")
        os.replace(OUT + ".tmp", OUT)
    return OUT


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}")
    noise = ("is not a recognized feature", "packed-fp32-ops")
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if ln and not any(n in ln for n in noise)]
    if verbose and msgs:
        print("\n".join(msgs))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
