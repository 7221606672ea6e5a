"""Build libkda.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_prefill.hip", "kda_epilogue.hip",
           "kda_shortconv.hip", "kda_backward.hip", "kda_general.hip", "kda_noalloc.hip",
           "kda_copy.hip"]
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")


def hipcc_command(out: str) -> list:
    return (["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17",
             "-fPIC", "-shared", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             # packed fp32 VALU forms are kept out of generated code
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # MFMA accumulators in ordinary VGPRs: the state and the tiles that
             # VALU code rescales every chunk would otherwise be copied between
             # the accumulation registers and the VGPRs on each use
             "-mllvm", "-amdgpu-mfma-vgpr-form=true",
             "-Wno-unused-result", "-o", out]
            + [os.path.join(CSRC, s) for s in SOURCES])


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
