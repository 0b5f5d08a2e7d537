"""Build libtm.so (HIP for gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled for the device (they are never written by hand either).  Objects go
to ``_build/`` at the repository root; the shared library is placed next to
this file so it travels with the package.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtm.so")
CEILING = os.path.join(HERE, "tm_ceiling")   # hardware-ceiling microbenchmarks (bench.py --ceiling)
SOURCES = ["tm_api.hip", "k_quant.hip", "k_trav.hip", "k_prefill.hip", "k_prefill_pipe.hip", "k_decode.hip",
           "k_select.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libtm")


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in ordinary VGPRs: the kernels rescale them
            # with VALU ops, which would otherwise copy them out of AGPRs
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False, jobs: int = 4) -> str:
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()

    def one(src):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [cc] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs, file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = OUT + ".tmp"
    r = subprocess.run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    # the ceiling microbenchmarks: a separate executable, not part of libtm
    tmp = CEILING + ".tmp"
    r = subprocess.run([cc] + flags() + [os.path.join(CSRC, "ceiling.hip"), "-o", tmp], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on ceiling.hip:\n" + r.stdout + r.stderr)
    os.replace(tmp, CEILING)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
