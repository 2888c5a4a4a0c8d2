"""Builds libmoe.so in place: every HIP source for gfx950, one shared library."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["api.hip", "route.hip", "gemv.hip", "grouped.hip", "misc.hip", "accept.hip", "noalloc.hip"]

HIPCC = "/opt/rocm/bin/hipcc"
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fno-gpu-rdc", "-ffp-contract=fast", "-Wall", "-Wno-unused-function",
    # keep packed fp32 instructions out of the code objects
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the grouped GEMMs rescale every int32 block
    # result on the VALU, which cannot read accumulation registers directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _run(cmd):
    r = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return r.stderr


def build(jobs=8):
    os.makedirs(os.path.join(HERE, "_obj"), exist_ok=True)
    objs = [os.path.join(HERE, "_obj", s.replace(".hip", ".o")) for s in SOURCES]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _run([HIPCC, *FLAGS, "-c", so[0], "-o", so[1]]), zip(SOURCES, objs)))
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB])
    return LIB


if __name__ == "__main__":
    print(build())
