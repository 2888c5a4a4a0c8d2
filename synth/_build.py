"""Builds the synthetic-input libraries in place (host: gcc, device: hipcc gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libsynth.so")
DEV_LIB = os.path.join(HERE, "libsynth_dev.so")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))


def build_host():
    _run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
          "synth.c", "-o", HOST_LIB, "-lm"])


def build_device():
    _run(["/opt/rocm/bin/hipcc", *HIP_FLAGS, "synth_dev.hip", "-o", DEV_LIB])


def build():
    build_host()
    build_device()


if __name__ == "__main__":
    build()
