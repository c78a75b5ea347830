"""Build the seeded input generator: libsynth_host.so (gcc) and libsynth_dev.so (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libsynth_host.so")
DEV_LIB = os.path.join(HERE, "libsynth_dev.so")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))


def build_host():
    _run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-Wall", "-o", HOST_LIB + ".tmp", "synth_host.c", "-lm"])
    os.replace(HOST_LIB + ".tmp", HOST_LIB)


def build_device():
    _run(["hipcc"] + HIP_FLAGS + ["-o", DEV_LIB + ".tmp", "synth_device.hip"])
    os.replace(DEV_LIB + ".tmp", DEV_LIB)


def build():
    build_host()
    build_device()


if __name__ == "__main__":
    build()
