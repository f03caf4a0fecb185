"""Build the seeded input generator: a host library (gcc, OpenMP) and a device
library (hipcc for gfx950).  Both compile gen_core.h, the one definition of
every generated value."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libsynth_host.so")
DEV_LIB = os.path.join(HERE, "libsynth_dev.so")

HIPCC = "/opt/rocm/bin/hipcc"
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC"]
# packed fp32 arithmetic off, for the device pass only (the host compiler does
# not know the feature)
DEVICE_FEATURES = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))


def build_host():
    _run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fvisibility=hidden", "-o", HOST_LIB + ".tmp",
          "gen_host.c"])
    os.replace(HOST_LIB + ".tmp", HOST_LIB)


def build_device():
    obj = os.path.join(HERE, "_build")
    os.makedirs(obj, exist_ok=True)
    fb, o = os.path.join(obj, "gen_device.fb"), os.path.join(obj, "gen_device.o")
    _run([HIPCC, *COMMON, "--cuda-device-only", *DEVICE_FEATURES, "-c", "gen_device.hip", "-o", fb])
    _run([HIPCC, *COMMON, "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fb,
          "-c", "gen_device.hip", "-o", o])
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", DEV_LIB + ".tmp", o])
    os.replace(DEV_LIB + ".tmp", DEV_LIB)


def build():
    build_host()
    build_device()


if __name__ == "__main__":
    build()
