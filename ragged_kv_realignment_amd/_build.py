"""Build libspecdec.so (the C-ABI library and its HIP kernels) for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libspecdec.so")
SOURCES = ["csrc/api.cpp", "csrc/verify.hip", "csrc/realign.hip", "csrc/realign_inplace.hip", "csrc/sample_logits.hip", "csrc/group.hip",
           "csrc/paged.hip", "csrc/pool.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
         "-I" + os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(extra_flags=(), out=LIB):
    cmd = ["/opt/rocm/bin/hipcc", *FLAGS, *extra_flags, "-o", out + ".tmp", *SOURCES]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libspecdec build failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(out + ".tmp", out)
    return r.stderr


if __name__ == "__main__":
    err = build()
    if err.strip():
        print(err)
