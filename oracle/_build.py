"""Build the oracle's shared libraries with gcc: liboracle.so (plain C, one
thread), which the tests load, and liboracle_omp.so, the same source with
OpenMP, which serves only to time the oracle on all host cores."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
LIB_OMP = os.path.join(HERE, "liboracle_omp.so")
_FLAGS = ["-O2", "-ffp-contract=off", "-Wall", "-fPIC", "-shared", "-fvisibility=hidden"]


def _gcc(out, extra):
    cmd = ["gcc"] + _FLAGS + extra + ["-o", out + ".tmp", "oracle.c", "-lm"]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(out + ".tmp", out)


def build():
    _gcc(LIB, [])
    _gcc(LIB_OMP, ["-fopenmp"])


if __name__ == "__main__":
    build()
