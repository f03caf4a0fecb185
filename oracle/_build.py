"""Build the oracle's shared library with gcc (plain C, single-threaded)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build():
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-Wall", "-fPIC", "-shared", "-fvisibility=hidden", "-o", LIB + ".tmp", "oracle.c", "-lm"]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(LIB + ".tmp", LIB)


if __name__ == "__main__":
    build()
