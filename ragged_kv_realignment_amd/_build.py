"""Build libspecdec.so (the C-ABI library and its HIP kernels) for gfx950.

Each .hip source is compiled twice: a device-only pass for gfx950, which alone
gets the target-feature flags (packed fp32 arithmetic off), and a host-only pass
that embeds the device pass's offload bundle.  The host compiler therefore never
sees an AMDGPU feature it does not know.  The sources compile in parallel."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libspecdec.so")
# the benchmark's measurement kernels (bare reads with library kernels' launch shapes), not part of the C ABI
MEASURE_LIB = os.path.join(HERE, "libspecdec_measure.so")
MEASURE_SOURCES = ["csrc/measure.hip"]
OBJ = os.path.join(HERE, "_build")
HIP_SOURCES = ["csrc/verify.hip", "csrc/realign.hip", "csrc/realign_inplace.hip", "csrc/sample_logits.hip",
               "csrc/group.hip", "csrc/paged.hip", "csrc/pool.hip", "csrc/scratch.hip"]
CPP_SOURCES = ["csrc/api.cpp"]
HIPCC = "/opt/rocm/bin/hipcc"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-I" + os.path.join(ROOT, "include")]
DEVICE_ONLY = ["--offload-arch=gfx950", "--cuda-device-only",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libspecdec build failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return r.stderr


def _compile_hip(src, extra):
    stem = os.path.join(OBJ, os.path.basename(src))
    err = _run([HIPCC, *COMMON, *DEVICE_ONLY, *extra, "-c", src, "-o", stem + ".fb"])
    err += _run([HIPCC, *COMMON, "--offload-arch=gfx950", "--cuda-host-only", *extra,
                 "-Xclang", "-fcuda-include-gpubinary", "-Xclang", stem + ".fb", "-c", src, "-o", stem + ".o"])
    return stem + ".o", err


def _compile_cpp(src, extra):
    out = os.path.join(OBJ, os.path.basename(src) + ".o")
    return out, _run([HIPCC, *COMMON, *extra, "-c", src, "-o", out])


def build(extra_flags=(), out=LIB, measure=True):
    os.makedirs(OBJ, exist_ok=True)
    srcs = HIP_SOURCES + (MEASURE_SOURCES if measure else [])
    jobs = [(_compile_hip, s) for s in srcs] + [(_compile_cpp, s) for s in CPP_SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        done = list(ex.map(lambda j: j[0](j[1], list(extra_flags)), jobs))
    obj = {src: o for (_, src), (o, _) in zip(jobs, done)}
    err = "".join(e for _, e in done)
    links = [(out, [obj[s] for s in HIP_SOURCES + CPP_SOURCES])]
    if measure:
        links.append((MEASURE_LIB, [obj[s] for s in MEASURE_SOURCES]))
    for lib, objs in links:
        err += _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp", *objs])
        os.replace(lib + ".tmp", lib)
    return err


if __name__ == "__main__":
    err = build()
    if err.strip():
        print(err)
