"""Builds the native libraries in-tree.

libsttd.so        the HIP kernels + C ABI (hipcc, gfx950 only)
libsttd_synth.so  the host-only seeded input generator (gcc, OpenMP)
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-munsafe-fp-atomics",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build failed: " + " ".join(cmd))
    return out


def build_synth():
    out = os.path.join(HERE, "libsttd_synth.so")
    _run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", os.path.join(CSRC, "synth.c"), "-o", out + ".tmp", "-lm"])
    os.replace(out + ".tmp", out)
    return out


def build_hip():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        return None
    out = os.path.join(HERE, "libsttd.so")
    objs = [os.path.join(CSRC, "_obj_" + os.path.basename(s) + ".o") for s in srcs]
    cmds = [[HIPCC] + [f for f in HIP_FLAGS if f != "-shared"] + ["-I", os.path.join(ROOT, "include"), "-c", s, "-o", o]
            for s, o in zip(srcs, objs)]
    # one compiler per source file, at most `jobs` at a time
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as pool:
        list(pool.map(_run, cmds))
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", out + ".tmp"])
    os.replace(out + ".tmp", out)
    for o in objs:
        os.remove(o)
    return out


def build_all():
    build_synth()
    build_hip()


if __name__ == "__main__":
    build_all()
