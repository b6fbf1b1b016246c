"""Build libmoe_expert.so in-tree with hipcc for gfx950.

    python -m expert_ffn_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SO = os.path.join(HERE, "libmoe_expert.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are kept out of the generated code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-I" + INCLUDE, "-Wall", "-Wno-unused-function"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("command failed: " + " ".join(cmd))
    if out.strip():
        sys.stderr.write(out + "\n")


def _variant_objects():
    """(source, object, defines) of the fused kernel's variant groups."""
    src = os.path.join(CSRC, "expert_launch.hip")
    out = []
    for b in (0, 1):
        for m in (0, 1):
            for s in (0, 1):
                out.append((src, os.path.join(BUILD, "expert_launch_%d%d%d.o" % (b, m, s)),
                            ["-DMOE_K_BF16=%d" % b, "-DMOE_K_MODE=%d" % m, "-DMOE_K_SH=%d" % s]))
    return out


def build(verbose=False, jobs=None):
    """Compile every translation unit (in parallel, `jobs` at a time; default: the
    CPU count, at most 8) and link the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    hip = [(os.path.join(CSRC, "moe_expert.hip"), os.path.join(BUILD, "moe_expert.o"), [])] + _variant_objects()
    cmds = [[HIPCC, "--offload-arch=" + ARCH, *COMMON, *DEVICE_FLAGS, *defs, "-c", src, "-o", obj]
            for src, obj, defs in hip]
    o2 = os.path.join(BUILD, "host_model.o")
    cmds.append([HIPCC, *COMMON, "-x", "c++", "-c", os.path.join(CSRC, "host_model.cpp"), "-o", o2])
    jobs = jobs or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        for f in [pool.submit(_run, c) for c in cmds]:
            f.result()
    objs = [obj for _, obj, _ in hip] + [o2]
    tmp = SO + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build())
