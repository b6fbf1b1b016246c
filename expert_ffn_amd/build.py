"""Build libmoe_expert.so in-tree with hipcc for gfx950.

    python -m expert_ffn_amd.build
"""
import os
import subprocess
import sys

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


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    hip_src = os.path.join(CSRC, "moe_expert.hip")
    o1 = os.path.join(BUILD, "moe_expert.o")
    _run([HIPCC, "--offload-arch=" + ARCH, *COMMON, *DEVICE_FLAGS, "-c", hip_src, "-o", o1])
    objs.append(o1)
    o2 = os.path.join(BUILD, "host_model.o")
    _run([HIPCC, *COMMON, "-x", "c++", "-c", os.path.join(CSRC, "host_model.cpp"), "-o", o2])
    objs.append(o2)
    tmp = SO + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build())
