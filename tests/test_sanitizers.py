"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

host_model.cpp (byte accounting, step-time model, fits, error bounds, subtree
selection) and the C oracle are each built with -fsanitize=address,undefined (no
recovery) together with a driver that calls every entry point on seeded random and
edge-case inputs (tests/c/san_host_model.c, tests/c/san_oracle.c); a report of an
invalid access, a leak or undefined behaviour fails the run.  The two builds are
separate: the oracle and the library share no code.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmds, exe):
    for c in cmds:
        r = subprocess.run(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, " ".join(c) + "\n" + r.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=ENV, timeout=600)
    assert r.returncode == 0 and "ERROR" not in r.stdout and "runtime error" not in r.stdout, r.stdout[-4000:]
    last = r.stdout.strip().splitlines()[-1]
    assert last.startswith("ok ") and int(last.split()[1]) > 100, r.stdout[-2000:]


def test_host_model_under_asan_ubsan(tmp_path):
    inc = os.path.join(ROOT, "include")
    obj = str(tmp_path / "host_model.o")
    drv = str(tmp_path / "san_host_model.o")
    exe = str(tmp_path / "san_host_model")
    _run([["g++", "-std=c++17", *SAN, "-I", inc, "-c", os.path.join(ROOT, "expert_ffn_amd", "csrc", "host_model.cpp"),
           "-o", obj],
          ["gcc", "-std=c99", *SAN, "-I", inc, "-c", os.path.join(ROOT, "tests", "c", "san_host_model.c"), "-o", drv],
          ["g++", *SAN, drv, obj, "-o", exe, "-lm"]], exe)


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "san_oracle")
    _run([["gcc", "-std=c99", *SAN, os.path.join(ROOT, "oracle", "moe_oracle.c"),
           os.path.join(ROOT, "tests", "c", "san_oracle.c"), "-o", exe, "-lm"]], exe)
