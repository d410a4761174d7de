"""Builds the C++ client of the C ABI (hs_client), linked against the in-tree libhisparse.so."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "hs_client.cpp")
BIN = os.path.join(HERE, "hs_client")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    tmp = BIN + ".tmp"
    cmd = [HIPCC, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp,
           "-L", os.path.join(ROOT, "hierarchical_memory_amd"), "-lhisparse",
           "-Wl,-rpath,$ORIGIN/../../hierarchical_memory_amd"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build the C ABI client")
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
