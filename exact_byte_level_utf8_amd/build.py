"""Build the HIP tokenizer library (libtok.so, gfx950) and the CPU rules harness.

    python -m exact_byte_level_utf8_amd.build

The library is compiled in-tree with hipcc for gfx950.  Packed FP32
instructions are disabled for all device code (the tokenizer has no floating
point on its path; the flag keeps the compiler from emitting them anywhere).
librules_cpu.so is a g++ build of the per-code-point rule functions used only
by the tests.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtok.so")
RULES_LIB = os.path.join(HERE, "librules_cpu.so")
SOURCES = ["capi.hip", "repair.hip", "k_pretok.hip", "k_pretok_case.hip", "k_bpe.hip", "k_assemble.hip",
           "k_added.hip", "k_repair.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def hipcc_cmd(out: str) -> list[str]:
    return [
        HIPCC, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wl,--no-undefined",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build_lib() -> str:
    tmp = LIB + ".tmp"
    subprocess.check_call(hipcc_cmd(tmp))
    os.replace(tmp, LIB)
    return LIB


def build_rules() -> str:
    tmp = RULES_LIB + ".tmp"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-I", CSRC, "-o", tmp,
                           os.path.join(CSRC, "rules_cpu.cpp")])
    os.replace(tmp, RULES_LIB)
    return RULES_LIB


def main() -> None:
    build_rules()
    build_lib()
    print("built", LIB, RULES_LIB)


if __name__ == "__main__":
    sys.exit(main())
