"""Compile abi_check.c (a plain C caller of libnbx_paged) into tests/c/abi_check.

Run by __graft_entry__.build() after the library is built; gcc only (the
program has no device code), linked against the in-tree libnbx_paged.so with
an rpath relative to the binary so that the tree can move.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_check.c")
BIN = os.path.join(HERE, "abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def flags(syntax_only: bool = False) -> list:
    f = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
         "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC]
    if syntax_only:
        return f + ["-fsyntax-only"]
    return f + ["-o", BIN, "-L", os.path.join(ROOT, "paged_split_kv_append_amd"), "-lnbx_paged",
                "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                "-Wl,-rpath,$ORIGIN/../../paged_split_kv_append_amd",
                "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"]


def build() -> str:
    r = subprocess.run(flags(), capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for {SRC}:\n{r.stdout}\n{r.stderr}")
    return BIN


if __name__ == "__main__":
    print("built", build())
