"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so.

The flags keep every binary32 operation a single IEEE operation: no contraction
into fused multiply-add, no fast-math reassociation, no flush-to-zero.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["onebit_oracle.c"]
TARGET = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", TARGET + ".tmp", *[os.path.join(HERE, s) for s in SOURCES], "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(TARGET + ".tmp", TARGET)
    return TARGET


def build_from_text(source_text: str, out_path: str) -> str:
    """Compile a (possibly modified) copy of the oracle source with the same flags."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    flags = [f for f in CFLAGS if f != "-Werror"]  # a planted mistake may leave a variable unused
    subprocess.run(["gcc", *flags, "-o", out_path, src, "-lm"], check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
