"""Build the float64 CPU oracle library (``oracle/libssd_oracle.so``) with gcc.

Test infrastructure: the product library never links this.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssd_oracle.c")
LIB = os.path.join(HERE, "libssd_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


CHECK_SRC = os.path.join(HERE, "sanitize_check.c")
CHECK = os.path.join(HERE, "_build", "sanitize_check")


def build_sanitize_check(verbose: bool = False) -> str:
    """The oracle under AddressSanitizer and UndefinedBehaviorSanitizer, driven by
    sanitize_check.c."""
    os.makedirs(os.path.dirname(CHECK), exist_ok=True)
    cmd = ["gcc", "-O1", "-g", "-fopenmp", "-std=c11", "-Wall", "-Wextra", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", SRC, CHECK_SRC, "-o", CHECK + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(CHECK + ".tmp", CHECK)
    return CHECK


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
