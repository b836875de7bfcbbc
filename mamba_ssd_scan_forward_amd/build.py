"""Build ``libssd.so`` (the HIP kernels and the C ABI of ``include/ssd.h``) and
``libssd_probe.so`` (the machine measurements of ``include/ssd_probe.h``) for gfx950.

hipcc cross-compiles without a GPU, so this runs on any host with ROCm installed.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "ssd_api.hip")
LIB = os.path.join(HERE, "libssd.so")
PROBE_SRC = os.path.join(HERE, "csrc", "ssd_probe.hip")
PROBE_LIB = os.path.join(HERE, "libssd_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms are kept out of every device code path
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
]


def build(verbose: bool = False) -> str:
    compile_one(PROBE_SRC, PROBE_LIB, verbose)
    return compile_one(SRC, LIB, verbose)


def compile_one(src: str, lib: str, verbose: bool = False) -> str:
    tmp = lib + ".tmp"
    cmd = [HIPCC] + FLAGS + [src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in ln and "-target-feature" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)
    return lib


HOST_CHECK_SRC = os.path.join(HERE, "csrc", "host_check.cpp")
HOST_CHECK = os.path.join(HERE, "_build", "host_check")
# host code under AddressSanitizer and UndefinedBehaviorSanitizer (each -fsanitize= for the
# host pass only: the device code is built as usual and never run by the check)
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def build_host_check(verbose: bool = False) -> str:
    """The host-code check: ssd_api.hip and host_check.cpp linked into one program."""
    os.makedirs(os.path.dirname(HOST_CHECK), exist_ok=True)
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC", "-O3")]
    tmp = HOST_CHECK + ".tmp"
    cmd = [HIPCC] + flags + SANITIZE + [SRC, HOST_CHECK_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    os.replace(tmp, HOST_CHECK)
    return HOST_CHECK


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
