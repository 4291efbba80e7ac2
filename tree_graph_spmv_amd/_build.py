"""Build the HIP library libk2spmv.so in-tree (hipcc, gfx950 only)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libk2spmv.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
DEVICE_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-pthread", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]

SOURCES = [("k2_device.hip", DEVICE_FLAGS), ("k2_probe.hip", DEVICE_FLAGS), ("k2_build.cpp", HOST_FLAGS),
           ("k2_plan.cpp", HOST_FLAGS), ("k2_api.cpp", HOST_FLAGS)]


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src, flags in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [HIPCC, "-x", "c++"] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd, stderr=subprocess.STDOUT if not verbose else None)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-pthread"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
