"""Build libcbd.so (HIP kernels for gfx950 + the host runtime) in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcbd.so")
ROOT = os.path.dirname(HERE)

SOURCES = ["runtime.cpp", "gemm_skinny.hip", "attention.hip", "elementwise.hip"]

# Packed fp32 VALU ops are disabled for every device pass; the host pass
# reports the feature as unknown, which is harmless.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def defines() -> list:
    """Build options from the environment: CBD_DEFINES="NAME=VALUE ..." adds -DNAME=VALUE per item
    (e.g. CBD_VALU_ROWS=4 CBD_VALU_DEPTH=2 for the vector-ALU small-batch products)."""
    return ["-D" + d for d in os.environ.get("CBD_DEFINES", "").split() if d]


def build(verbose: bool = False) -> str:
    """Compile every source into libcbd.so (always rebuilds). Returns the library path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ([hipcc()] + HIPCC_FLAGS + defines() + ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + srcs +
           ["-o", tmp])
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + msgs)
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
