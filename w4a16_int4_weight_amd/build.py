"""Builds the HIP library libw4a16.so in-tree for gfx950 with hipcc.

Usage: python -m w4a16_int4_weight_amd.build   (or build() from Python).
"""

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libw4a16.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["api.hip", "repack.hip", "gemv.hip", "gemv_strip.hip", "gemv_small.hip", "gemm.hip", "embedding.hip", "w4a8.hip", "measure.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    # keep hipcc from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the W4A16 library needs ROCm's hipcc to build")


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the host code only (the
# C ABI's validation, plans and launchers); the device code is built as usual. The
# library then needs the ASan runtime preloaded into the process that loads it.
SANITIZE_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime():
    """Path of the ASan runtime a host-sanitized library needs preloaded."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the ASan runtime of the ROCm compiler was not found")
    return path


def build(verbose=False, out=None, sanitize_host=False):
    """Compiles every source into LIB_PATH, or `out` (always recompiles). Returns the path.
    sanitize_host: host code built with ASan and UBSan (see SANITIZE_HOST_FLAGS)."""
    target = out or LIB_PATH
    tmp = target + ".tmp"
    flags = HIPCC_FLAGS + (SANITIZE_HOST_FLAGS if sanitize_host else [])
    cmd = [hipcc()] + flags + ["-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so: harmless
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
