"""Build libgptoss_attn.so (the HIP kernels + C ABI) in-tree for gfx950.

Usage: python -m attention_attn_fwd_amd.build   (or __graft_entry__.build()).
The library is written next to this file; loaders never build on their own.
"""

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libgptoss_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["api.cpp", "plan.cpp", "fwd.hip", "decode.hip", "bwd.hip", "rope.hip"]

# Packed-fp32 VALU forms are kept out of generated code; hipcc's host pass
# warns that it does not know the feature, which is harmless.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
]


def hipcc_path():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose=False):
    """Compile every source into LIB_PATH (always recompiles)."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc_path(), *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.unlink(tmp)
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
