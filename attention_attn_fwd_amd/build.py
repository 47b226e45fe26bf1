"""Build libgptoss_attn.so (the HIP kernels + C ABI) in-tree for gfx950.

Usage: python -m attention_attn_fwd_amd.build   (or __graft_entry__.build()).
The library is written next to this file; loaders never build on their own.
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libgptoss_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["api.cpp", "plan.cpp", "fwd.hip", "decode.hip", "decode_paged.hip", "bwd.hip", "rope.hip"]

# Packed-fp32 VALU forms are kept out of generated code; hipcc's host pass
# warns that it does not know the feature, which is harmless.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
]

# Per-source additions: LLVM machine-scheduler strategies chosen by
# interleaved timing of builds that differ only in the flag (results
# bit-identical).  The forward with the iterative ILP scheduler: full-causal
# forward about 3% faster (589-592 against 606-619 us at B=4 S=4096).  The
# packed-cache decode with the max-ILP scheduler: the 128-sequence full layer
# 25.5-25.8 against 26.4-26.7 us, the sliding layer unchanged; the
# paged-cache decode kernels (decode_paged.hip) ran 2.3% slower with it and
# keep the default, as do the backward kernels (2-6% slower with either).
SOURCE_FLAGS = {"fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
                "decode.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def hipcc_path():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose=False):
    """Compile every source (in parallel, each into its own object) and link
    them into LIB_PATH (always recompiles)."""
    hipcc = hipcc_path()
    tmpdir = tempfile.mkdtemp(prefix="gptoss_build_")
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    try:
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            cmd = [hipcc, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), "-I", os.path.join(ROOT, "include"),
                   "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                                     text=True)))
        objs, errors, noise = [], [], []
        for src, obj, proc in procs:
            out, err = proc.communicate()
            if proc.returncode != 0:
                errors.append(f"{src}:\n{out}{err}")
            noise += [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln]
            objs.append(obj)
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + res.stdout + res.stderr)
        if verbose and noise:
            print("\n".join(noise), file=sys.stderr)
        os.replace(tmp, LIB_PATH)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
