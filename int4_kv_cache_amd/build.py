"""Build libsawkv.so (gfx950) in-tree with hipcc.

    python -m int4_kv_cache_amd.build

Compiles int4_kv_cache_amd/csrc/sawkv.hip (write path and read-back),
sawkv_attn.hip (decode attention) and sawkv_controls.hip (uncompressed cache
write, token-wise INT8) into int4_kv_cache_amd/libsawkv.so.
Flags: -ffp-contract=off (every float32 operation rounds on its own, as the
bit-exact definition needs), no fast-math, denormals kept (the HIP default),
packed-fp32 instructions disabled, MFMA accumulators in VGPRs.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f)
        for f in ("sawkv.hip", "sawkv_attn.hip", "sawkv_controls.hip")]
OUT = os.path.join(PKG, "libsawkv.so")
ARCH = "gfx950"


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsawkv.so)")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep matrix-core accumulators in VGPRs (the attention loop rescales
        # them with VALU ops; AGPR accumulators would be copied every step)
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I", os.path.join(ROOT, "include"),
        "-I", os.path.join(PKG, "csrc"),
    ]


def build(verbose=False):
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + flags() + SRCS + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines()
            if "is not a recognized feature for this target" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
