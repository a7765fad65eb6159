"""Build the gfx950 HIP library in-tree (hipcc, no JIT cache)."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libmlasd.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["mlasd_decode.hip", "mlasd_combine.hip", "mlasd_append.hip", "mlasd_topk.hip", "mlasd_noalloc.hip", "mlasd_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU forms are disabled for every HIP translation unit.  The
# SDWA peephole is off too: a v_max_u16_sdwa reading the high word of its
# second operand returned the low word's maximum on gfx950 (a per-head q
# maximum lost its odd elements), so no sub-dword-select instruction is
# formed.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-sdwa-peephole=0",
         "-Wno-unused-command-line-argument"]


def build(verbose=False):
    """Compile libmlasd.so next to this file; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
