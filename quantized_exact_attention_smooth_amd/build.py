"""Build the gfx950 HIP library libsage_attn.so in-tree with hipcc.

Usage: python -m quantized_exact_attention_smooth_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsage_attn.so")
SOURCES = ["prep.hip", "attn_fwd.hip", "attn_split.hip", "sage_api.hip"]

# -packed-fp32-ops off: no packed fp32 VALU instructions are generated.
# -amdgpu-mfma-vgpr-form: matrix-core results land in VGPRs, which the
# softmax and RO update read directly (no AGPR-to-VGPR copies).
# -disable-machine-sink: machine sinking moves values down to their first use
# past the main loop's mask branches and so keeps more of them live at once;
# with it the main loop no longer fits its register budget (168 VGPRs for
# three waves per SIMD at D = 128) and spills.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-disable-machine-sink",
               "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library (always rebuilds)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-shared", "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
