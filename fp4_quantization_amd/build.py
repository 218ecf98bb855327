"""Build libufp4.so (all HIP sources, gfx950 only) in the package directory."""
from __future__ import annotations

import os
import shutil
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(_HERE, "csrc", f)
           for f in ("ufp4_quant.hip", "ufp4_misc.hip", "ufp4_gemm.hip", "ufp4_host.hip", "ufp4_api.hip")]
OUT = os.path.join(_HERE, "libufp4.so")

# -ffp-contract=off: no implicit fused multiply-add (every rounding step is
# the one written).  The packed-fp32 feature is disabled: the kernels never
# use packed binary32 instructions.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall"]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def build(verbose: bool = False) -> str:
    cmd = [hipcc()] + HIPCC_FLAGS + ["-o", OUT + ".tmp"] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
