"""Build libtern.so (the C-ABI HIP library) in-tree with hipcc for gfx950.

Usage: python -m ternary_weight_linear_tern_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtern.so")
SOURCES = ["tern_kernels.hip", "tern_panel.hip", "tern_group.hip", "tern_optim.hip", "tern_noalloc.hip", "tern_api.cpp",
           "tern_layer.cpp", "tern_plan.cpp"]
ARCH = "gfx950"

# Packed FP32 VALU forms are turned off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def build(out: str = LIB, verbose: bool = False, save_temps_dir: str | None = None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-I", os.path.join(ROOT, "include"), *DEVICE_FLAGS, *srcs, "-o", out + ".tmp"]
    if save_temps_dir:
        cmd[1:1] = ["-save-temps=obj"]
    env = dict(os.environ)
    r = subprocess.run(cmd, capture_output=True, text=True, env=env,
                       cwd=save_temps_dir or None)
    # hipcc's host pass does not know the device-only feature flag; drop that note
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}")
    if verbose and err.strip():
        sys.stderr.write(err + "\n")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
