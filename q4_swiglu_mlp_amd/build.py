"""Build the HIP library ``_lib/libzinc_mlp.so`` for gfx950 with hipcc.

Every source under ``csrc/`` is compiled in one hipcc invocation into a shared
library that exports the C ABI of ``include/zinc_mlp.h``.  The per-kernel
register/LDS/occupancy report (``-Rpass-analysis=kernel-resource-usage``) is
kept in ``_lib/resource_usage.txt``.  Runs on a machine without a GPU.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_DIR = os.path.join(HERE, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libzinc_mlp.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # hardware float atomics for the fp32 split reductions
    "-munsafe-fp-atomics",
    # no packed-fp32 VALU instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",
]


def sources() -> list[str]:
    csrc = os.path.join(HERE, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip"))) + sorted(glob.glob(os.path.join(csrc, "*.cpp")))


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *sources(), "-o", tmp]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    report = [ln for ln in proc.stdout.splitlines() if "remark:" in ln]
    other = [ln for ln in proc.stdout.splitlines()
             if (" error:" in ln or " warning:" in ln) and "packed-fp32-ops" not in ln]
    with open(os.path.join(LIB_DIR, "resource_usage.txt"), "w") as f:
        f.write("\n".join(report) + "\n")
    if proc.returncode != 0:
        sys.stderr.write("\n".join(other) + "\n")
        raise RuntimeError(f"hipcc failed with exit code {proc.returncode}")
    if verbose and other:
        sys.stderr.write("\n".join(other) + "\n")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
