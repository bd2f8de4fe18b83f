"""Build the HIP library ``_lib/libzinc_mlp.so`` for gfx950 with hipcc.

Every source under ``csrc/`` is compiled by its own hipcc process (in
parallel), and the objects are linked into a shared library that exports the
C ABI of ``include/zinc_mlp.h``.  The per-kernel register/LDS/occupancy report
(``-Rpass-analysis=kernel-resource-usage``) is written to
``_lib/resource_usage.txt`` (a build log, not tracked).  Runs on a machine
without a GPU.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_DIR = os.path.join(HERE, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libzinc_mlp.so")
# the benchmark's measured-peak kernels (MFMA loop, HBM stream read and copy):
# a library of their own, not part of the MLP library
PEAKS_SRC = os.path.join(HERE, "peaks", "peaks.hip")
PEAKS_PATH = os.path.join(LIB_DIR, "libzinc_peaks.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # hardware float atomics for the fp32 split reductions
    "-munsafe-fp-atomics",
    # no packed-fp32 VALU instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",
]


def sources() -> list[str]:
    csrc = os.path.join(HERE, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip"))) + sorted(glob.glob(os.path.join(csrc, "*.cpp")))


def _jobs() -> int:
    try:
        n = int(os.environ.get("MAX_JOBS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n or (os.cpu_count() or 1), 16))


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    obj_dir = os.path.join(LIB_DIR, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *HIPCC_FLAGS, "-c", *lang, src, "-o", obj]
        proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        return src, obj, proc

    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        peaks = ex.submit(subprocess.run, [hipcc, *HIPCC_FLAGS[:-1], "-shared", "-x", "hip", PEAKS_SRC, "-o",
                                           PEAKS_PATH + ".tmp"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                          text=True)
        results = list(ex.map(compile_one, srcs))
        peaks = peaks.result()
    if peaks.returncode != 0:
        sys.stderr.write(peaks.stdout + "\n")
        raise RuntimeError("hipcc failed on peaks.hip")
    os.replace(PEAKS_PATH + ".tmp", PEAKS_PATH)
    report, other, failed = [], [], []
    for src, _obj, proc in results:
        lines = proc.stdout.splitlines()
        report += [ln for ln in lines if "remark:" in ln]
        other += [ln for ln in lines if (" error:" in ln or " warning:" in ln) and "packed-fp32-ops" not in ln]
        if proc.returncode != 0:
            failed.append(os.path.basename(src))
    with open(os.path.join(LIB_DIR, "resource_usage.txt"), "w") as f:
        f.write("\n".join(report) + "\n")
    if failed:
        sys.stderr.write("\n".join(other) + "\n")
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    if verbose and other:
        sys.stderr.write("\n".join(other) + "\n")
    tmp = LIB_PATH + ".tmp"
    link = subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o, _ in results],
                           "-o", tmp], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if link.returncode != 0:
        sys.stderr.write(link.stdout + "\n")
        raise RuntimeError(f"link failed with exit code {link.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
