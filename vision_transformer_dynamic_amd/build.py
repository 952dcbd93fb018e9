"""Build ``libbra.so`` (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: ``python -m vision_transformer_dynamic_amd.build`` (or call ``build()``).
Every call recompiles; the library is written next to this file and replaced
atomically so a process that has it loaded is never handed a half-written file.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libbra.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["pool.hip", "route.hip", "attend.hip", "attend_dense.hip", "lce.hip", "backward.hip", "backward_image.hip", "backward_top1.hip", "backward_dense.hip", "qkv.hip", "bra_api.hip"]
# achievable-peak probes of the benchmark: a library of their own
PEAK_LIB_NAME = "libbra_peak.so"
PEAK_LIB_PATH = os.path.join(PKG, PEAK_LIB_NAME)
PEAK_SOURCES = ["peak.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are switched off: the compiler's automatic v_pk_* fp32
# forms are avoided on this target.
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results go straight to VGPRs (no copies through AGPRs)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{proc.stdout}")
    return proc.stdout


def _check_resources(report: str, src: str):
    """Reject kernels that spill registers or use scratch: on this path every
    per-thread array must live in registers."""
    current = None
    for line in report.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            current = m.group(1)
            continue
        m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill): (\d+)", line)
        if m and int(m.group(2)) != 0:
            raise RuntimeError(f"{src}: kernel {current} has {m.group(1)} = {m.group(2)}")


def _link(objs, tmp, name, dest):
    tmp_lib = os.path.join(tmp, name)
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp_lib, *objs])
    staged = dest + ".tmp"
    shutil.copyfile(tmp_lib, staged)
    os.replace(staged, dest)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every HIP source and link the shared libraries (the operator's
    and the benchmark's peak probes); return the operator library's path."""
    tmp = tempfile.mkdtemp(prefix="bra_build_")
    try:
        srcs = SOURCES + PEAK_SOURCES
        objs = {}
        cmds = []
        for src in srcs:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            objs[src] = obj
            cmds.append([HIPCC, *CFLAGS, "-Rpass-analysis=kernel-resource-usage",
                         "-c", os.path.join(CSRC, src), "-o", obj])
        with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
            for src, out in zip(srcs, ex.map(_run, cmds)):
                _check_resources(out, src)
                if verbose:
                    for line in out.splitlines():
                        if "remark" in line and ("Name" in line or "VGPRs:" in line or "Occupancy" in line):
                            print(line.split("remark: ")[-1], file=sys.stderr)
        _link([objs[s_] for s_ in SOURCES], tmp, LIB_NAME, LIB_PATH)
        _link([objs[s_] for s_ in PEAK_SOURCES], tmp, PEAK_LIB_NAME, PEAK_LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
